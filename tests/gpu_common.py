"""Helpers for the GPU parity tests: build a chunk's inputs on the GPU from the
seeded generators, run the oracle on the same values, and compare within the
stated tolerances.

Tolerances (the target's):
  * token log-prob: abs <= 1e-5 for fp32 logits, <= 2e-3 for bf16 logits;
  * loss: |dL| <= 1e-4 * max(|L|, sum|l_t| / N) (relative, guarded near 0);
  * dlogits: relative L2 <= 1e-3 against the oracle rounded once to the
    output dtype (bf16 storage alone is ~1.7e-3 off float64);
  * entropy (no stated bound): abs <= 1e-4 + 1e-5 * H, from fp32 sums over V;
  * plans, counts, flags: exact.
"""

import numpy as np
import torch

import oracle
from grpo_token_level_amd import ops

DEV = "cuda"


def tol_logp(dtype):
    return 1e-5 if dtype == torch.float32 else 2e-3


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(got, want):
    num = float(np.sqrt(np.sum((got - want) ** 2)))
    den = float(np.sqrt(np.sum(want ** 2)))
    return num / den if den > 0 else num


def make_chunk(n_tok, V, dtype=torch.float32, seed=0, n_rows=None, logit_std=2.0, noise=0.05,
               masked_frac=0.25, ld=None, with_old=True):
    """Random chunk on the GPU: logits [n_tok, V] (row stride ld), targets,
    mask, per-row advantages, rows of near-equal size, and old log-probs from
    the oracle's log-probs plus N(0, noise) (computed on the CPU)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    ld = ld or V
    base = torch.randn((n_tok, ld), generator=g, dtype=torch.float32) * logit_std
    logits_cpu = base.to(dtype)
    rng = np.random.default_rng(seed)
    target = rng.integers(0, V, n_tok).astype(np.int32)
    mask = (rng.random(n_tok) > masked_frac).astype(np.uint8)
    n_rows = n_rows or max(1, n_tok // 7)
    cuts = np.sort(rng.choice(np.arange(1, max(n_tok, 2)), size=min(n_rows - 1, max(n_tok - 1, 0)), replace=False)) \
        if n_rows > 1 and n_tok > 1 else np.array([], np.int64)
    row_off = np.concatenate([[0], cuts, [n_tok]]).astype(np.int64)
    n_rows = len(row_off) - 1
    adv_row = rng.normal(0, 1, n_rows).astype(np.float32)
    tok_row = np.zeros(n_tok, np.int32)
    for r in range(n_rows):
        tok_row[row_off[r]:row_off[r + 1]] = r
    z64 = logits_cpu[:, :V].double().numpy()
    if with_old:
        lp = oracle.logprob_fwd(z64, target, np.ones(n_tok, np.uint8))["logp"]
        old = (lp + rng.normal(0, noise, n_tok)).astype(np.float32)
    else:
        old = np.zeros(n_tok, np.float32)
    full = logits_cpu.to(DEV)
    d = dict(logits=full[:, :V], logits_full=full, z64=z64, target=target, mask=mask, old=old,
             row_off=row_off, adv_row=adv_row, tok_row=tok_row, V=V, dtype=dtype)
    d["g"] = {k: torch.from_numpy(np.ascontiguousarray(d[k])).to(DEV)
              for k in ("target", "mask", "old", "row_off", "adv_row", "tok_row")}
    return d


def run_oracle(d, scale, eps=(0.2, 0.2), idx=None):
    """Oracle outputs for the whole chunk (or the tokens ``idx``)."""
    sel = np.arange(d["z64"].shape[0]) if idx is None else np.asarray(idx)
    adv_tok = d["adv_row"].astype(np.float64)[d["tok_row"][sel]]
    return oracle.loss_fwd_bwd(d["z64"][sel], d["target"][sel], d["mask"][sel],
                               d["old"].astype(np.float64)[sel], adv_tok, scale, eps[0], eps[1])


def run_gpu(d, scale=1.0, denom=None, eps=(0.2, 0.2), dlogits="new", out_dtype=None):
    g = d["g"]
    return ops.loss_fwd_bwd(d["logits"], g["target"], g["mask"], g["old"], g["tok_row"], g["adv_row"],
                            g["row_off"], scale=scale, denom=denom, eps_low=eps[0], eps_high=eps[1],
                            dlogits=dlogits, out_dtype=out_dtype)


def assert_tokens_match(ws, ref, d, idx=None, check_dz=True, eps=(0.2, 0.2)):
    """Per-token outputs and dlogits vs the oracle (``idx``: token subset).

    The clip decision is a float comparison taken in float32 by the kernel
    and in float64 by the oracle; a token whose ratio lies within 1e-4
    (relative) of a clip edge may fall either way.  Such tokens, when the two
    sides disagree, are left out of the flag and dlogits comparisons (their
    loss is continuous across the edge and stays in); any other disagreement
    fails."""
    sel_np = np.arange(d["z64"].shape[0]) if idx is None else np.asarray(idx)
    sel = torch.as_tensor(sel_np, device=DEV)
    dtype = d["dtype"]
    valid = ref["valid"]
    logp = to_f64(ws["logp"][sel])
    ent = to_f64(ws["entropy"][sel])
    lt = to_f64(ws["loss_tok"][sel])
    flags = ws["tok_flags"][sel].cpu().numpy()
    assert np.array_equal((flags & 1).astype(bool), valid)
    assert np.array_equal(((flags >> 2) & 1).astype(bool), ref["nonfinite"])
    fin = valid & ~ref["nonfinite"]
    with np.errstate(over="ignore", invalid="ignore"):
        rho = np.exp(ref["logp"] - d["old"].astype(np.float64)[sel_np])
    hi, lo = 1.0 + eps[1], 1.0 - eps[0]
    edge = fin & ((np.abs(rho - hi) <= 1e-4 * hi) | (np.abs(rho - lo) <= 1e-4))
    gclip = ((flags >> 1) & 1).astype(bool)
    differ = gclip != (ref["clipped"] & valid)
    assert not np.any(differ & ~edge), np.nonzero(differ & ~edge)
    keep = ~differ
    assert np.all(np.abs(logp[fin] - ref["logp"][fin]) <= tol_logp(dtype)), np.max(np.abs(logp[fin] - ref["logp"][fin]))
    assert np.all(np.abs(ent[fin] - ref["entropy"][fin]) <= 1e-4 + 1e-5 * np.abs(ref["entropy"][fin]))
    assert np.all(logp[~valid] == 0) and np.all(lt[~valid] == 0) and np.all(ent[~valid] == 0)
    # loss (as a sum over the chunk): |dL| <= 1e-4 * max(|L|, sum |l_t|)
    L_ref = float(np.sum(ref["loss_tok"][fin]))
    bound = 1e-4 * max(abs(L_ref), float(np.sum(np.abs(ref["loss_tok"][fin]))))
    assert abs(float(np.sum(lt[fin])) - L_ref) <= max(bound, 1e-12)
    if check_dz and ws.get("dlogits") is not None:
        dz = to_f64(ws["dlogits"][sel])[keep]
        want = ref["dz"][keep]
        if ws["dlogits"].dtype == torch.bfloat16:
            want = oracle.round_to_bf16(want)
        assert rel_l2(dz, want) <= 1e-3, rel_l2(dz, want)
        assert not dz[~valid[keep]].any()
    return int(differ.sum())


def torch_logp(logits, target, block=512):
    """Current log-probs from a plain PyTorch fp32 log-softmax (used only to
    shape old log-probs as "current + small drift" for large inputs)."""
    out = torch.empty(logits.shape[0], dtype=torch.float32, device=logits.device)
    for a in range(0, logits.shape[0], block):
        b = min(a + block, logits.shape[0])
        lp = torch.log_softmax(logits[a:b].float(), dim=-1)
        out[a:b] = lp.gather(1, target[a:b].long()[:, None])[:, 0]
    return out


def padded_on_gpu(workload, seed=0, **over):
    """A padded workload resident on the GPU: logits drawn row by row from the
    seeded streams, old log-probs = torch log-probs + the workload's noise."""
    from synth import fill_normal_rows, padded_batch
    b = padded_batch(workload, seed=seed, **over)
    n_rows, T, V = b["n_rows"], b["T"], b["V"]
    dt = torch.bfloat16 if b["dtype"] == "bf16" else torch.float32
    logits = torch.empty((n_rows * T, V), dtype=dt, device=DEV)
    fill_normal_rows(logits, range(n_rows), [r * T for r in range(n_rows)], [T] * n_rows, b["logit_std"], seed, workload)
    G = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    target, mask = G(b["target"]), G(b["mask"])
    old = (torch_logp(logits, target).double() + G(b["logratio_noise"])).float()
    return b, logits, target, mask, old


def oracle_tokens(logits, target, mask, old, adv_tok, scale, idx, eps=(0.2, 0.2)):
    """Oracle outputs for the sampled token indices ``idx`` of a GPU batch."""
    ii = torch.as_tensor(np.asarray(idx), device=DEV)
    z = logits[ii].double().cpu().numpy()
    return oracle.loss_fwd_bwd(z, target[ii].cpu().numpy(), mask[ii].cpu().numpy(),
                               old[ii].double().cpu().numpy(), np.asarray(adv_tok, np.float64)[np.asarray(idx)],
                               scale, eps[0], eps[1])


def compare_sampled(out, ref, idx, old_np, dtype, dz_rows=None, eps=(0.2, 0.2)):
    """Per-token outputs (dicts of full-length GPU tensors) at ``idx`` vs the
    oracle dict ``ref``; ``dz_rows``: the kernel's dlogits rows at ``idx``."""
    ii = torch.as_tensor(np.asarray(idx), device=DEV)
    valid = ref["valid"]
    flags = out["tok_flags"][ii].cpu().numpy()
    assert np.array_equal((flags & 1).astype(bool), valid)
    fin = valid & ~ref["nonfinite"]
    logp = to_f64(out["logp"][ii])
    assert np.all(np.abs(logp[fin] - ref["logp"][fin]) <= tol_logp(dtype)), np.max(np.abs(logp[fin] - ref["logp"][fin]))
    ent = to_f64(out["entropy"][ii])
    assert np.all(np.abs(ent[fin] - ref["entropy"][fin]) <= 1e-4 + 1e-5 * np.abs(ref["entropy"][fin]))
    lt = to_f64(out["loss_tok"][ii])
    assert np.all(np.abs(lt[fin] - ref["loss_tok"][fin]) <= 1e-4 * np.maximum(np.abs(ref["loss_tok"][fin]), 1e-3))
    with np.errstate(over="ignore", invalid="ignore"):
        rho = np.exp(ref["logp"] - old_np)
    hi, lo = 1.0 + eps[1], 1.0 - eps[0]
    edge = fin & ((np.abs(rho - hi) <= 1e-4 * hi) | (np.abs(rho - lo) <= 1e-4))
    differ = ((flags >> 1) & 1).astype(bool) != (ref["clipped"] & valid)
    assert not np.any(differ & ~edge)
    if dz_rows is not None:
        keep = ~differ
        dz = to_f64(dz_rows)[keep]
        want = ref["dz"][keep]
        if dz_rows.dtype == torch.bfloat16:
            want = oracle.round_to_bf16(want)
        assert rel_l2(dz, want) <= 1e-3, rel_l2(dz, want)
        assert not dz[~valid[keep]].any()


def sample_tokens(mask_np, row_len, n_valid=24, n_masked=8, seed=0):
    """Token indices to check one by one: first/last positions of rows, random
    valid tokens, random masked tokens."""
    rng = np.random.default_rng(seed)
    v = np.nonzero(mask_np)[0]
    m = np.nonzero(mask_np == 0)[0]
    pick = list(rng.choice(v, size=min(n_valid, len(v)), replace=False))
    if len(m):
        pick += list(rng.choice(m, size=min(n_masked, len(m)), replace=False))
    pick += [0, len(mask_np) - 1]
    for r0 in np.cumsum(np.concatenate([[0], row_len]))[:-1][:4]:
        pick.append(int(r0))
    return np.unique(np.asarray(pick, np.int64))
