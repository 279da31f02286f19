"""Helpers for the GPU parity tests: build a chunk's inputs on the GPU from the
seeded generators, run the oracle on the same values, and compare within the
stated tolerances.

Tolerances (the target's), applied token by token:
  * token log-prob: abs <= 1e-5 for fp32 logits, <= 2e-3 for bf16 logits;
  * loss: |dl_t| <= 1e-4 |l_t| per token, and for a chunk's sum
    |dL| <= 1e-4 * max(|L|, sum|l_t| / N) (relative, guarded near 0);
  * dlogits, per token: every element within one bf16 ulp of the oracle
    rounded once to bf16 (bf16 output; bf16 storage alone is ~1.7e-3 off
    float64) or within 1e-5 relative (fp32 output), absolute floor at the
    fp32 normal minimum, plus the float32 cancellation allowance of elements
    that are differences; the non-target elements no further from the exact
    row than the once-rounded oracle plus 1e-3 of the row's norm
    (check_dz_rows);
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


FP32_NORMAL_MIN = 2.0 ** -126


def bf16_ulp(x):
    """Spacing of the bf16 grid at |x| (8 significant bits): 2^(e-7) for
    2^e <= |x| < 2^(e+1); 2^-133 in the subnormal range."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)                       # ax = m 2^e, 0.5 <= m < 1
    return np.exp2(np.maximum(e - 8, -133).astype(np.float64))


def check_dz_rows(dz, want, target, valid, check, out_bf16, coef, mag=None, extra=None, label=""):
    """dlogits rows of the compared tokens against the oracle, token by token.

    ``dz``: the kernel's rows (float64 [n, V]); ``want``: the oracle's exact
    rows; ``check``: tokens whose values are compared (valid, finite, and with
    the same clip decision on both sides).  Masked tokens must be exactly zero.

    Per element: within one bf16 ulp of the oracle rounded once to bf16 (bf16
    output), or within 1e-5 relative (fp32 output), with an absolute floor at
    the fp32 normal minimum.  Where an element is a difference of larger
    summands, 1e-5 of the summands' magnitude ``mag`` is added (the float32
    cancellation error): by default ``mag`` = |dz_v| + |coef| [v = y] (the
    target element coef (p_y - 1)); with extra terms the caller passes it
    (KL: coef itself is a difference; entropy bonus: p_v (z_v - lse + H)).
    ``extra`` (absolute, per element) carries what an input error does to the
    element: with a KL term, the kernel's log-prob error moves coef through
    dKL/dlogp, and the caller passes that movement times (p_v + [v = y]).

    Per token, over the non-target elements (the target element carries most
    of a row's norm): the distance of the kernel's row to the exact row is at
    most that of the exact row rounded once to the output dtype, plus 1e-3 of
    the row's norm.  (A 1-ulp disagreement on one dominant element of a short
    row is an unavoidable consequence of rounding a float32 result that lies
    within 1e-6 of a rounding midpoint; it leaves the row as close to the
    exact one as the once-rounded oracle.)"""
    n, V = dz.shape
    assert not dz[~valid].any(), f"{label}: a masked token has a non-zero dlogits row"
    if not check.any():
        return
    got = dz[check]
    exact = want[check]
    tg = np.asarray(target)[check].astype(np.int64)
    inr = (tg >= 0) & (tg < V)
    if mag is None:
        m = np.abs(exact)
        m[np.nonzero(inr)[0], tg[inr]] += np.abs(np.asarray(coef, np.float64)[check][inr])
    else:
        m = mag[check]
    if out_bf16:
        ref = oracle.round_to_bf16(exact)
        bound = np.maximum(bf16_ulp(ref), FP32_NORMAL_MIN) + 1e-5 * m
    else:
        ref = exact
        bound = 1e-5 * np.maximum(m, np.abs(ref)) + FP32_NORMAL_MIN
    if extra is not None:
        bound = bound + extra[check]
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        t, v = np.argwhere(bad)[0]
        tok = np.nonzero(check)[0][t]
        raise AssertionError(f"{label}: {int(bad.sum())} elements outside the bound; first token {tok} v {v}: "
                             f"got {got[t, v]!r} want {ref[t, v]!r} bound {bound[t, v]!r}")
    off = np.ones_like(got, dtype=bool)
    off[np.nonzero(inr)[0], tg[inr]] = False
    norm = lambda x: np.sqrt(np.sum(np.where(off, x * x, 0.0), axis=1))  # noqa: E731
    excess = norm(got - exact) - norm(ref - exact) - 1e-3 * norm(exact)
    worst = int(np.argmax(excess))
    assert excess[worst] <= 0.0, (f"{label}: token {np.nonzero(check)[0][worst]}: non-target distance to the exact "
                                  f"row exceeds the once-rounded oracle's by {excess[worst]!r} beyond 1e-3 of its norm")


def check_tokens(out, ref, idx, old_np, in_dtype, dz_rows=None, eps=(0.2, 0.2), logp_tol=None, label="",
                 mag=None, extra=None):
    """Per-token outputs (dict of full-length GPU tensors) at token indices
    ``idx`` against the oracle dict ``ref`` (arrays over ``idx``), one token at
    a time:

    * flags: valid and non-finite exactly; the clip decision exactly except
      where the ratio lies within 1e-4 (relative) of a clip edge, since the
      kernel decides in float32 and the oracle in float64 -- such tokens may
      fall either way and are then left out of the dlogits comparison (their
      loss is continuous across the edge and stays in);
    * logp: abs <= 1e-5 (fp32 logits) / 2e-3 (bf16 logits); entropy:
      abs <= 1e-4 + 1e-5 H; loss: |dl_t| <= 1e-4 |l_t| (the relative bound with
      the near-zero guard of a single token); masked tokens: all zeros;
    * dlogits rows (``dz_rows``, the kernel's rows at ``idx``): check_dz_rows.

    Returns the number of clip-edge tokens whose decision differed."""
    idx = np.asarray(idx)
    ii = torch.as_tensor(idx, device=DEV)
    tol = logp_tol if logp_tol is not None else tol_logp(in_dtype)
    valid = ref["valid"]
    flags = out["tok_flags"][ii].cpu().numpy()
    assert np.array_equal((flags & 1).astype(bool), valid), label
    assert np.array_equal(((flags >> 2) & 1).astype(bool), ref["nonfinite"]), label
    fin = valid & ~ref["nonfinite"]
    logp = to_f64(out["logp"][ii])
    ent = to_f64(out["entropy"][ii])
    lt = to_f64(out["loss_tok"][ii])
    d_logp = np.abs(logp[fin] - ref["logp"][fin])
    assert np.all(d_logp <= tol), (label, float(np.max(d_logp)))
    d_ent = np.abs(ent[fin] - ref["entropy"][fin])
    assert np.all(d_ent <= 1e-4 + 1e-5 * np.abs(ref["entropy"][fin])), (label, float(np.max(d_ent)))
    d_l = np.abs(lt[fin] - ref["loss_tok"][fin])
    assert np.all(d_l <= 1e-4 * np.abs(ref["loss_tok"][fin])), (label, float(np.max(d_l - 1e-4 * np.abs(
        ref["loss_tok"][fin]))))
    assert not logp[~valid].any() and not lt[~valid].any() and not ent[~valid].any(), label
    with np.errstate(over="ignore", invalid="ignore"):
        rho = np.exp(ref["logp"] - np.asarray(old_np, np.float64))
    hi, lo = 1.0 + eps[1], 1.0 - eps[0]
    edge = fin & ((np.abs(rho - hi) <= 1e-4 * hi) | (np.abs(rho - lo) <= 1e-4))
    gclip = ((flags >> 1) & 1).astype(bool)
    differ = gclip != (ref["clipped"] & valid)
    assert not np.any(differ & ~edge), (label, np.nonzero(differ & ~edge))
    if dz_rows is not None:
        want = ref["dz"]
        check_dz_rows(to_f64(dz_rows), want, ref["_target"], valid, fin & ~differ, dz_rows.dtype == torch.bfloat16,
                      ref["coef"], mag=mag, extra=extra, label=label)
    return int(differ.sum())


def summand_magnitude(z64, ref, target, coef_mag, s_tok=None, ent_coef=0.0):
    """Magnitude of the summands that form each dz element (float64 [n, V]):
    coef_mag_t (p_v + [v = y]) plus, with an entropy bonus,
    |ent_coef s_t| p_v (|z_v - lse| + H).  ``coef_mag``: per token, the summed
    magnitudes of the terms of coef (|s A rho g| + |s kl_coef dKL/dlogp|)."""
    lse = ref["lse"][:, None]
    n, V = z64.shape
    with np.errstate(invalid="ignore", over="ignore"):
        fin = np.isfinite(z64)
        p = np.where(fin, np.exp(np.where(fin, z64, 0.0) - lse), 0.0)
        mag = np.asarray(coef_mag, np.float64)[:, None] * p
        tg = np.asarray(target).astype(np.int64)
        inr = (tg >= 0) & (tg < V)
        mag[np.nonzero(inr)[0], tg[inr]] += np.asarray(coef_mag, np.float64)[inr]
        if ent_coef:
            mag += np.abs(ent_coef * np.asarray(s_tok, np.float64))[:, None] * p * (
                np.where(fin, np.abs(np.where(fin, z64, 0.0) - lse), 0.0) + np.abs(ref["entropy"])[:, None])
    mag[~ref["valid"]] = 0.0
    return mag


def assert_tokens_match(ws, ref, d, idx=None, check_dz=True, eps=(0.2, 0.2), coef_mag=None, s_tok=None,
                        ent_coef=0.0, coef_err=None):
    """Per-token outputs and dlogits of a chunk (``make_chunk``) vs the oracle,
    token by token (``idx``: a token subset); see check_tokens.  With extra
    terms, ``coef_mag`` is each token's |s A rho g| + |s kl_coef dKL/dlogp|,
    ``s_tok`` its factor, ``ent_coef`` the entropy-bonus weight and
    ``coef_err`` the movement of coef that the kernel's log-prob error
    causes (per token)."""
    sel = np.arange(d["z64"].shape[0]) if idx is None else np.asarray(idx)
    ref = dict(ref, _target=d["target"][sel])
    dz = ws.get("dlogits") if check_dz else None
    dz_rows = dz[torch.as_tensor(sel, device=DEV)] if dz is not None else None
    mag = extra = None
    if dz_rows is not None and (coef_mag is not None or ent_coef):
        cm = np.abs(ref["coef"]) if coef_mag is None else np.asarray(coef_mag)[sel]
        mag = summand_magnitude(d["z64"][sel], ref, d["target"][sel], cm, None if s_tok is None else
                                np.asarray(s_tok)[sel], ent_coef)
    if dz_rows is not None and coef_err is not None:
        extra = summand_magnitude(d["z64"][sel], ref, d["target"][sel], np.asarray(coef_err)[sel])
    differ = check_tokens(ws, ref, sel, d["old"][sel], d["dtype"], dz_rows=dz_rows, eps=eps, mag=mag, extra=extra)
    # the chunk's loss as a sum, with the guarded relative bound
    fin = ref["valid"] & ~ref["nonfinite"]
    lt = to_f64(ws["loss_tok"][torch.as_tensor(sel, device=DEV)])
    L_ref = float(np.sum(ref["loss_tok"][fin]))
    bound = 1e-4 * max(abs(L_ref), float(np.sum(np.abs(ref["loss_tok"][fin]))))
    assert abs(float(np.sum(lt[fin])) - L_ref) <= max(bound, 1e-12)
    return differ


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


def compare_sampled(out, ref, idx, old_np, dtype, dz_rows=None, eps=(0.2, 0.2), target=None, logp_tol=None):
    """Per-token outputs (dicts of full-length GPU tensors) at ``idx`` vs the
    oracle dict ``ref``; ``dz_rows``: the kernel's dlogits rows at ``idx``
    (``target``: the targets at ``idx``, needed with dz_rows).  See
    check_tokens."""
    if dz_rows is not None and target is None:
        raise ValueError("compare_sampled: the targets at idx are needed to compare dlogits rows")
    ref = dict(ref, _target=np.asarray(target) if target is not None else None)
    return check_tokens(out, ref, idx, old_np, dtype, dz_rows=dz_rows, eps=eps, logp_tol=logp_tol)


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



CLIP_EDGE = 1e-3


def old_at_kernel_clip(flags, ref, old, adv_tok, eps=(0.2, 0.2)):
    """Old log-probs that make the oracle take the kernel's clip decision
    (bit 1 of ``flags``, the kernel's tok_flags over the tokens of ``ref``).

    The gate of the clipped surrogate is an integer decision on the ratio: the
    kernel takes it in float32, the oracle in float64, and where the ratio
    lies within CLIP_EDGE (relative) of the bound that applies (1 + eps_high
    for A > 0, 1 - eps_low for A < 0) both are right.  A token's own gradient
    row follows its own decision, but a sum over tokens (dW) holds every one,
    so the reference is re-evaluated at the kernel's decision: an edge token
    whose decision differs gets the old log-prob that puts the oracle's ratio
    1e-9 (relative) from the bound on the kernel's side, which moves its ratio
    by no more than the kernel's own log-prob error; no other input changes.
    A decision that differs away from an edge fails.

    Returns ``(old2, n_moved)``, ``old2`` None when every decision agrees."""
    old = np.asarray(old, np.float64)
    adv_tok = np.asarray(adv_tok, np.float64)
    valid = np.asarray(ref["valid"], bool)
    gclip = ((np.asarray(flags) >> 1) & 1).astype(bool) & valid
    differ = gclip != (np.asarray(ref["clipped"], bool) & valid)
    if not differ.any():
        return None, 0
    bound = np.where(adv_tok > 0, 1.0 + eps[1], 1.0 - eps[0])
    with np.errstate(over="ignore"):
        rho = np.exp(ref["logp"] - old)
    near = np.abs(rho - bound) <= CLIP_EDGE * bound
    assert np.all(near[differ]), ("clip decision differs away from an edge", np.nonzero(differ & ~near))
    side = np.sign(adv_tok) * np.where(gclip, 1.0, -1.0)   # +1: the ratio goes above the bound
    old2 = old.copy()
    old2[differ] = ref["logp"][differ] - (np.log(bound[differ]) + side[differ] * 1e-9)
    return old2, int(differ.sum())


def oracle_lmhead_at_kernel_clip(flags, h64, W64, target, mask, old, adv_tok, scale, eps=(0.2, 0.2), **terms):
    """oracle.lmhead_fwd_bwd with each clip-edge token at the kernel's clip
    decision (old_at_kernel_clip).  Returns ``(ref, n_moved)``."""
    old = np.asarray(old, np.float64)
    adv_tok = np.asarray(adv_tok, np.float64)
    ref = oracle.lmhead_fwd_bwd(h64, W64, target, mask, old, adv_tok, scale, eps[0], eps[1], **terms)
    old2, moved = old_at_kernel_clip(flags, ref, old, adv_tok, eps)
    if old2 is None:
        return ref, 0
    ref2 = oracle.lmhead_fwd_bwd(h64, W64, target, mask, old2, adv_tok, scale, eps[0], eps[1], **terms)
    gclip = ((np.asarray(flags) >> 1) & 1).astype(bool) & ref2["valid"]
    assert np.array_equal(ref2["clipped"] & ref2["valid"], gclip)
    return ref2, moved
