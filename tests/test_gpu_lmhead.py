"""GPU parity of the fused LM-head variant (grpo_lmhead_fwd_bwd) against the
oracle: per-token outputs, dh and the accumulated dW, on ragged shapes
(tokens, hidden size and vocabulary not multiples of the 256x256x32 tiles, a
vocabulary spanning several pass-2 chunks), plus the context-compaction
workload at full size checked on sampled tokens and by properties.

dh / dW tolerance: relative L2 <= 4e-3 over the whole matrix, and row by row
(each dW row, each token's dh row) ||got - want|| <= (2^-8 + 2^-12) * ||M||,
where M sums the magnitudes of the products that form the row
(|dz|^T |h| for dW, |dz| |W| for dh): dz enters the two gradient GEMMs
rounded once to bf16, which moves each product by at most 2^-8 of its size
(the unit roundoff of 8 significant bits),
and 2^-12 allows for the float32 accumulation.  Per-token outputs use the
fused-loss tolerances per token, with logp / entropy abs <= 1e-4 (logits
from fp32-accumulated bf16 products)."""

import gc

import numpy as np
import pytest
import torch

import oracle
from gpu_common import DEV, old_at_kernel_clip, oracle_lmhead_at_kernel_clip, rel_l2, to_f64
from grpo_token_level_amd import ops

pytestmark = pytest.mark.gpu

TOL_GRAD = 4e-3


def _case(n, H, V, seed, h_std=1.0, w_std=0.05, noise=0.3, masked_frac=0.2, n_rows=3):
    g = torch.Generator(device="cpu").manual_seed(seed)
    h = (torch.randn((n, H), generator=g) * h_std).to(torch.bfloat16)
    W = (torch.randn((V, H), generator=g) * w_std).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    target = rng.integers(0, V, n).astype(np.int32)
    mask = (rng.random(n) > masked_frac).astype(np.uint8)
    cuts = np.sort(rng.choice(np.arange(1, max(n, 2)), size=min(n_rows - 1, max(n - 1, 0)), replace=False)) \
        if n > 1 else np.array([], np.int64)
    row_off = np.concatenate([[0], cuts, [n]]).astype(np.int64)
    nr = len(row_off) - 1
    tok_row = np.zeros(n, np.int32)
    for r in range(nr):
        tok_row[row_off[r]:row_off[r + 1]] = r
    adv = rng.normal(0, 1, nr).astype(np.float32)
    h64, W64 = h.double().numpy(), W.double().numpy()
    lp = oracle.logprob_fwd(h64 @ W64.T, target, np.ones(n, np.uint8))["logp"]
    old = (lp + rng.normal(0, noise, n)).astype(np.float32)
    G = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    return dict(h=h.to(DEV), W=W.to(DEV), h64=h64, W64=W64, target=target, mask=mask, old=old, adv=adv,
                tok_row=tok_row, row_off=row_off,
                g={k: G(v) for k, v in (("target", target), ("mask", mask), ("old", old), ("adv", adv),
                                        ("tok_row", tok_row), ("row_off", row_off))})


def _run(c, dW, scale, Wt=None, eps=(0.2, 0.2), keep_z=False):
    if Wt is None:
        Wt = ops.transpose_bf16(c["W"])
    g = c["g"]
    return ops.lmhead_fwd_bwd(c["h"], c["W"], Wt, g["target"], g["mask"], g["old"], g["tok_row"], g["adv"],
                              g["row_off"], dW, scale=scale, eps_low=eps[0], eps_high=eps[1], keep_z=keep_z)


def _ref(c, ws, scale, mask=None, adv_tok=None, **terms):
    """The oracle on the case's inputs, clip-edge tokens at the kernel's
    decision (oracle_lmhead_at_kernel_clip)."""
    ref, _ = oracle_lmhead_at_kernel_clip(
        ws["tok_flags"].cpu().numpy(), c["h64"], c["W64"], c["target"], c["mask"] if mask is None else mask,
        c["old"], c["adv"].astype(np.float64)[c["tok_row"]] if adv_tok is None else adv_tok, scale, **terms)
    return ref


GRAD_ROW = 2.0 ** -8 + 2.0 ** -12


def check_grad_rows(got, want, mag, label):
    """Row by row: ||got_r - want_r|| <= GRAD_ROW * ||mag_r|| (see module text)."""
    err = np.sqrt(np.sum((got - want) ** 2, axis=1))
    bound = GRAD_ROW * np.sqrt(np.sum(mag ** 2, axis=1))
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), (label, worst, float(err[worst]), float(bound[worst]))


def _check(ws, dW, ref, c, dW_ref, dz_ref=None):
    valid = ref["valid"]
    flags = ws["tok_flags"].cpu().numpy()
    assert np.array_equal((flags & 1).astype(bool), valid)
    logp = to_f64(ws["logp"])
    assert np.max(np.abs(logp[valid] - ref["logp"][valid]), initial=0) <= 1e-4
    ent = to_f64(ws["entropy"])
    assert np.max(np.abs(ent[valid] - ref["entropy"][valid]), initial=0) <= 1e-4
    lt = to_f64(ws["loss_tok"])
    assert np.all(np.abs(lt[valid] - ref["loss_tok"][valid]) <= 1e-4 * np.abs(ref["loss_tok"][valid]))
    assert not lt[~valid].any() and not logp[~valid].any()
    L = float(np.sum(ref["loss_tok"][valid]))
    assert abs(float(np.sum(lt[valid])) - L) <= 1e-4 * max(abs(L), float(np.sum(np.abs(ref["loss_tok"])))) + 1e-12
    # ref takes the kernel's decision on clip-edge tokens (_ref)
    gclip = ((flags >> 1) & 1).astype(bool)
    assert np.array_equal(gclip, ref["clipped"] & valid)
    assert rel_l2(to_f64(ws["dh"]), ref["dh"]) <= TOL_GRAD, rel_l2(to_f64(ws["dh"]), ref["dh"])
    assert rel_l2(to_f64(dW), dW_ref) <= TOL_GRAD, rel_l2(to_f64(dW), dW_ref)
    assert not to_f64(ws["dh"])[~valid].any()
    dz = ref["dz"] if dz_ref is None else dz_ref
    check_grad_rows(to_f64(ws["dh"]), ref["dh"], np.abs(dz) @ np.abs(c["W64"]), "dh")
    check_grad_rows(to_f64(dW), dW_ref, np.abs(dz).T @ np.abs(c["h64"]), "dW")


# ragged shapes: tokens, hidden size and vocabulary off the 256 x 256 tiles;
# several 256-wide dW / dh tile columns (H = 512, 768); a vocabulary spanning
# two pass-2 chunks of 65536 columns
# (each with the logits kept for pass 2, GRPO_LMHEAD_KEEP_Z, and without)
@pytest.mark.parametrize("keep_z", [False, True])
@pytest.mark.parametrize("n,H,V", [(1, 64, 256), (37, 64, 1000), (130, 96, 520), (300, 128, 16520),
                                   (257, 256, 4096), (300, 768, 5000), (213, 512, 70000)])
def test_lmhead_matches_oracle(n, H, V, keep_z):
    print(f"lmhead parity n={n} H={H} V={V} keep_z={keep_z}", flush=True)
    c = _case(n, H, V, seed=n + H + V)
    N = max(1, int(c["mask"].sum()))
    dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    ws = _run(c, dW, 1.0 / N, keep_z=keep_z)
    torch.cuda.synchronize()
    ref = _ref(c, ws, 1.0 / N)
    _check(ws, dW, ref, c, ref["dW"])
    st = ops.stats_to_dicts(ws["chunk_stats"])[0]
    assert st["n_valid"] == int(c["mask"].sum())


def _random_lmhead_shapes(count=32, seed=909):
    """Seeded random shapes: tokens 1..1999, H and V multiples of 8 (V log-uniform
    up to 80000, so some span two pass-2 chunks), masked fraction and segment
    count drawn too, and keep_z on half of them; n is cut so that n*H*V stays
    where the oracle takes well under a second."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        n = int(rng.integers(1, 2000))
        H = 8 * int(rng.integers(1, 193))
        V = 8 * int(np.exp(rng.uniform(np.log(2), np.log(10000))))
        n = max(1, min(n, int(1e11 // (H * V))))
        out.append((k, n, H, V, bool(rng.random() < 0.5), float(rng.choice([0.0, 0.2, 0.9])),
                    int(rng.integers(1, 6))))
    return out


@pytest.mark.parametrize("k,n,H,V,keep_z,masked,n_rows", _random_lmhead_shapes())
def test_lmhead_random_shapes_match_oracle(k, n, H, V, keep_z, masked, n_rows):
    print(f"lmhead random k={k} n={n} H={H} V={V} keep_z={keep_z} masked={masked} rows={n_rows}", flush=True)
    c = _case(n, H, V, seed=3000 + k, masked_frac=masked, n_rows=n_rows)
    N = max(1, int(c["mask"].sum()))
    dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    ws = _run(c, dW, 1.0 / N, keep_z=keep_z)
    torch.cuda.synchronize()
    ref = _ref(c, ws, 1.0 / N)
    _check(ws, dW, ref, c, ref["dW"])


def test_lmhead_accumulates_dW_over_chunks():
    # two micro-batch chunks: dW holds the sum, dh each chunk's own
    n, H, V = 160, 64, 2048
    c = _case(n, H, V, seed=5)
    N = int(c["mask"].sum())
    Wt = ops.transpose_bf16(c["W"])
    dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    dhs, flags = [], []
    for a, b in ((0, 90), (90, n)):
        sub = dict(c)
        sub["h"] = c["h"][a:b]
        sub["g"] = dict(c["g"])
        for k in ("target", "mask", "old", "tok_row"):
            sub["g"][k] = c["g"][k][a:b]
        sub["g"]["tok_row"] = torch.zeros(b - a, dtype=torch.int32, device=DEV)
        sub["g"]["adv"] = c["g"]["adv"][:1].clone()
        sub["g"]["row_off"] = torch.tensor([0, b - a], dtype=torch.int64, device=DEV)
        ws = _run(sub, dW, 1.0 / N, Wt=Wt)
        dhs.append(ws["dh"].clone())
        flags.append(ws["tok_flags"].clone())
    torch.cuda.synchronize()
    adv_tok = np.full(n, float(c["adv"][0]))
    ref = _ref(c, {"tok_flags": torch.cat(flags)}, 1.0 / N, adv_tok=adv_tok)
    assert rel_l2(to_f64(dW), ref["dW"]) <= TOL_GRAD
    assert rel_l2(to_f64(torch.cat(dhs)), ref["dh"]) <= TOL_GRAD


@pytest.mark.parametrize("n,H,V,bonus", [(700, 256, 70000, 0.0), (513, 512, 20000, 0.01)])
def test_keep_z_equals_the_recompute(n, H, V, bonus):
    # Pass 2 from the stored logits forms dz with the recomputing GEMM's
    # arithmetic on the same fp32 z: per-token outputs and dW (each dW element
    # one GEMM tile over the tokens in the same order) are equal bit for bit;
    # dh sums the same bf16 products split over the vocabulary another way,
    # so its rows agree to float32 summation order.  With the entropy bonus
    # (dz = p (ea + eb t)) as well.
    print(f"keep_z vs recompute n={n} H={H} V={V} bonus={bonus}", flush=True)
    c = _case(n, H, V, seed=90 + n)
    N = max(1, int(c["mask"].sum()))
    Wt = ops.transpose_bf16(c["W"])
    out = []
    for keep in (False, True):
        dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
        g = c["g"]
        ws = ops.lmhead_fwd_bwd(c["h"], c["W"], Wt, g["target"], g["mask"], g["old"], g["tok_row"], g["adv"],
                                g["row_off"], dW, scale=1.0 / N, ent_coef=bonus, keep_z=keep)
        out.append((ws, dW))
    torch.cuda.synchronize()
    (wa, dWa), (wb, dWb) = out
    for k in ("logp", "lse", "entropy", "loss_tok", "tok_flags", "row_stats", "chunk_stats"):
        assert torch.equal(wa[k], wb[k]), k
    assert torch.equal(dWa, dWb)
    a, b = to_f64(wa["dh"]), to_f64(wb["dh"])
    err = np.sqrt(np.sum((a - b) ** 2, axis=1))
    assert np.all(err <= 1e-5 * np.sqrt(np.sum(a * a, axis=1)) + 1e-30), float(np.max(err))
    # the fixed-scratch entry point cannot keep the logits
    with pytest.raises(ops.GrpoError) as e:
        g = c["g"]
        ops.lmhead_fwd_bwd(c["h"], c["W"], Wt, g["target"], g["mask"], g["old"], g["tok_row"], g["adv"],
                           g["row_off"], dWa, scale=1.0 / N, noalloc=True, keep_z=True)
    assert e.value.kind == "EINVAL"


def test_lmhead_equals_materialised_path():
    # The fused LM head against the materialised path made of a plain fp32
    # GEMM and this library's fused loss kernel: per-token outputs agree to
    # fp32 accuracy.
    n, H, V = 96, 128, 3000
    c = _case(n, H, V, seed=9)
    N = int(c["mask"].sum())
    dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    ws = _run(c, dW, 1.0 / N)
    z = (c["h"].float() @ c["W"].float().t()).contiguous()
    g = c["g"]
    ref = ops.loss_fwd_bwd(z, g["target"], g["mask"], g["old"], g["tok_row"], g["adv"], g["row_off"], scale=1.0 / N)
    torch.cuda.synchronize()
    v = torch.from_numpy(c["mask"].astype(bool)).to(DEV)
    assert float((ws["logp"][v] - ref["logp"][v]).abs().max()) <= 2e-5
    assert float((ws["entropy"][v] - ref["entropy"][v]).abs().max()) <= 2e-5
    assert torch.equal(ws["tok_flags"] & 1, ref["tok_flags"] & 1)
    dz = ref["dlogits"].double().cpu().numpy()
    assert rel_l2(to_f64(ws["dh"]), dz @ c["W64"]) <= TOL_GRAD


@pytest.mark.parametrize("pattern", ["blocks", "sparse"])
def test_lmhead_skips_masked_tokens(pattern):
    # The GEMMs run over the valid tokens only (listed on the device): a chunk
    # spanning three 256-row tiles whose masked tokens come in long runs or
    # leave only one token in eight, against the oracle; dh rows of masked
    # tokens are zero and dW (pre-filled) gains exactly the valid tokens' share.
    n, H, V = 700, 128, 2000
    c = _case(n, H, V, seed=31 if pattern == "blocks" else 32, masked_frac=0.0)
    m = np.zeros(n, np.uint8)
    if pattern == "blocks":
        m[40:170] = 1
        m[300:310] = 1
        m[650:] = 1
    else:
        m[::8] = 1
    c["mask"] = m
    c["g"]["mask"] = torch.from_numpy(m).to(DEV)
    N = int(m.sum())
    base = torch.randn((V, H), generator=torch.Generator(device="cpu").manual_seed(3)).to(DEV) * 1e-3
    dW = base.clone()
    ws = _run(c, dW, 1.0 / N)
    torch.cuda.synchronize()
    ref = _ref(c, ws, 1.0 / N, mask=m)
    _check(ws, dW - base, ref, c, ref["dW"])
    assert ops.stats_to_dicts(ws["chunk_stats"])[0]["n_valid"] == N


def test_lmhead_all_masked_chunk():
    # no valid token: every GEMM tile exits, dW keeps its bits, outputs are zero
    n, H, V = 300, 64, 1000
    c = _case(n, H, V, seed=33)
    c["mask"] = np.zeros(n, np.uint8)
    c["g"]["mask"] = torch.zeros(n, dtype=torch.uint8, device=DEV)
    dW = torch.randn((V, H), generator=torch.Generator(device="cpu").manual_seed(4)).to(DEV)
    before = dW.clone()
    ws = _run(c, dW, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(dW, before)
    for k in ("dh", "logp", "entropy", "loss_tok", "tok_flags"):
        assert not ws[k].any(), k
    st = ops.stats_to_dicts(ws["chunk_stats"])[0]
    assert st["n_valid"] == 0 and st["loss_sum"] == 0.0


def _chunk_calls(c, bounds, scale, dW=None, window=None, keep_z=False, Wt=None):
    """Each [a, b) of ``bounds`` as a call of its own (one row, the advantage
    adv[i] of chunk i).  Returns the per-token outputs of all chunks
    concatenated and each token's advantage."""
    if Wt is None:
        Wt = ops.transpose_bf16(c["W"])
    n = c["h"].shape[0]
    adv_tok = np.zeros(n)
    out = {k: [] for k in ("dh", "logp", "entropy", "loss_tok", "tok_flags")}
    for i, (a, b) in enumerate(bounds):
        A = float(c["adv"][i % len(c["adv"])])
        adv_tok[a:b] = A
        g = c["g"]
        ws = ops.lmhead_fwd_bwd(c["h"][a:b], c["W"], Wt, g["target"][a:b], g["mask"][a:b], g["old"][a:b],
                                torch.zeros(b - a, dtype=torch.int32, device=DEV),
                                torch.tensor([A], dtype=torch.float32, device=DEV),
                                torch.tensor([0, b - a], dtype=torch.int64, device=DEV), dW, scale=scale,
                                keep_z=keep_z, dw_window=window)
        for k in out:
            out[k].append(ws[k].clone())
    return {k: torch.cat(v) for k, v in out.items()}, adv_tok


# GRPO_LMHEAD_DEFER_DW: chunks of 130, 1, 319 and 250 tokens (a one-token
# chunk; columns 192 + 64 + 320 + 256 = 832 = the window's exact capacity)
# append to one window; the flush adds the step's dW to a non-zero dW.  H =
# 320 has a ragged 256-wide tile column; V = 70000 spans two pass-2 chunks on
# the default path.  Against the oracle over all tokens, and against the
# chunk-by-chunk dW: the same dz bits, so the two differ only by the order of
# the float32 sums (row by row within 2^-16 of the products' magnitudes).
@pytest.mark.parametrize("keep_z", [False, True])
def test_deferred_dW_matches_oracle(keep_z):
    n, H, V = 700, 320, 70000
    print(f"deferred dW n={n} H={H} V={V} keep_z={keep_z}", flush=True)
    c = _case(n, H, V, seed=77)
    N = int(c["mask"].sum())
    bounds = [(0, 130), (130, 131), (131, 450), (450, n)]
    Wt = ops.transpose_bf16(c["W"])
    win = ops.LmheadDwWindow(832, H, V, device=DEV)
    out, adv_tok = _chunk_calls(c, bounds, 1.0 / N, window=win, keep_z=keep_z, Wt=Wt)
    assert win.reserved == 832
    base = torch.randn((V, H), generator=torch.Generator(device="cpu").manual_seed(8)).to(DEV) * 1e-3
    dW = base.clone()
    win.flush(dW)
    assert win.reserved == 0
    dW_chunked = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    out2, _ = _chunk_calls(c, bounds, 1.0 / N, dW=dW_chunked, keep_z=keep_z, Wt=Wt)
    torch.cuda.synchronize()
    for k in ("logp", "entropy", "loss_tok", "tok_flags"):
        assert torch.equal(out[k], out2[k]), k
    ref = _ref(c, {"tok_flags": out["tok_flags"]}, 1.0 / N, adv_tok=adv_tok)
    _check(out, dW - base, ref, c, ref["dW"])
    got, chunked = to_f64(dW - base), to_f64(dW_chunked)
    mag = np.abs(ref["dz"]).T @ np.abs(c["h64"])
    err = np.sqrt(np.sum((got - chunked) ** 2, axis=1))
    assert np.all(err <= 2.0 ** -16 * np.sqrt(np.sum(mag ** 2, axis=1))), float(np.max(err))


def _random_window_cases(count=12, seed=31):
    """Seeded random chunk splits through one dW window: tokens 2..1499 in 1-5
    chunks, H and V multiples of 8 (V up to 96000), masked fraction drawn,
    kept logits on half of them, and a window with 0-2 spare 64-column blocks."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        n = int(rng.integers(2, 1500))
        H = 8 * int(rng.integers(1, 129))
        V = 8 * int(np.exp(rng.uniform(np.log(2), np.log(12000))))
        n = max(2, min(n, int(8e10 // (H * V))))
        keep = bool(rng.random() < 0.5)
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(int(rng.integers(0, 5)), n - 1), replace=False))
        bounds = tuple(zip([0, *cuts.tolist()], [*cuts.tolist(), n]))
        out.append((k, n, H, V, keep, bounds, float(rng.choice([0.0, 0.2, 0.9])), int(rng.integers(0, 3))))
    return out


@pytest.mark.parametrize("k,n,H,V,keep_z,bounds,masked,spare", _random_window_cases())
def test_random_chunk_splits_through_a_window_match_oracle(k, n, H, V, keep_z, bounds, masked, spare):
    print(f"window random k={k} n={n} H={H} V={V} keep_z={keep_z} chunks={len(bounds)}", flush=True)
    c = _case(n, H, V, seed=6000 + k, masked_frac=masked)
    N = max(1, int(c["mask"].sum()))
    win = ops.LmheadDwWindow(sum((b - a + 63) // 64 * 64 for a, b in bounds) + 64 * spare, H, V, device=DEV)
    out, adv_tok = _chunk_calls(c, list(bounds), 1.0 / N, window=win, keep_z=keep_z)
    dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    win.flush(dW)
    torch.cuda.synchronize()
    ref = _ref(c, {"tok_flags": out["tok_flags"]}, 1.0 / N, adv_tok=adv_tok)
    _check(out, dW, ref, c, ref["dW"])


def test_dW_window_capacity_reuse_and_empty_flushes():
    n, H, V = 200, 64, 1000
    c = _case(n, H, V, seed=12)
    N = int(c["mask"].sum())
    Wt = ops.transpose_bf16(c["W"])
    win = ops.LmheadDwWindow(256, H, V, device=DEV)
    dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    # an empty window's flush leaves dW as it is
    win.flush(dW)
    out_a, adv_a = _chunk_calls(c, [(0, 200)], 1.0 / N, window=win, Wt=Wt)
    assert win.reserved == 256
    # no room for one more token: refused before any launch, nothing reserved
    with pytest.raises(ops.GrpoError) as e:
        _chunk_calls(c, [(0, 1)], 1.0 / N, window=win, Wt=Wt)
    assert e.value.kind == "ECAPACITY" and win.reserved == 256
    win.flush(dW)
    torch.cuda.synchronize()
    ref = _ref(c, {"tok_flags": out_a["tok_flags"]}, 1.0 / N, adv_tok=adv_a)
    _check(out_a, dW, ref, c, ref["dW"])
    # a second empty flush, and an all-masked chunk, change no bit of dW
    before = dW.clone()
    win.flush(dW)
    masked = dict(c)
    masked["g"] = dict(c["g"])
    masked["g"]["mask"] = torch.zeros(n, dtype=torch.uint8, device=DEV)
    _chunk_calls(masked, [(0, 150)], 1.0 / N, window=win, Wt=Wt)
    assert win.reserved == 192
    win.flush(dW)
    torch.cuda.synchronize()
    assert torch.equal(dW, before) and win.reserved == 0
    # the window starts over after a flush: the same chunk again doubles dW
    _chunk_calls(c, [(0, 200)], 1.0 / N, window=win, Wt=Wt)
    win.flush(dW)
    torch.cuda.synchronize()
    check_grad_rows(to_f64(dW), 2.0 * ref["dW"], 2.0 * np.abs(ref["dz"]).T @ np.abs(c["h64"]), "dW twice")
    # the fixed-scratch entry point refuses the window
    g = c["g"]
    with pytest.raises(ops.GrpoError) as e:
        ops.lmhead_fwd_bwd(c["h"], c["W"], Wt, g["target"], g["mask"], g["old"], g["tok_row"], g["adv"],
                           g["row_off"], None, noalloc=True, dw_window=win)
    assert e.value.kind == "EINVAL"


# grpo_transpose_bf16 equals torch's transpose bit for bit: the 16-byte path
# (aligned pointers, row strides multiples of 8) and the element-wise one
# (a source stride of 1003, a destination view one element off 16-byte
# alignment), ragged edges of the 64 x 64 tiles, and the LM head's W
@pytest.mark.parametrize("rows,cols,ld_src,out_off", [(1, 1, 1, 0), (7, 13, 13, 0), (64, 64, 64, 0),
                                                     (65, 130, 136, 0), (300, 1000, 1003, 0), (257, 520, 520, 1),
                                                     (151936, 2048, 2048 + 8, 0)])
def test_transpose_bf16_matches_torch(rows, cols, ld_src, out_off):
    print(f"transpose rows={rows} cols={cols} ld_src={ld_src} out_off={out_off}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(rows + cols)
    base = torch.randn((rows, ld_src), generator=g, device=DEV).to(torch.bfloat16)
    x = base[:, :cols]
    store = torch.full((cols * rows + out_off,), 7.0, dtype=torch.bfloat16, device=DEV)
    out = store[out_off:].view(cols, rows)
    ops.transpose_bf16(x, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, x.t())
    assert out_off == 0 or float(store[0]) == 7.0


def test_lmhead_rejects_small_workspace_and_bad_shapes():
    c = _case(8, 64, 256, seed=1)
    Wt = ops.transpose_bf16(c["W"])
    g = c["g"]
    dW = torch.zeros((256, 64), dtype=torch.float32, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ops.GrpoError) as e:
        ops.lmhead_fwd_bwd(c["h"], c["W"], Wt, g["target"], g["mask"], g["old"], g["tok_row"], g["adv"],
                           g["row_off"], dW, workspace=small)
    assert e.value.kind in ("ECAPACITY",) or "workspace" in str(e.value)


@pytest.mark.timeout(900)
def test_compaction_workload_full_size_sampled():
    """8 prompts x 4 rollouts, U{1..5} segment rows of U{256..1024} tokens, groups
    padded to a multiple of Q = 4 with masked copies of a real row, micro-batches
    of 4 rows, hidden 2048, V = 151936: every chunk through the fused LM head,
    dW accumulated over the chunks."""
    print("compaction workload at full size", flush=True)
    from synth import compaction_batch
    b = compaction_batch(seed=0)
    plan = ops.plan_compaction(b["rows_per_rollout"], b["n_groups"], b["group"], b["Q"],
                               b["n_groups"] * b["group"])
    want = oracle.plan_compaction(b["rows_per_rollout"].tolist(), b["n_groups"], b["group"], b["Q"],
                                  b["n_groups"] * b["group"])
    assert plan["row_src"].tolist() == want["row_src"] and plan["is_pad"].tolist() == want["is_pad"]
    H, V = b["H"], b["V"]
    seg_len = b["seg_len"]
    row_len = np.array([seg_len[s] for s in plan["row_src"]], np.int64)
    off = np.concatenate([[0], np.cumsum(row_len)])
    n_tok = int(off[-1])
    seg_off = np.concatenate([[0], np.cumsum(seg_len)])
    # token-level inputs in padded-row order; a pad copies its source row's tokens
    src_tok = np.concatenate([np.arange(seg_off[s], seg_off[s] + seg_len[s]) for s in plan["row_src"]])
    target = b["target"][src_tok]
    mask = np.repeat(1 - plan["is_pad"].astype(np.uint8), row_len).astype(np.uint8)
    noise = b["logratio_noise"][src_tok]
    gen = torch.Generator(device=DEV).manual_seed(11)
    W = (torch.randn((V, H), generator=gen, device=DEV) * b["w_std"]).to(torch.bfloat16)
    h_seg = (torch.randn((int(seg_off[-1]), H), generator=gen, device=DEV) * b["h_std"]).to(torch.bfloat16)
    h = h_seg[torch.as_tensor(src_tok, device=DEV)].contiguous()
    Wt = ops.transpose_bf16(W)
    adv_roll = ops.group_advantage(b["reward"], b["group"])
    adv_row = ops.rows_advantage(adv_roll, plan["row_rollout"])
    G = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    tgt_d, mask_d = G(target), G(mask)
    # old log-probs: current log-probs (plain PyTorch fp32 on the materialised
    # rows of one chunk at a time) plus the workload's drift
    old = torch.empty(n_tok, dtype=torch.float32, device=DEV)
    Wf = W.float()
    for a in range(0, n_tok, 1024):
        e = min(a + 1024, n_tok)
        z = h[a:e].float() @ Wf.t()
        old[a:e] = torch.log_softmax(z, -1).gather(1, tgt_d[a:e].long()[:, None])[:, 0]
    old += G(noise).float()
    del Wf, z
    N = ops.count_valid(mask_d)
    assert int(N.item()) == int(mask.sum())
    dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    dh = torch.empty((n_tok, H), dtype=torch.float32, device=DEV)
    out = {k: torch.empty(n_tok, dtype=torch.float32, device=DEV) for k in ("logp", "lse", "entropy", "loss_tok")}
    out["tok_flags"] = torch.empty(n_tok, dtype=torch.uint8, device=DEV)
    chunks = oracle.compaction_micro_chunks(plan["n_rows"], b["micro"])
    stats = torch.empty((len(chunks), ops.STATS_BYTES), dtype=torch.uint8, device=DEV)
    row_stats = torch.empty((plan["n_rows"], ops.STATS_BYTES), dtype=torch.uint8, device=DEV)
    workspace = torch.empty(ops.lmhead_workspace_bytes(int(max(off[e] - off[a] for a, e in chunks)), H, V),
                            dtype=torch.uint8, device=DEV)
    for k, (a, e) in enumerate(chunks):
        t0, t1 = int(off[a]), int(off[e])
        ro = G(off[a:e + 1] - off[a])
        tr = ops.tok_row(ro, t1 - t0)
        ws = {kk: out[kk][t0:t1] for kk in out}
        ws["row_stats"] = row_stats[a:e]
        ws["chunk_stats"] = stats[k:k + 1]
        ops.lmhead_fwd_bwd(h[t0:t1], W, Wt, tgt_d[t0:t1], mask_d[t0:t1], old[t0:t1], tr, G(adv_row[a:e]), ro, dW,
                           denom=N, dh=dh[t0:t1], ws=ws, workspace=workspace)
    torch.cuda.synchronize()
    st = ops.stats_to_dicts(stats)
    assert sum(s["n_valid"] for s in st) == int(mask.sum())
    rows = ops.stats_to_dicts(row_stats)
    assert [r["n_valid"] for r in rows] == (row_len * (1 - plan["is_pad"])).tolist()
    # sampled tokens one by one against the oracle (z = W h_t in float64)
    rng = np.random.default_rng(4)
    valid_idx = np.nonzero(mask)[0]
    idx = np.concatenate([rng.choice(valid_idx, 12, replace=False), rng.choice(np.nonzero(mask == 0)[0], 2)])
    W64 = W.double().cpu().numpy()
    hh = h[torch.as_tensor(idx, device=DEV)].double().cpu().numpy()
    row_of = np.searchsorted(off, idx, side="right") - 1
    Nn = int(mask.sum())
    ii = torch.as_tensor(idx, device=DEV)
    ref, _ = oracle_lmhead_at_kernel_clip(out["tok_flags"][ii].cpu().numpy(), hh, W64, target[idx], mask[idx],
                                          old[ii].double().cpu().numpy(), adv_row.astype(np.float64)[row_of],
                                          1.0 / Nn)
    v = ref["valid"]
    assert np.max(np.abs(to_f64(out["logp"][ii])[v] - ref["logp"][v])) <= 1e-4
    assert rel_l2(to_f64(dh[ii]), ref["dh"]) <= TOL_GRAD
    # dW column sums vanish up to the bf16 rounding of dz: |sum_v dW[v,:]| is
    # bounded by sum_t |h_t| * 2^-8 |coef_t|
    col = dW.double().sum(0).abs()
    scale_ref = dW.double().abs().sum(0)
    assert float((col / scale_ref).max()) <= 1e-2
    # The step's chunks again, through one dW window (GRPO_LMHEAD_DEFER_DW, 23.6 GB
    # here): the same dz bits, so the flushed dW differs from the chunk-by-chunk dW
    # only by the order of its float32 sums over the step's 64.6 k valid tokens
    # (relative L2 <= 1e-4), and the per-token outputs are equal bit for bit (dh
    # rows to float32 summation order: the plan may split its vocabulary otherwise)
    print("compaction: the step's chunks through one dW window", flush=True)
    win = ops.LmheadDwWindow(sum((int(off[e] - off[a]) + 63) // 64 * 64 for a, e in chunks), H, V, device=DEV)
    ws_defer = torch.empty(ops.lmhead_workspace_bytes(int(max(off[e] - off[a] for a, e in chunks)), H, V,
                                                      defer_dw=True), dtype=torch.uint8, device=DEV)
    out_w = {kk: torch.empty_like(v) for kk, v in out.items()}
    dh_w = torch.empty_like(dh)
    for k, (a, e) in enumerate(chunks):
        t0, t1 = int(off[a]), int(off[e])
        ro = G(off[a:e + 1] - off[a])
        ws = {kk: out_w[kk][t0:t1] for kk in out_w}
        ws["row_stats"] = row_stats[a:e]
        ws["chunk_stats"] = stats[k:k + 1]
        ops.lmhead_fwd_bwd(h[t0:t1], W, Wt, tgt_d[t0:t1], mask_d[t0:t1], old[t0:t1], ops.tok_row(ro, t1 - t0),
                           G(adv_row[a:e]), ro, None, denom=N, dh=dh_w[t0:t1], ws=ws, workspace=ws_defer,
                           dw_window=win)
    dW_w = torch.zeros_like(dW)
    win.flush(dW_w)
    torch.cuda.synchronize()
    for key in ("logp", "entropy", "loss_tok", "tok_flags"):
        assert torch.equal(out_w[key], out[key]), key
    assert bool(((dh_w - dh).norm(dim=1) <= 1e-5 * dh.norm(dim=1) + 1e-30).all())
    rel = float((dW_w - dW).norm() / dW.norm())
    assert rel <= 1e-4, rel
    print(f"compaction: window dW vs chunk-by-chunk dW, relative L2 {rel:.2e}", flush=True)
    del win, ws_defer, dW_w, dh_w, out_w
    del dW
    gc.collect()
    torch.cuda.empty_cache()
    # One whole chunk alone, against the oracle on every token: z = h W^T as a
    # float32 product of the exact bf16 values on the host, float64 after.
    # dW rows of 64 vocabulary ids (the targets of some of the chunk's tokens
    # and random others) and dh rows of 128 tokens, row by row.
    k = int(np.argmax([int(mask[int(off[a]):int(off[e])].sum()) for a, e in chunks]))
    a, e = chunks[k]
    t0, t1 = int(off[a]), int(off[e])
    n_c = t1 - t0
    print(f"compaction: chunk {k} alone ({n_c} tokens) against the oracle", flush=True)
    ro = G(off[a:e + 1] - off[a])
    dW1 = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    dh1 = torch.empty((n_c, H), dtype=torch.float32, device=DEV)
    ws1 = ops.lmhead_fwd_bwd(h[t0:t1], W, Wt, tgt_d[t0:t1], mask_d[t0:t1], old[t0:t1], ops.tok_row(ro, n_c),
                             G(adv_row[a:e]), ro, dW1, denom=N, dh=dh1, workspace=workspace)
    # the same chunk with its logits kept for pass 2 (GRPO_LMHEAD_KEEP_Z): dz
    # has the same bits, so dW has; dh agrees to float32 summation order
    del workspace
    dW1k = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    dh1k = torch.empty((n_c, H), dtype=torch.float32, device=DEV)
    ws1k = ops.lmhead_fwd_bwd(h[t0:t1], W, Wt, tgt_d[t0:t1], mask_d[t0:t1], old[t0:t1], ops.tok_row(ro, n_c),
                              G(adv_row[a:e]), ro, dW1k, denom=N, dh=dh1k, keep_z=True)
    torch.cuda.synchronize()
    assert torch.equal(dW1k, dW1)
    for key in ("logp", "entropy", "loss_tok", "tok_flags"):
        assert torch.equal(ws1k[key], ws1[key]), key
    dka, dkb = to_f64(dh1), to_f64(dh1k)
    assert np.all(np.sqrt(np.sum((dka - dkb) ** 2, axis=1)) <= 1e-5 * np.sqrt(np.sum(dka * dka, axis=1)) + 1e-30)
    del dW1k, dh1k, ws1k, dka, dkb
    torch.cuda.empty_cache()
    h_c = h[t0:t1].float().cpu().numpy()
    Wf32 = W.float().cpu().numpy()
    z = h_c @ Wf32.T
    del Wf32
    row_c = np.searchsorted(off[a:e + 1] - off[a], np.arange(n_c), side="right") - 1
    m_c = mask[t0:t1]
    vrows = np.nonzero(m_c)[0]
    rows = np.sort(rng.choice(vrows, size=min(128, len(vrows)), replace=False))
    cols = np.unique(np.concatenate([target[t0:t1][rng.choice(vrows, 32, replace=False)],
                                     rng.choice(V, 32, replace=False)]))
    while len(cols) < 64:
        cols = np.unique(np.concatenate([cols, rng.choice(V, 64 - len(cols), replace=False)]))
    from oracle_pool import OraclePool
    old_c, adv_c = old[t0:t1].double().cpu().numpy(), adv_row.astype(np.float64)[a + row_c]
    with OraclePool() as P:
        ref = P.loss_host(z, target[t0:t1], m_c, old_c, adv_c, 1.0 / Nn, cols=cols, rows=rows)
        # clip-edge tokens at the kernel's decision (old_at_kernel_clip)
        old2, _ = old_at_kernel_clip(ws1["tok_flags"].cpu().numpy(), ref, old_c, adv_c)
        if old2 is not None:
            ref = P.loss_host(z, target[t0:t1], m_c, old2, adv_c, 1.0 / Nn, cols=cols, rows=rows)
    del z
    gclip = ((ws1["tok_flags"].cpu().numpy() >> 1) & 1).astype(bool)
    assert np.array_equal(gclip, ref["clipped"] & ref["valid"])
    for key in ("logp", "entropy"):
        got = to_f64(ws1[key])
        assert np.max(np.abs(got[m_c == 1] - ref[key][m_c == 1])) <= 1e-4, key
    lt = to_f64(ws1["loss_tok"])
    assert np.all(np.abs(lt - ref["loss_tok"]) <= 1e-4 * np.abs(ref["loss_tok"]))
    assert np.array_equal((ws1["tok_flags"].cpu().numpy() & 1).astype(bool), ref["valid"])
    h64 = h_c.astype(np.float64)
    dzc = ref["dz_cols"]
    check_grad_rows(to_f64(dW1[torch.as_tensor(cols, device=DEV)]), dzc.T @ h64, np.abs(dzc).T @ np.abs(h64),
                    "dW rows")
    dzr = np.stack([ref["dz_rows"][int(r)] for r in rows])
    check_grad_rows(to_f64(dh1[torch.as_tensor(rows, device=DEV)]), dzr @ W64, np.abs(dzr) @ np.abs(W64), "dh rows")
    assert not to_f64(dh1[torch.from_numpy(m_c == 0).to(DEV)]).any()
    del W, Wt, dW1, h, h_seg, W64
    gc.collect()
    torch.cuda.empty_cache()
