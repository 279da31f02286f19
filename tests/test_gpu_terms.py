"""GPU parity of the aggregation modes and the extra loss terms (entropy
bonus, KL against a reference) against the oracle: the row-count and
row-weight kernels, the fused loss on both kernel paths and dtypes, the
LM-head variant, chunk invariance of the seq-level modes, and the identity
of the plain path when the terms are off.

Tolerances as for the fused loss, with two allowances in the dlogits
element bound: the float32 cancellation between the terms that form an
element, and the movement of coef that the kernel's log-prob error causes
through the ratio and dKL/dlogp; KL per token abs <= 1e-5 (fp32 logits)
or 2e-4 (bf16: the log-prob error times |dKL/dlogp| <= ~0.5 here); row
weights relative 2^-23 (one float32 rounding of 1/(B L)); objective and KL
sums relative 1e-4 of the sum of magnitudes."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import DEV, assert_tokens_match, make_chunk, oracle_lmhead_at_kernel_clip, rel_l2, to_f64
from grpo_token_level_amd import ops
from grpo_token_level_amd._capi import KL_K1, KL_K2, KL_K3, AGG_SEQ_MEAN_TOKEN_MEAN, AGG_SEQ_MEAN_TOKEN_SUM, \
    AGG_TOKEN_MEAN

pytestmark = pytest.mark.gpu

MODES = (AGG_TOKEN_MEAN, AGG_SEQ_MEAN_TOKEN_SUM, AGG_SEQ_MEAN_TOKEN_MEAN)


def _with_ref(d, seed, std=0.3):
    rng = np.random.default_rng(seed + 1000)
    lp = oracle.logprob_fwd(d["z64"], d["target"], np.ones(len(d["target"]), np.uint8))["logp"]
    d["ref"] = (lp + rng.normal(0, std, len(lp))).astype(np.float32)
    d["g"]["ref"] = torch.from_numpy(d["ref"]).to(DEV)
    return d


def _weights(d, mode):
    g = d["g"]
    B = ops.count_rows(g["mask"], g["row_off"])
    w = ops.row_weights(g["mask"], g["row_off"], mode, B)
    return B, w


def _oracle_terms(d, mode, ent, kap, kind, scale):
    off = d["row_off"].tolist()
    B = oracle.count_rows(d["mask"], off)
    w_tok = np.repeat(oracle.row_weights(d["mask"], off, mode, B), np.diff(off))
    adv_tok = d["adv_row"].astype(np.float64)[d["tok_row"]]
    return oracle.loss_fwd_bwd(d["z64"], d["target"], d["mask"], d["old"].astype(np.float64), adv_tok, scale,
                               w_tok=w_tok, ent_coef=ent, kl_coef=kap, ref_logp=d["ref"].astype(np.float64),
                               kl_type=kind)


def _s_tok(d, mode, scale):
    """Each token's factor: scale times its row's aggregation weight."""
    off = d["row_off"].tolist()
    B = oracle.count_rows(d["mask"], off)
    return scale * np.repeat(np.asarray(oracle.row_weights(d["mask"], off, mode, B), np.float64), np.diff(off))


def _coef_mag(d, ref, mode, scale, kap, kind):
    """|s A rho g| + |s kl_coef dKL/dlogp| per token: the two terms of coef,
    whose float32 difference the dz bound allows for."""
    s = _s_tok(d, mode, scale)
    A = d["adv_row"].astype(np.float64)[d["tok_row"]]
    with np.errstate(over="ignore", invalid="ignore"):
        rho = np.where(ref["valid"], np.exp(ref["logp"] - d["old"].astype(np.float64)), 0.0)
    g = np.where(ref["clipped"], 0.0, 1.0)
    dkl = np.array([oracle.kl_term(lp, r, kind)[1] for lp, r in zip(ref["logp"], d["ref"].astype(np.float64))])
    return np.abs(s) * (np.abs(A * rho * g) + np.abs(kap * dkl))


def _coef_err(d, ref, ws, mode, scale, kap, kind):
    """How far coef moves when logp carries the kernel's own log-prob error
    (measured per token, which the logp bound limits): |d coef / d logp| =
    |s| (|A rho g| + |kl_coef d2KL/dlogp2|) with d2KL/dlogp2 = 0, 1, e^d for
    k1, k2, k3 (d = ref - logp), times that error plus float32 rounding."""
    s = _s_tok(d, mode, scale)
    A = d["adv_row"].astype(np.float64)[d["tok_row"]]
    with np.errstate(over="ignore", invalid="ignore"):
        rho = np.where(ref["valid"], np.exp(ref["logp"] - d["old"].astype(np.float64)), 0.0)
        dd = d["ref"].astype(np.float64) - ref["logp"]
        k2 = {KL_K1: 0.0 * dd, KL_K2: np.ones_like(dd), KL_K3: np.exp(dd)}[kind]
    g = np.where(ref["clipped"], 0.0, 1.0)
    dlogp = np.abs(to_f64(ws["logp"]) - ref["logp"]) + 2.0 ** -20 * (1.0 + np.abs(ref["logp"]))
    return np.where(ref["valid"], np.abs(s) * (np.abs(A * rho * g) + np.abs(kap * k2)) * dlogp, 0.0)


def _check_stats(ws, ref, d):
    # Row sums of signed terms (the k1 estimate, the objective) can cancel,
    # so the bound scales with the row's sum of magnitudes, as for the chunk.
    rows = ops.stats_to_dicts(ws["row_stats"])
    off = d["row_off"].tolist()
    want = oracle.row_stats(ref, off)
    for r, (g, w) in enumerate(zip(rows, want)):
        for k, per_tok in (("kl_sum", ref["kl"]), ("obj_sum", ref["obj"])):
            mag = float(np.sum(np.abs(per_tok[off[r]:off[r + 1]])))
            assert abs(g[k] - w[k]) <= 1e-4 * mag + 1e-9, (k, g[k], w[k], mag)
        assert g["n_valid"] == w["n_valid"]
    ch = ops.stats_to_dicts(ws["chunk_stats"])[0]
    cw = oracle.chunk_stats(ref, d["row_off"].tolist())
    mag = float(np.sum(np.abs(ref["obj"])))
    assert abs(ch["obj_sum"] - cw["obj_sum"]) <= 1e-4 * mag + 1e-9
    assert abs(ch["kl_sum"] - cw["kl_sum"]) <= 1e-4 * float(np.sum(np.abs(ref["kl"]))) + 1e-9


def test_count_rows_and_row_weights_match_oracle():
    for seed, n in ((1, 300), (2, 57), (3, 1)):
        d = make_chunk(n, 64, seed=seed, n_rows=max(1, n // 11), masked_frac=0.5)
        d["mask"][d["row_off"][0]:d["row_off"][1]] = 0          # one row fully masked (a pad)
        d["g"]["mask"].copy_(torch.from_numpy(d["mask"]))
        off = d["row_off"].tolist()
        B_ref = oracle.count_rows(d["mask"], off)
        for mode in MODES:
            B, w = _weights(d, mode)
            assert int(B.item()) == B_ref
            want = np.asarray(oracle.row_weights(d["mask"], off, mode, B_ref))
            got = to_f64(w[:len(want)])
            assert np.all(np.abs(got - want) <= 2.0 ** -23 * np.abs(want)), (mode, got, want)
    # empty mini-batch: B = 0, weights finite
    d = make_chunk(40, 64, seed=4, n_rows=5)
    d["g"]["mask"].zero_()
    B, w = _weights(d, AGG_SEQ_MEAN_TOKEN_MEAN)
    assert int(B.item()) == 0 and torch.all(w[:5] == 0)


@pytest.mark.parametrize("dtype,out_dtype", [(torch.float32, torch.float32), (torch.bfloat16, torch.bfloat16),
                                             (torch.bfloat16, torch.float32)])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("ent,kap,kind", [(0.01, 0.0, KL_K3), (0.0, 0.1, KL_K3), (0.02, 0.05, KL_K2),
                                          (0.005, 0.2, KL_K1)])
def test_terms_match_oracle(dtype, out_dtype, mode, ent, kap, kind):
    print(f"terms dtype={dtype} out={out_dtype} mode={mode} ent={ent} kl={kap}/{kind}", flush=True)
    d = _with_ref(make_chunk(96, 1000, dtype, seed=mode * 10 + kind, n_rows=9, noise=0.3), seed=kind)
    N = int(d["mask"].sum())
    scale = 1.0 / max(N, 1) if mode == AGG_TOKEN_MEAN else 1.0
    _, w = _weights(d, mode)
    g = d["g"]
    ws = ops.loss_fwd_bwd(d["logits"], g["target"], g["mask"], g["old"], g["tok_row"], g["adv_row"], g["row_off"],
                          scale=scale, out_dtype=out_dtype, row_weight=w, ref_logp=g["ref"], ent_coef=ent,
                          kl_coef=kap, kl_type=kind)
    torch.cuda.synchronize()
    ref = _oracle_terms(d, mode, ent, kap, kind, scale)
    assert_tokens_match(ws, ref, d, coef_mag=_coef_mag(d, ref, mode, scale, kap, kind), s_tok=_s_tok(d, mode, scale),
                        ent_coef=ent, coef_err=_coef_err(d, ref, ws, mode, scale, kap, kind))
    valid = ref["valid"]
    kl = to_f64(ws["kl_tok"])
    tol = 1e-5 if dtype == torch.float32 else 2e-4
    assert np.max(np.abs(kl[valid] - ref["kl"][valid]), initial=0) <= tol
    assert not kl[~valid].any()
    _check_stats(ws, ref, d)


def test_terms_on_the_generic_path():
    # a row stride that is not a multiple of 8 elements takes the streaming kernel
    d = _with_ref(make_chunk(40, 500, torch.bfloat16, seed=8, ld=501, noise=0.3), seed=8)
    _, w = _weights(d, AGG_SEQ_MEAN_TOKEN_MEAN)
    g = d["g"]
    ws = ops.loss_fwd_bwd(d["logits"], g["target"], g["mask"], g["old"], g["tok_row"], g["adv_row"], g["row_off"],
                          scale=1.0, out_dtype=torch.float32, row_weight=w, ref_logp=g["ref"], ent_coef=0.03,
                          kl_coef=0.1, kl_type=KL_K3)
    torch.cuda.synchronize()
    ref = _oracle_terms(d, AGG_SEQ_MEAN_TOKEN_MEAN, 0.03, 0.1, KL_K3, 1.0)
    assert_tokens_match(ws, ref, d, coef_mag=_coef_mag(d, ref, AGG_SEQ_MEAN_TOKEN_MEAN, 1.0, 0.1, KL_K3),
                        s_tok=_s_tok(d, AGG_SEQ_MEAN_TOKEN_MEAN, 1.0), ent_coef=0.03,
                        coef_err=_coef_err(d, ref, ws, AGG_SEQ_MEAN_TOKEN_MEAN, 1.0, 0.1, KL_K3))
    _check_stats(ws, ref, d)


@pytest.mark.parametrize("V", [151936, 256000])
def test_full_vocabulary_with_terms(V):
    # the 1024-thread register path with the bonus sweep (256000: the part of
    # each row past registers and LDS is read again in that sweep)
    d = _with_ref(make_chunk(12, V, torch.bfloat16, seed=9, n_rows=3, logit_std=3.0, noise=0.3), seed=9)
    _, w = _weights(d, AGG_SEQ_MEAN_TOKEN_SUM)
    g = d["g"]
    ws = ops.loss_fwd_bwd(d["logits"], g["target"], g["mask"], g["old"], g["tok_row"], g["adv_row"], g["row_off"],
                          scale=1.0, row_weight=w, ref_logp=g["ref"], ent_coef=0.01, kl_coef=0.05, kl_type=KL_K3)
    torch.cuda.synchronize()
    ref = _oracle_terms(d, AGG_SEQ_MEAN_TOKEN_SUM, 0.01, 0.05, KL_K3, 1.0)
    assert_tokens_match(ws, ref, d, coef_mag=_coef_mag(d, ref, AGG_SEQ_MEAN_TOKEN_SUM, 1.0, 0.05, KL_K3),
                        s_tok=_s_tok(d, AGG_SEQ_MEAN_TOKEN_SUM, 1.0), ent_coef=0.01,
                        coef_err=_coef_err(d, ref, ws, AGG_SEQ_MEAN_TOKEN_SUM, 1.0, 0.05, KL_K3))
    _check_stats(ws, ref, d)


def test_seq_mode_chunked_equals_unchunked():
    # global B and per-row weights: chunk by rows, dlogits bit-identical, objective adds up
    d = _with_ref(make_chunk(240, 512, torch.bfloat16, seed=10, n_rows=12, noise=0.3), seed=10)
    g = d["g"]
    _, w = _weights(d, AGG_SEQ_MEAN_TOKEN_MEAN)
    kw = dict(scale=1.0, ref_logp=g["ref"], ent_coef=0.02, kl_coef=0.1, kl_type=KL_K3)
    full = ops.loss_fwd_bwd(d["logits"], g["target"], g["mask"], g["old"], g["tok_row"], g["adv_row"], g["row_off"],
                            row_weight=w, **kw)
    full_dz = full["dlogits"].clone()
    full_obj = ops.stats_to_dicts(full["chunk_stats"])[0]["obj_sum"]
    off = d["row_off"]
    objs = 0.0
    for ra, rb in ((0, 5), (5, 12)):
        a, b = int(off[ra]), int(off[rb])
        sub_off = torch.from_numpy(off[ra:rb + 1] - a).to(DEV)
        sub_row = torch.from_numpy(d["tok_row"][a:b] - ra).to(DEV)
        ws = ops.loss_fwd_bwd(d["logits"][a:b], g["target"][a:b], g["mask"][a:b], g["old"][a:b], sub_row,
                              g["adv_row"][ra:rb], sub_off, row_weight=w[ra:rb],
                              **dict(kw, ref_logp=g["ref"][a:b]))
        assert torch.equal(ws["dlogits"], full_dz[a:b])
        objs += ops.stats_to_dicts(ws["chunk_stats"])[0]["obj_sum"]
    assert objs == pytest.approx(full_obj, rel=1e-12)


def test_terms_off_leave_the_plain_path_bit_identical():
    d = make_chunk(64, 1000, torch.bfloat16, seed=11, n_rows=6)
    d = _with_ref(d, 11)
    g = d["g"]
    args = (d["logits"], g["target"], g["mask"], g["old"], g["tok_row"], g["adv_row"], g["row_off"])
    plain = ops.loss_fwd_bwd(*args, scale=0.01)
    ones = torch.ones(6, dtype=torch.float32, device=DEV)
    same = ops.loss_fwd_bwd(*args, scale=0.01, row_weight=ones, ref_logp=g["ref"], ent_coef=0.0, kl_coef=0.0)
    assert torch.equal(plain["dlogits"], same["dlogits"])
    assert torch.equal(plain["loss_tok"], same["loss_tok"])
    st = ops.stats_to_dicts(same["chunk_stats"])[0]
    assert st["kl_sum"] != 0.0     # the KL is still reported as a metric


def test_term_argument_errors():
    d = make_chunk(8, 64, seed=12)
    g = d["g"]
    args = (d["logits"], g["target"], g["mask"], g["old"], g["tok_row"], g["adv_row"], g["row_off"])
    with pytest.raises(ops.GrpoError) as e:
        ops.loss_fwd_bwd(*args, kl_coef=0.1)                       # KL weight without a reference
    assert e.value.kind == "EINVAL"
    with pytest.raises(ops.GrpoError):
        ops.loss_fwd_bwd(*args, ref_logp=g["old"], kl_type=7)
    with pytest.raises(ops.GrpoError):
        ops.loss_fwd_bwd(*args, ent_coef=float("nan"))
    with pytest.raises(ops.GrpoError):
        ops.row_weights(g["mask"], g["row_off"], 5, ops.count_rows(g["mask"], g["row_off"]))


def _lm_case(n, H, V, seed):
    gcpu = torch.Generator(device="cpu").manual_seed(seed)
    h = (torch.randn((n, H), generator=gcpu)).to(torch.bfloat16)
    W = (torch.randn((V, H), generator=gcpu) * 0.05).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    target = rng.integers(0, V, n).astype(np.int32)
    mask = (rng.random(n) > 0.2).astype(np.uint8)
    row_off = np.array([0, n // 3, n // 3 + 5, n], np.int64)
    tok_row = np.repeat(np.arange(3, dtype=np.int32), np.diff(row_off))
    adv = rng.normal(0, 1, 3).astype(np.float32)
    h64, W64 = h.double().numpy(), W.double().numpy()
    lp = oracle.logprob_fwd(h64 @ W64.T, target, np.ones(n, np.uint8))["logp"]
    old = (lp + rng.normal(0, 0.3, n)).astype(np.float32)
    ref = (lp + rng.normal(0, 0.3, n)).astype(np.float32)
    G = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    return dict(h=h.to(DEV), W=W.to(DEV), h64=h64, W64=W64, target=target, mask=mask, old=old, ref=ref, adv=adv,
                tok_row=tok_row, row_off=row_off,
                g={k: G(v) for k, v in (("target", target), ("mask", mask), ("old", old), ("ref", ref),
                                        ("adv", adv), ("tok_row", tok_row), ("row_off", row_off))})


@pytest.mark.parametrize("n,H,V", [(70, 64, 1000), (260, 128, 4104)])
def test_lmhead_terms_match_oracle(n, H, V):
    c = _lm_case(n, H, V, seed=n + V)
    g = c["g"]
    B = ops.count_rows(g["mask"], g["row_off"])
    w = ops.row_weights(g["mask"], g["row_off"], AGG_SEQ_MEAN_TOKEN_MEAN, B)
    dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    Wt = ops.transpose_bf16(c["W"])
    ws = ops.lmhead_fwd_bwd(c["h"], c["W"], Wt, g["target"], g["mask"], g["old"], g["tok_row"], g["adv"],
                            g["row_off"], dW, scale=1.0, row_weight=w, ref_logp=g["ref"], ent_coef=0.02,
                            kl_coef=0.1, kl_type=KL_K3)
    torch.cuda.synchronize()
    off = c["row_off"].tolist()
    w_tok = np.repeat(oracle.row_weights(c["mask"], off, AGG_SEQ_MEAN_TOKEN_MEAN, oracle.count_rows(c["mask"], off)),
                      np.diff(off))
    ref, _ = oracle_lmhead_at_kernel_clip(ws["tok_flags"].cpu().numpy(), c["h64"], c["W64"], c["target"],
                                          c["mask"], c["old"], c["adv"].astype(np.float64)[c["tok_row"]], 1.0,
                                          w_tok=w_tok, ent_coef=0.02, kl_coef=0.1,
                                          ref_logp=c["ref"].astype(np.float64), kl_type=KL_K3)
    valid = ref["valid"]
    assert np.max(np.abs(to_f64(ws["logp"])[valid] - ref["logp"][valid])) <= 1e-4
    assert np.max(np.abs(to_f64(ws["kl_tok"])[valid] - ref["kl"][valid])) <= 2e-4
    assert rel_l2(to_f64(ws["dh"]), ref["dh"]) <= 4e-3, rel_l2(to_f64(ws["dh"]), ref["dh"])
    assert rel_l2(to_f64(dW), ref["dW"]) <= 4e-3, rel_l2(to_f64(dW), ref["dW"])
    ch = ops.stats_to_dicts(ws["chunk_stats"])[0]
    cw = oracle.chunk_stats(ref, off)
    assert abs(ch["obj_sum"] - cw["obj_sum"]) <= 1e-4 * float(np.sum(np.abs(ref["obj"]))) + 1e-9
