"""Pins of the oracle's loss arithmetic: closed forms, library routines on
special cases, finite differences, and the pages' identities (chunked ==
un-chunked, token-weighted roll-up, pads and empty batches)."""

import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rounding_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 20000), rng.normal(0, 1e-30, 2000),
                        rng.normal(0, 1e38, 200), [0.0, -0.0, 1.0, -2.5]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_rounding_is_single_rounding_from_float64():
    # 1 + 2^-8 is the midpoint between 1 and 1 + 2^-7: ties go to even (1.0).
    assert oracle.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # A hair above the midpoint must round up; going through float32 first
    # would drop the 2^-40 and round to even instead.
    assert oracle.round_to_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7
    # 1 + 3*2^-8 is a midpoint with an odd lower neighbour: rounds up.
    assert oracle.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # subnormal quantum 2^-133 and overflow to infinity
    assert oracle.round_to_bf16(np.array([2.0 ** -134 * 1.5]))[0] == 2.0 ** -133
    assert oracle.round_to_bf16(np.array([3.5e38]))[0] == np.inf
    assert np.isnan(oracle.round_to_bf16(np.array([np.nan]))[0])


# ---------------------------------------------------------------- one token

@pytest.mark.parametrize("V,c", [(1, 0.0), (7, 3.25), (1024, -11.0), (151936, 2.0)])
def test_constant_row_closed_form(V, c):
    lse, logp, H, p = oracle.token_forward(np.full(V, c), V // 2)
    assert lse == pytest.approx(c + math.log(V), abs=1e-12 * max(1, abs(c) + math.log(V)))
    assert logp == pytest.approx(-math.log(V), abs=1e-11)
    assert H == pytest.approx(math.log(V), abs=1e-10)
    assert np.allclose(p, 1.0 / V, rtol=1e-12)


@pytest.mark.parametrize("V,a,d", [(16, 0.5, 0.25), (1000, -3.0, 0.01), (5000, 2.0, -0.003)])
def test_arithmetic_row_closed_form(V, a, d):
    z = a + d * np.arange(V)
    lse, logp, H, p = oracle.token_forward(z, 3)
    # sum_v e^{a+vd} = e^a (e^{Vd}-1)/(e^d-1)
    want = a + math.log(math.expm1(V * d) / math.expm1(d))
    assert lse == pytest.approx(want, rel=1e-13, abs=1e-12)
    assert logp == pytest.approx(a + 3 * d - want, abs=1e-12)


def test_dominant_logit_entropy_vanishes():
    z = np.zeros(1000)
    z[17] = 200.0
    lse, logp, H, p = oracle.token_forward(z, 17)
    assert logp == pytest.approx(0.0, abs=1e-80)
    assert 0.0 <= H < 1e-80
    assert lse == pytest.approx(200.0)


def test_matches_library_logsumexp_and_entropy():
    rng = np.random.default_rng(1)
    for V in (2, 33, 1024, 65536):
        z = rng.normal(0, 3, V)
        y = int(rng.integers(0, V))
        lse, logp, H, p = oracle.token_forward(z, y)
        assert lse == pytest.approx(scipy.special.logsumexp(z), rel=1e-14)
        assert logp == pytest.approx(z[y] - scipy.special.logsumexp(z), abs=1e-12)
        assert H == pytest.approx(scipy.stats.entropy(scipy.special.softmax(z)), rel=1e-11)


def test_minus_inf_logits_are_dropped():
    z = np.array([1.0, -np.inf, 2.0, -np.inf])
    lse, logp, H, p = oracle.token_forward(z, 2)
    ref = oracle.token_forward(np.array([1.0, 2.0]), 1)
    assert lse == pytest.approx(ref[0]) and logp == pytest.approx(ref[1]) and H == pytest.approx(ref[2])
    assert p[1] == 0.0 and p[3] == 0.0


def test_invalid_target_is_nan():
    assert math.isnan(oracle.token_forward(np.zeros(4), 4)[1])
    assert math.isnan(oracle.token_forward(np.zeros(4), -1)[1])


# ---------------------------------------------------------------- surrogate

@pytest.mark.parametrize("A,rho,loss,g", [
    (1.5, 1.5, -1.2 * 1.5, 0),      # A>0, ratio above the band: clipped, no gradient
    (1.5, 0.5, -0.5 * 1.5, 1),      # A>0, ratio below: unclipped branch is smaller
    (-1.5, 1.5, 1.5 * 1.5, 1),      # A<0, ratio above: unclipped branch is smaller
    (-1.5, 0.5, 0.8 * 1.5, 0),      # A<0, ratio below: clipped, no gradient
    (0.7, 1.1, -1.1 * 0.7, 1),      # inside the band
    (0.7, 1.2, -1.2 * 0.7, 1),      # on the upper edge: gradient kept
    (-0.7, 0.8, 0.8 * 0.7, 1),      # on the lower edge: gradient kept
    (0.0, 3.0, 0.0, 1),             # zero advantage
])
def test_surrogate_quadrants(A, rho, loss, g):
    l, gg, r = oracle.surrogate(math.log(rho), 0.0, A, 0.2, 0.2)
    assert r == pytest.approx(rho, rel=1e-14)
    assert l == pytest.approx(loss, rel=1e-12, abs=1e-15)
    assert gg == g


def test_surrogate_asymmetric_clip():
    l, g, _ = oracle.surrogate(math.log(1.25), 0.0, 1.0, 0.2, 0.28)
    assert g == 1 and l == pytest.approx(-1.25)
    l, g, _ = oracle.surrogate(math.log(1.3), 0.0, 1.0, 0.2, 0.28)
    assert g == 0 and l == pytest.approx(-1.28)


# ---------------------------------------------------------------- gradient

def _chunk(seed, n, V, logit_std=2.0, noise=0.05, masked_frac=0.3):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, logit_std, (n, V))
    y = rng.integers(0, V, n)
    mask = (rng.random(n) > masked_frac).astype(np.uint8)
    adv = rng.normal(0, 1, n)
    lp = oracle.logprob_fwd(z, y, np.ones(n, np.uint8))["logp"]
    old = lp + rng.normal(0, noise, n)
    return z, y, mask, old, adv


def _total_loss(z, y, mask, old, adv, scale):
    o = oracle.loss_fwd_bwd(z, y, mask, old, adv, scale, want_dz=False)
    return scale * float(np.sum(o["loss_tok"]))


def test_gradient_matches_finite_differences():
    # Central differences of L(z) = scale * sum_t l_t(z) in float64, V <= 16,
    # tokens away from the clip edges (N(0, 0.5) log-ratio noise gives clipped
    # tokens in both directions).
    z, y, mask, old, adv = _chunk(7, 24, 13, noise=0.5)
    scale = 1.0 / max(1, int(mask.sum()))
    o = oracle.loss_fwd_bwd(z, y, mask, old, adv, scale)
    rho = np.exp(o["logp"] - old)
    near_edge = (np.abs(rho - 0.8) < 1e-3) | (np.abs(rho - 1.2) < 1e-3)
    assert o["clipped"].sum() >= 3 and (~o["clipped"] & mask.astype(bool)).sum() >= 3
    h = 1e-6
    for t in range(z.shape[0]):
        if near_edge[t]:
            continue
        for v in range(z.shape[1]):
            zp = z.copy(); zp[t, v] += h
            zm = z.copy(); zm[t, v] -= h
            fd = (_total_loss(zp, y, mask, old, adv, scale) - _total_loss(zm, y, mask, old, adv, scale)) / (2 * h)
            assert o["dz"][t, v] == pytest.approx(fd, abs=2e-8)


def test_gradient_row_identities():
    z, y, mask, old, adv = _chunk(8, 40, 50)
    o = oracle.loss_fwd_bwd(z, y, mask, old, adv, 0.01)
    assert np.allclose(o["dz"].sum(axis=1), 0.0, atol=1e-15)          # sum_v dz_v = 0
    for t in range(40):
        if mask[t]:
            p_y = math.exp(o["logp"][t])
            assert o["dz"][t, y[t]] == pytest.approx(o["coef"][t] * (p_y - 1.0), rel=1e-12, abs=1e-18)
        else:
            assert not o["dz"][t].any()
            assert o["loss_tok"][t] == 0 and o["logp"][t] == 0 and o["entropy"][t] == 0


def test_ratio_one_gives_minus_mean_advantage():
    # With old = logp the ratio is exactly 1 and nothing clips: L = -sum_t A_t / N.
    z, y, mask, _, adv = _chunk(9, 64, 31)
    old = oracle.logprob_fwd(z, y, mask)["logp"]
    N = int(mask.sum())
    o = oracle.loss_fwd_bwd(z, y, mask, old, adv, 1.0 / N)
    L = float(np.sum(o["loss_tok"])) / N
    assert L == pytest.approx(-float(np.sum(adv[mask.astype(bool)])) / N, rel=1e-12)
    assert not o["clipped"].any()


def test_empty_batch_is_zero_not_nan():
    z, y, mask, old, adv = _chunk(10, 12, 9)
    mask[:] = 0
    N = oracle.valid_count(mask)
    o = oracle.loss_fwd_bwd(z, y, mask, old, adv, 1.0 / max(N, 1))
    st = oracle.chunk_stats(o, [0, 12])
    assert N == 0 and st["loss_sum"] == 0.0 and st["n_valid"] == 0
    assert not o["dz"].any() and np.isfinite(o["dz"]).all()


def test_chunked_equals_unchunked():
    # [P1] the micro-chunked gradient equals the un-chunked one: the same
    # per-token scale 1/N over the whole step makes dz identical.
    z, y, mask, old, adv = _chunk(11, 96, 40)
    scale = 1.0 / oracle.valid_count(mask)
    full = oracle.loss_fwd_bwd(z, y, mask, old, adv, scale)
    parts = [oracle.loss_fwd_bwd(z[a:a + 24], y[a:a + 24], mask[a:a + 24], old[a:a + 24], adv[a:a + 24], scale)
             for a in range(0, 96, 24)]
    assert np.array_equal(np.concatenate([p["dz"] for p in parts]), full["dz"])
    Ls = sum(float(np.sum(p["loss_tok"])) for p in parts)
    assert Ls == pytest.approx(float(np.sum(full["loss_tok"])), rel=1e-12)


def test_token_weighted_rollup_vs_mean_of_means():
    # [P1] "Metric roll-up": sum(loss_i * denom_i) / sum(denom_i) is the batch
    # loss; the plain mean of chunk means differs on unequal chunks.
    z, y, mask, old, adv = _chunk(12, 60, 20, noise=0.3)
    mask[:30] = 1
    mask[30:] = 0
    mask[30:33] = 1                                  # chunk 2 has 3 valid tokens, chunk 1 has 30
    full = oracle.loss_fwd_bwd(z, y, mask, old, adv, 1.0)
    L = float(np.sum(full["loss_tok"])) / oracle.valid_count(mask)
    c1 = oracle.chunk_stats(oracle.loss_fwd_bwd(z[:30], y[:30], mask[:30], old[:30], adv[:30], 1.0), [0, 30])
    c2 = oracle.chunk_stats(oracle.loss_fwd_bwd(z[30:], y[30:], mask[30:], old[30:], adv[30:], 1.0), [0, 30])
    l1, l2 = c1["loss_sum"] / c1["n_valid"], c2["loss_sum"] / c2["n_valid"]
    rolled = (l1 * c1["n_valid"] + l2 * c2["n_valid"]) / (c1["n_valid"] + c2["n_valid"])
    assert rolled == pytest.approx(L, rel=1e-12)
    assert abs(0.5 * (l1 + l2) - L) > 1e-3


def test_pads_add_nothing():
    # A pad row (copy of a real row, mask 0, advantage 0) leaves loss, N and
    # the real rows' gradient unchanged.
    z, y, mask, old, adv = _chunk(13, 20, 17)
    zz = np.concatenate([z, z[:5]])
    yy = np.concatenate([y, y[:5]])
    mm = np.concatenate([mask, np.zeros(5, np.uint8)])
    oo = np.concatenate([old, old[:5]])
    aa = np.concatenate([adv, np.zeros(5)])
    a = oracle.loss_fwd_bwd(z, y, mask, old, adv, 0.1)
    b = oracle.loss_fwd_bwd(zz, yy, mm, oo, aa, 0.1)
    assert np.array_equal(b["dz"][:20], a["dz"]) and not b["dz"][20:].any()
    assert oracle.valid_count(mm) == oracle.valid_count(mask)
    assert np.sum(b["loss_tok"]) == np.sum(a["loss_tok"])


def test_row_stats_sum_to_chunk_stats():
    z, y, mask, old, adv = _chunk(14, 50, 11, noise=0.4)
    o = oracle.loss_fwd_bwd(z, y, mask, old, adv, 1.0)
    off = [0, 7, 7, 30, 50]
    rows = oracle.row_stats(o, off)
    tot = oracle.chunk_stats(o, off)
    assert tot["n_valid"] == int(mask.sum())
    assert tot["loss_sum"] == pytest.approx(float(np.sum(o["loss_tok"])), rel=1e-13)
    assert rows[1]["n_valid"] == 0 and rows[1]["n_valid_rows"] == 0
    assert tot["n_clipped"] == int(o["clipped"].sum())


def test_nonfinite_flagged():
    z, y, mask, old, adv = _chunk(15, 10, 8)
    mask[:] = 1
    z[3, 2] = np.nan
    y[6] = 8                                        # outside [0, V)
    o = oracle.loss_fwd_bwd(z, y, mask, old, adv, 1.0)
    assert o["nonfinite"][3] and o["nonfinite"][6]
    assert oracle.chunk_stats(o, [0, 10])["n_nonfinite"] == 2
