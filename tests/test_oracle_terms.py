"""Pins of the oracle's aggregation modes, entropy bonus and KL term
(CPU only): hand-worked aggregation values, identities between the modes,
closed forms of the entropy and KL derivatives, and central finite
differences of the aggregated objective in float64."""

import math

import numpy as np
import pytest

import oracle
from oracle import AGG_SEQ_MEAN_TOKEN_MEAN as SMTM, AGG_SEQ_MEAN_TOKEN_SUM as SMTS, AGG_TOKEN_MEAN as TM


# ---------------------------------------------------------------- aggregation

def test_agg_modes_hand_worked():
    # [P3] section 5 names token-mean (global token count) and the seq-level
    # modes (global batch size).  Rows: r0 = (1, 2, masked 9, 3), r1 = (4),
    # r2 = a masked pad row.  N = 4 valid tokens, B = 2 rows with a valid token.
    l = [1.0, 2.0, 9.0, 3.0, 4.0, 7.0, 7.0]
    mask = [1, 1, 0, 1, 1, 0, 0]
    off = [0, 4, 5, 7]
    assert oracle.row_valid_counts(mask, off) == [3, 1, 0]
    assert oracle.count_rows(mask, off) == 2
    assert oracle.agg_loss(l, mask, off, TM, 4, 2) == pytest.approx(10 / 4)        # (1+2+3+4)/4
    assert oracle.agg_loss(l, mask, off, SMTS, 4, 2) == pytest.approx((6 + 4) / 2)
    assert oracle.agg_loss(l, mask, off, SMTM, 4, 2) == pytest.approx((6 / 3 + 4 / 1) / 2)
    assert oracle.row_weights(mask, off, SMTM, 2) == [1 / 6, 1 / 2, 0.0]
    assert oracle.row_weights(mask, off, SMTS, 2) == [0.5, 0.5, 0.5]
    assert oracle.row_weights(mask, off, TM, 2) == [1.0, 1.0, 1.0]


def test_agg_modes_identities():
    rng = np.random.default_rng(0)
    # equal valid lengths: seq-mean-token-mean == token-mean, seq-mean-token-sum == L * token-mean
    R, L = 6, 5
    l = rng.normal(size=R * L)
    mask = np.ones(R * L, np.uint8)
    off = list(range(0, R * L + 1, L))
    tm = oracle.agg_loss(l, mask, off, TM, R * L, R)
    assert oracle.agg_loss(l, mask, off, SMTM, R * L, R) == pytest.approx(tm, rel=1e-14)
    assert oracle.agg_loss(l, mask, off, SMTS, R * L, R) == pytest.approx(L * tm, rel=1e-14)
    # empty mini-batch: every mode gives 0, not NaN
    z = np.zeros(R * L, np.uint8)
    for mode in (TM, SMTS, SMTM):
        assert oracle.agg_loss(l, z, off, mode, 0, 0) == 0.0


def test_agg_of_ones_counts():
    # the aggregate of l_t = 1: token-mean 1, seq-mean-token-sum N/B, seq-mean-token-mean 1
    rng = np.random.default_rng(1)
    lens = rng.integers(1, 9, 7)
    off = [0] + np.cumsum(lens).tolist()
    mask = (rng.random(off[-1]) < 0.7).astype(np.uint8)
    N, B = int(mask.sum()), oracle.count_rows(mask, off)
    ones = np.ones(off[-1])
    assert oracle.agg_loss(ones, mask, off, TM, N, B) == pytest.approx(1.0)
    assert oracle.agg_loss(ones, mask, off, SMTS, N, B) == pytest.approx(N / B)
    assert oracle.agg_loss(ones, mask, off, SMTM, N, B) == pytest.approx(1.0)


# ---------------------------------------------------------------- KL estimators

@pytest.mark.parametrize("d", [-1.3, -0.2, 0.0, 0.05, 0.7])
def test_kl_estimators_closed_forms(d):
    logp, ref = -2.0, -2.0 + d
    k1, g1 = oracle.kl_term(logp, ref, oracle.KL_K1)
    k2, g2 = oracle.kl_term(logp, ref, oracle.KL_K2)
    k3, g3 = oracle.kl_term(logp, ref, oracle.KL_K3)
    assert k1 == pytest.approx(logp - ref) and g1 == 1.0
    assert k2 == pytest.approx(0.5 * (logp - ref) ** 2) and g2 == pytest.approx(logp - ref)
    assert k3 >= 0.0                                       # e^d >= 1 + d
    assert k3 == pytest.approx(math.exp(d) - d - 1.0, abs=1e-15)
    # derivatives by central differences in logp
    h = 1e-6
    for kind, g in ((oracle.KL_K1, g1), (oracle.KL_K2, g2), (oracle.KL_K3, g3)):
        fd = (oracle.kl_term(logp + h, ref, kind)[0] - oracle.kl_term(logp - h, ref, kind)[0]) / (2 * h)
        assert g == pytest.approx(fd, abs=1e-8)
    if d == 0.0:
        assert k3 == 0.0 and g3 == 0.0 and k2 == 0.0


# ---------------------------------------------------------------- gradients

def _chunk(seed, n, V, noise=0.5):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 2.0, (n, V))
    y = rng.integers(0, V, n)
    mask = (rng.random(n) > 0.25).astype(np.uint8)
    adv = rng.normal(0, 1, n)
    lp = oracle.logprob_fwd(z, y, np.ones(n, np.uint8))["logp"]
    old = lp + rng.normal(0, noise, n)
    ref = lp + rng.normal(0, 0.3, n)
    return z, y, mask, old, adv, ref


def test_entropy_bonus_two_logit_closed_form():
    # V = 2, z = (a, 0), A = 0, no KL: the only gradient is the bonus'.
    # H(a) = log(1 + e^a) - a sigma(a), dH/da = -a sigma(a) (1 - sigma(a)), so
    # d(-beta s H)/dz_0 = beta s a p (1 - p) and dz_1 = -dz_0.
    beta, s = 0.3, 0.25
    for a in (-2.0, -0.4, 0.0, 1.1, 3.0):
        z = np.array([[a, 0.0]])
        o = oracle.loss_fwd_bwd(z, [1], [1], [-0.7], [0.0], s, ent_coef=beta)
        p = 1.0 / (1.0 + math.exp(-a))
        assert o["entropy"][0] == pytest.approx(math.log(1 + math.exp(a)) - a * p, rel=1e-13)
        assert o["dz"][0, 0] == pytest.approx(beta * s * a * p * (1 - p), abs=1e-15)
        assert o["dz"][0, 1] == pytest.approx(-beta * s * a * p * (1 - p), abs=1e-15)
        assert o["obj"][0] == pytest.approx(-s * beta * o["entropy"][0], rel=1e-13)


def test_entropy_bonus_vanishes_on_uniform_logits():
    # uniform logits maximise H: its gradient is 0, so the bonus leaves dz alone
    z = np.full((3, 7), 0.4)
    args = ([1, 2, 3], [1, 1, 1], [-2.0, -1.9, -1.95], [0.5, -1.0, 2.0], 0.1)
    a = oracle.loss_fwd_bwd(z, *args)
    b = oracle.loss_fwd_bwd(z, *args, ent_coef=0.7)
    assert np.allclose(a["dz"], b["dz"], atol=1e-16, rtol=0)


def test_kl_k1_gradient_closed_form():
    # A = 0, k1: the objective is kappa s (logp - ref), so dz = -kappa s (p - onehot)
    rng = np.random.default_rng(3)
    z = rng.normal(size=(4, 9))
    y = [0, 3, 8, 5]
    kappa, s = 0.05, 0.5
    o = oracle.loss_fwd_bwd(z, y, [1] * 4, [-2.0] * 4, [0.0] * 4, s, kl_coef=kappa,
                            ref_logp=[-2.1] * 4, kl_type=oracle.KL_K1)
    for t in range(4):
        p = np.exp(z[t] - (np.max(z[t]) + math.log(np.sum(np.exp(z[t] - np.max(z[t]))))))
        want = -kappa * s * p
        want[y[t]] += kappa * s
        assert np.allclose(o["dz"][t], want, atol=1e-16, rtol=1e-13)


def _objective(z, y, mask, old, adv, ref, scale, w_tok, ent, kap, kind):
    o = oracle.loss_fwd_bwd(z, y, mask, old, adv, scale, want_dz=False, w_tok=w_tok, ent_coef=ent,
                            kl_coef=kap, ref_logp=ref, kl_type=kind)
    return float(np.sum(o["obj"]))


@pytest.mark.parametrize("ent,kap,kind", [(0.3, 0.0, oracle.KL_K3), (0.0, 0.2, oracle.KL_K3),
                                          (0.1, 0.4, oracle.KL_K2), (0.2, 0.1, oracle.KL_K1)])
def test_terms_gradient_matches_finite_differences(ent, kap, kind):
    z, y, mask, old, adv, ref = _chunk(5, 16, 11)
    off = [0, 5, 9, 16]
    w = oracle.row_weights(mask, off, SMTM, oracle.count_rows(mask, off))
    w_tok = np.repeat(w, np.diff(off))
    o = oracle.loss_fwd_bwd(z, y, mask, old, adv, 1.0, w_tok=w_tok, ent_coef=ent, kl_coef=kap,
                            ref_logp=ref, kl_type=kind)
    rho = np.exp(o["logp"] - old)
    near_edge = (np.abs(rho - 0.8) < 1e-3) | (np.abs(rho - 1.2) < 1e-3)
    h = 1e-6
    for t in range(z.shape[0]):
        if near_edge[t]:
            continue
        for v in range(z.shape[1]):
            zp = z.copy(); zp[t, v] += h
            zm = z.copy(); zm[t, v] -= h
            fd = (_objective(zp, y, mask, old, adv, ref, 1.0, w_tok, ent, kap, kind)
                  - _objective(zm, y, mask, old, adv, ref, 1.0, w_tok, ent, kap, kind)) / (2 * h)
            assert o["dz"][t, v] == pytest.approx(fd, abs=3e-8)


@pytest.mark.parametrize("mode", [TM, SMTS, SMTM])
def test_row_weighted_gradient_is_the_aggregate_gradient(mode):
    # d agg_loss(l(z)) / dz (finite differences, agg_loss by its definition)
    # equals dz from loss_fwd_bwd with the mode's row weights.
    z, y, mask, old, adv, _ = _chunk(6, 14, 7)
    off = [0, 3, 4, 10, 14]
    N, B = int(mask.sum()), oracle.count_rows(mask, off)
    w_tok = np.repeat(oracle.row_weights(mask, off, mode, B), np.diff(off))
    scale = 1.0 / max(N, 1) if mode == TM else 1.0
    o = oracle.loss_fwd_bwd(z, y, mask, old, adv, scale, w_tok=w_tok)

    def J(zz):
        lt = oracle.loss_fwd_bwd(zz, y, mask, old, adv, 1.0, want_dz=False)["loss_tok"]
        return oracle.agg_loss(lt, mask, off, mode, N, B)

    rho = np.exp(o["logp"] - old)
    near_edge = (np.abs(rho - 0.8) < 1e-3) | (np.abs(rho - 1.2) < 1e-3)
    h = 1e-6
    for t in range(z.shape[0]):
        if near_edge[t]:
            continue
        for v in range(z.shape[1]):
            zp = z.copy(); zp[t, v] += h
            zm = z.copy(); zm[t, v] -= h
            assert o["dz"][t, v] == pytest.approx((J(zp) - J(zm)) / (2 * h), abs=3e-8)
    # and the chunk's objective share is the aggregate itself
    st = oracle.chunk_stats(o, off)
    assert st["obj_sum"] == pytest.approx(J(z), rel=1e-12, abs=1e-15)


def test_seq_mode_objective_is_chunk_invariant():
    # global B and per-row L_r make the chunk shares add up to the batch value
    z, y, mask, old, adv, ref = _chunk(7, 40, 6)
    off = [0, 7, 12, 20, 26, 33, 40]
    B = oracle.count_rows(mask, off)
    w_tok = np.repeat(oracle.row_weights(mask, off, SMTM, B), np.diff(off))
    full = oracle.chunk_stats(oracle.loss_fwd_bwd(z, y, mask, old, adv, 1.0, w_tok=w_tok, ent_coef=0.1,
                                                  kl_coef=0.2, ref_logp=ref), off)
    parts = 0.0
    for a, b in ((0, 3), (3, 6)):
        lo, hi = off[a], off[b]
        o = oracle.loss_fwd_bwd(z[lo:hi], y[lo:hi], mask[lo:hi], old[lo:hi], adv[lo:hi], 1.0, w_tok=w_tok[lo:hi],
                                ent_coef=0.1, kl_coef=0.2, ref_logp=ref[lo:hi])
        parts += oracle.chunk_stats(o, [x - lo for x in off[a:b + 1]])["obj_sum"]
    assert parts == pytest.approx(full["obj_sum"], rel=1e-13)


def test_accumulator_sums_kl_and_objective_and_flags_nonfinite_objective():
    acc = oracle.Accumulator(2)
    base = {"loss_sum": 1.0, "entropy_sum": 2.0, "kl_sum": 0.5, "obj_sum": 0.25, "n_valid": 4,
            "n_clipped": 0, "n_nonfinite": 0, "n_valid_rows": 1}
    assert acc.add(base) == oracle.ACC_OK and acc.add(base) == oracle.ACC_OK
    r = acc.finalize()
    assert r["kl"] == pytest.approx(1.0 / 8) and r["obj_sum"] == pytest.approx(0.5)
    bad = dict(base, obj_sum=float("inf"))
    assert acc.add(bad) == oracle.ACC_NONFINITE and acc.add(base) == oracle.ACC_SKIPPED
