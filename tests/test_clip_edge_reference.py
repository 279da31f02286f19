"""The GPU tests' reference at the kernel's clip decision (gpu_common's
old_at_kernel_clip / oracle_lmhead_at_kernel_clip), on the CPU: a token whose
ratio sits on a clip bound takes the decision the kernel's flags give, every
other token keeps the oracle's result bit for bit, and a decision that differs
away from an edge is refused."""

import numpy as np
import pytest

import oracle
from gpu_common import oracle_lmhead_at_kernel_clip


def _case(seed=0, n=12, H=16, V=40):
    rng = np.random.default_rng(seed)
    h = rng.normal(0, 1, (n, H))
    W = rng.normal(0, 0.2, (V, H))
    target = rng.integers(0, V, n).astype(np.int32)
    mask = np.ones(n, np.uint8)
    mask[5] = 0
    adv = rng.normal(0, 1, n)
    adv[2], adv[7] = 0.8, -0.6
    lp = oracle.logprob_fwd(h @ W.T, target, mask)["logp"]
    old = lp + rng.normal(0, 0.05, n)
    # token 2 (A > 0) just inside the upper bound, token 7 (A < 0) just past the lower one
    old[2] = lp[2] - np.log(1.2 * (1 - 1e-5))
    old[7] = lp[7] - np.log(0.8 * (1 - 1e-5))
    return h, W, target, mask, adv, old


def _flags(ref):
    return (ref["valid"].astype(np.uint8) | ((ref["clipped"] & ref["valid"]).astype(np.uint8) << 1))


def test_agreeing_decisions_leave_the_oracle_as_it_is():
    h, W, target, mask, adv, old = _case()
    want = oracle.lmhead_fwd_bwd(h, W, target, mask, old, adv, 0.1)
    got, moved = oracle_lmhead_at_kernel_clip(_flags(want), h, W, target, mask, old, adv, 0.1)
    assert moved == 0
    for k in ("dh", "dW", "dz", "loss_tok", "clipped"):
        assert np.array_equal(got[k], want[k]), k


def test_edge_tokens_take_the_kernel_decision():
    h, W, target, mask, adv, old = _case()
    base = oracle.lmhead_fwd_bwd(h, W, target, mask, old, adv, 0.1)
    assert not base["clipped"][2] and base["clipped"][7]
    flags = _flags(base)
    flags[2] |= 2               # the kernel clipped token 2 ...
    flags[7] &= ~np.uint8(2)    # ... and kept token 7
    got, moved = oracle_lmhead_at_kernel_clip(flags, h, W, target, mask, old, adv, 0.1)
    assert moved == 2
    assert got["clipped"][2] and not got["clipped"][7]
    # token 2 clipped: no gradient; token 7 kept: coef = s A rho with rho on the bound
    assert not got["dz"][2].any() and not got["dh"][2].any()
    assert np.isclose(got["coef"][7], 0.1 * adv[7] * 0.8, rtol=1e-8)
    # the others are unchanged, and dW is the sum over tokens of the new rows
    keep = np.ones(len(old), bool)
    keep[[2, 7]] = False
    assert np.array_equal(got["dz"][keep], base["dz"][keep])
    assert np.allclose(got["dW"], got["dz"].T @ h, rtol=0, atol=1e-12)
    # the loss is continuous across the edge
    assert np.allclose(got["loss_tok"], base["loss_tok"], rtol=2e-5, atol=0)


def test_a_decision_that_differs_away_from_an_edge_fails():
    h, W, target, mask, adv, old = _case()
    base = oracle.lmhead_fwd_bwd(h, W, target, mask, old, adv, 0.1)
    flags = _flags(base)
    t = next(i for i in range(len(old)) if i not in (2, 5, 7) and adv[i] != 0
             and abs(np.exp(base["logp"][i] - old[i]) - 1) < 0.1)
    flags[t] ^= 2
    with pytest.raises(AssertionError, match="away from an edge"):
        oracle_lmhead_at_kernel_clip(flags, h, W, target, mask, old, adv, 0.1)
