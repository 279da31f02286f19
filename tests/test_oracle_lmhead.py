"""Pins of the oracle's LM-head variant: finite differences of the loss with
respect to h and W, and the column-sum identity of dW."""

import numpy as np
import pytest

import oracle


def _case(seed=0, n=40, H=32, V=64):
    rng = np.random.default_rng(seed)
    h = rng.normal(0, 1, (n, H))
    W = rng.normal(0, 0.3, (V, H))
    y = rng.integers(0, V, n)
    mask = (rng.random(n) > 0.25).astype(np.uint8)
    adv = rng.normal(0, 1, n)
    lp = oracle.logprob_fwd(h @ W.T, y, np.ones(n, np.uint8))["logp"]
    old = lp + rng.normal(0, 0.4, n)
    return h, W, y, mask, old, adv


def _L(h, W, y, mask, old, adv, scale):
    o = oracle.loss_fwd_bwd(h @ W.T, y, mask, old, adv, scale, want_dz=False)
    return scale * float(np.sum(o["loss_tok"]))


def test_lmhead_gradients_match_finite_differences():
    h, W, y, mask, old, adv = _case()
    scale = 1.0 / int(mask.sum())
    o = oracle.lmhead_fwd_bwd(h, W, y, mask, old, adv, scale)
    rho = np.exp(o["logp"] - old)
    assert not ((np.abs(rho - 0.8) < 1e-4) | (np.abs(rho - 1.2) < 1e-4)).any()
    rng = np.random.default_rng(1)
    eps = 1e-6
    for _ in range(25):
        t, k = int(rng.integers(0, h.shape[0])), int(rng.integers(0, h.shape[1]))
        hp = h.copy(); hp[t, k] += eps
        hm = h.copy(); hm[t, k] -= eps
        fd = (_L(hp, W, y, mask, old, adv, scale) - _L(hm, W, y, mask, old, adv, scale)) / (2 * eps)
        assert o["dh"][t, k] == pytest.approx(fd, abs=1e-8)
    for _ in range(25):
        v, k = int(rng.integers(0, W.shape[0])), int(rng.integers(0, W.shape[1]))
        Wp = W.copy(); Wp[v, k] += eps
        Wm = W.copy(); Wm[v, k] -= eps
        fd = (_L(h, Wp, y, mask, old, adv, scale) - _L(h, Wm, y, mask, old, adv, scale)) / (2 * eps)
        assert o["dW"][v, k] == pytest.approx(fd, abs=1e-8)


def test_lmhead_identities():
    h, W, y, mask, old, adv = _case(3)
    o = oracle.lmhead_fwd_bwd(h, W, y, mask, old, adv, 0.05)
    # sum over the vocabulary of dz is 0 per token, so dW's column sums vanish
    assert np.allclose(o["dW"].sum(axis=0), 0.0, atol=1e-13)
    # masked tokens get no hidden-state gradient
    assert not o["dh"][mask == 0].any()
    # chunk gradients add up to the step gradient
    a = oracle.lmhead_fwd_bwd(h[:17], W, y[:17], mask[:17], old[:17], adv[:17], 0.05)
    b = oracle.lmhead_fwd_bwd(h[17:], W, y[17:], mask[17:], old[17:], adv[17:], 0.05)
    assert np.allclose(a["dW"] + b["dW"], o["dW"], rtol=1e-12, atol=1e-15)
    assert np.allclose(np.concatenate([a["dh"], b["dh"]]), o["dh"], rtol=1e-12, atol=1e-15)
