"""Pins of the oracle's ahead-pass gate, old-log-prob cache and determinism
probe ([P1] "pi_old must be frozen across the window -- the ahead pass"):
the gate's truth table, pairing by call order, the strict probe gate, and
the page's central claim simulated end to end -- with pi_old recomputed the
ratio is 1 and nothing clips at n_mini > 1; with the cache the ratio departs
from 1 and the clip binds."""

import numpy as np
import pytest

import oracle
from oracle import CacheError


def test_gate_truth_table():
    # n_mini > 1 AND not rollout log-probs AND the objective consumes pi_old
    assert oracle.needs_ahead_pass(2, False, True)
    assert oracle.needs_ahead_pass(32, False, True)
    assert not oracle.needs_ahead_pass(1, False, True)        # n_mini = 1 skips it entirely
    assert not oracle.needs_ahead_pass(4, True, True)         # rollout log-probs: the cache is never consulted
    assert not oracle.needs_ahead_pass(4, False, False)       # an objective without a ratio


def _batch(seed, n_rows=8, T=6, V=11):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 1.5, (n_rows * T, V))
    y = rng.integers(0, V, n_rows * T)
    mask = (rng.random(n_rows * T) > 0.2).astype(np.uint8)
    return z, y, mask, T


def test_records_pair_with_training_calls_by_order():
    z, y, mask, T = _batch(0)
    plan = oracle.plan_fixed(8, 2, 4, 2)              # 2 mini x 2 micro
    calls = oracle.train_calls(plan)
    cache = oracle.OldLogprobCache(len(calls), capacity=z.shape[0])
    for i, j in calls:
        a, e = oracle.chunk_rows(plan, i, j)
        cache.record(z[a * T:e * T], y[a * T:e * T], mask[a * T:e * T])
    for i, j in calls:
        a, e = oracle.chunk_rows(plan, i, j)
        got = cache.replay((e - a) * T)
        want = oracle.logprob_fwd(z[a * T:e * T], y[a * T:e * T], mask[a * T:e * T])["logp"].astype(np.float32)
        assert np.array_equal(got, want)
    cache.reset()
    assert cache.used == 0 and cache.replayed == 0


def test_cache_misuse_is_an_error():
    z, y, mask, T = _batch(1)
    c = oracle.OldLogprobCache(2, capacity=3 * T)
    with pytest.raises(CacheError) as e:
        c.replay(T)                                    # nothing recorded yet
    assert e.value.kind == "ESTATE"
    c.record(z[:T], y[:T], mask[:T])
    with pytest.raises(CacheError) as e:
        c.record(z[:3 * T], y[:3 * T], mask[:3 * T])   # T + 3T tokens > capacity 3T
    assert e.value.kind == "ECAPACITY"
    c.record(z[T:2 * T], y[T:2 * T], mask[T:2 * T])
    with pytest.raises(CacheError) as e:
        c.record(z[:T], y[:T], mask[:T])               # the walk has two calls
    assert e.value.kind == "ESTATE"
    with pytest.raises(CacheError) as e:
        c.replay(T + 1)                                # walks diverged
    assert e.value.kind == "EINVAL"
    c.replay(T)
    with pytest.raises(CacheError) as e:
        c.record(z[:T], y[:T], mask[:T])               # record after replay began
    assert e.value.kind == "ESTATE"


def test_probe_strict_gate_and_fraction_gate():
    rec = np.linspace(-3.0, -1.0, 20).astype(np.float32)
    mask = np.ones(20, np.uint8)
    assert oracle.probe_compare(rec, rec, mask, 0.05) == (20, 0, 0.0)
    moved = rec.copy()
    moved[7] += 0.0625                                  # past 0.05 nats: strict gate fails
    n_valid, n_moved, mx = oracle.probe_compare(rec, moved, mask, oracle.PROBE_STRICT_BOUND)
    assert (n_valid, n_moved) == (20, 1) and mx == pytest.approx(0.0625, abs=1e-6)
    assert oracle.Probe().finish(n_valid, n_moved) is False
    small = rec.copy()
    small[7] += 0.03125                                 # within the bound
    assert oracle.Probe().finish(*oracle.probe_compare(rec, small, mask, 0.05)[:2]) is True
    # a declared tolerance: 10 % of tokens may move
    p = oracle.Probe(bound=0.05, max_fraction=0.1)
    two = rec.copy()
    two[[1, 2]] += 1.0
    assert p.finish(*oracle.probe_compare(rec, two, mask, 0.05)[:2]) is True
    three = rec.copy()
    three[[1, 2, 3]] += 1.0
    assert oracle.Probe(0.05, 0.1).finish(*oracle.probe_compare(rec, three, mask, 0.05)[:2]) is False
    # masked tokens are ignored; a non-finite value counts as moved
    m2 = mask.copy()
    m2[7] = 0
    assert oracle.probe_compare(rec, moved, m2, 0.05)[:2] == (19, 0)
    nan = rec.copy()
    nan[0] = np.nan
    assert oracle.probe_compare(rec, nan, mask, 0.05)[1] == 1
    assert oracle.probe_compare(rec, nan, mask, 0.05)[2] == float("inf")


def test_probe_runs_once_per_run():
    p = oracle.Probe()
    assert p.due()
    p.finish(10, 0)
    assert not p.due()
    with pytest.raises(CacheError) as e:
        p.finish(10, 0)
    assert e.value.kind == "ESTATE"


def test_frozen_pi_old_makes_the_clip_bind():
    # Two mini-batches of one collected batch.  Between them the policy takes
    # an optimizer step, emulated by a logit drift.  pi_old recomputed from
    # the current policy gives ratio 1 and no clipping in mini-batch 1; the
    # cached ahead pass keeps pi_old at the rollout policy, so the ratio
    # departs from 1 and the clip binds.
    rng = np.random.default_rng(5)
    n_rows, T, V = 8, 16, 13
    z0 = rng.normal(0, 1.5, (n_rows * T, V))
    y = rng.integers(0, V, n_rows * T)
    mask = np.ones(n_rows * T, np.uint8)
    adv = np.repeat(np.where(np.arange(n_rows) % 2 == 0, 1.0, -1.0), T)
    plan = oracle.plan_fixed(n_rows, 2, 4, 4)          # n_mini = 2, n_micro = 1
    assert oracle.needs_ahead_pass(plan[0], False, True)
    calls = oracle.train_calls(plan)
    cache = oracle.OldLogprobCache(len(calls), n_rows * T)
    for i, j in calls:
        a, e = oracle.chunk_rows(plan, i, j)
        cache.record(z0[a * T:e * T], y[a * T:e * T], mask[a * T:e * T])
    z1 = z0 + rng.normal(0, 0.6, z0.shape)              # the policy after mini-batch 0's step
    for i, j in calls:
        a, e = oracle.chunk_rows(plan, i, j)
        sl = slice(a * T, e * T)
        z = z0[sl] if i == 0 else z1[sl]
        frozen = cache.replay(e * T - a * T).astype(np.float64)
        recomputed = oracle.logprob_fwd(z, y[sl], mask[sl])["logp"]
        with_cache = oracle.loss_fwd_bwd(z, y[sl], mask[sl], frozen, adv[sl], 1.0)
        without = oracle.loss_fwd_bwd(z, y[sl], mask[sl], recomputed, adv[sl], 1.0)
        rho_c = np.exp(with_cache["logp"] - frozen)
        assert not without["clipped"].any()
        assert np.allclose(np.exp(without["logp"] - recomputed), 1.0, rtol=0, atol=1e-12)
        if i == 0:
            # nothing has moved yet: the record is the current policy
            assert np.allclose(rho_c, 1.0, rtol=0, atol=1e-6) and not with_cache["clipped"].any()
        else:
            assert np.max(np.abs(rho_c - 1.0)) > 0.2
            assert with_cache["clipped"].sum() >= 5
