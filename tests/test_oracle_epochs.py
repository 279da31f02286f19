"""Pins of the oracle's inner-epoch plan and seeded shuffle ([P3] section 1:
epochs and a seeded shuffle of the mini-batch iterator; [P1] "What's not
done", item 2: inner epochs reuse the frozen pi_old): the generator's
published reference outputs, a hand-worked Fisher-Yates run, uniformity of
the shuffle, partition invariants of every epoch, the cache's rewind and the
chunk gather."""

import itertools
import json
import os

import numpy as np
import pytest
import scipy.stats

import oracle
from oracle import CacheError, PlanError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_vectors.json")


def test_splitmix64_reference_outputs():
    for v in json.load(open(GOLDEN))["vectors"]:
        g = oracle.splitmix64_stream(v["seed"])
        want = [int(x, 16) for x in v["outputs_hex"]] if "outputs_hex" in v else v["outputs"]
        assert [next(g) for _ in want] == want


def test_fisher_yates_hand_worked():
    # n = 4, draws 5, 7, 2: i=3 j=5%4=1 -> [0,3,2,1]; i=2 j=7%3=1 -> [0,2,3,1]; i=1 j=2%2=0 -> [2,0,3,1]
    assert oracle.fisher_yates(4, iter([5, 7, 2])) == [2, 0, 3, 1]
    assert oracle.fisher_yates(1, iter([])) == [0]
    assert oracle.fisher_yates(0, iter([])) == []


def test_shuffle_is_uniform():
    # 6 permutations of 3 items from one stream: chi-square against uniform
    g = oracle.splitmix64_stream(99)
    perms = list(itertools.permutations(range(3)))
    counts = np.zeros(6)
    for _ in range(30000):
        counts[perms.index(tuple(oracle.fisher_yates(3, g)))] += 1
    assert scipy.stats.chisquare(counts).pvalue > 1e-4
    # and every position of a 10-item shuffle is uniform over the items
    g = oracle.splitmix64_stream(5)
    pos = np.zeros((10, 10))
    for _ in range(20000):
        for k, x in enumerate(oracle.fisher_yates(10, g)):
            pos[k, x] += 1
    assert scipy.stats.chisquare(pos.ravel()).pvalue > 1e-4


def test_epoch_plan_invariants():
    ep = oracle.plan_epochs(32, 4, 16, 8, 3, True, 7)
    assert (ep["n_mini"], ep["n_micro"], ep["mu"]) == (2, 2, 3)
    assert len(oracle.epoch_train_calls(ep)) == 12
    for e in range(3):
        assert sorted(ep["perm"][e]) == list(range(32))
        rows = [r for i in range(2) for j in range(2) for r in oracle.epoch_chunk_rows(ep, e, i, j)]
        assert rows == ep["perm"][e]                       # the chunks tile the epoch's order
    assert ep["perm"][0] != ep["perm"][1] != ep["perm"][2]  # reshuffled every epoch
    assert oracle.plan_epochs(32, 4, 16, 8, 3, True, 7)["perm"] == ep["perm"]       # seeded
    assert oracle.plan_epochs(32, 4, 16, 8, 3, True, 8)["perm"] != ep["perm"]
    # without the shuffle every epoch is the fixed plan
    fx = oracle.plan_epochs(32, 4, 16, 8, 2, False, 7)
    plan = oracle.plan_fixed(32, 4, 16, 8)
    for e, i, j in oracle.epoch_train_calls(fx):
        a, b = oracle.chunk_rows(plan, i, j)
        assert oracle.epoch_chunk_rows(fx, e, i, j) == list(range(a, b))
    # epoch 0 of a shuffled plan is the first permutation of the seed's stream
    assert ep["perm"][0] == oracle.fisher_yates(32, oracle.splitmix64_stream(7))


def test_epoch_plan_errors():
    with pytest.raises(PlanError) as e:
        oracle.plan_epochs(32, 4, 16, 8, 0, False, 1)
    assert e.value.kind == "EINVAL"
    with pytest.raises(PlanError) as e:
        oracle.plan_epochs(32, 4, 12, 0, 2, True, 1)
    assert e.value.kind == "EDIVISIBLE"
    ep = oracle.plan_epochs(8, 2, 4, 2, 2, True, 1)
    with pytest.raises(PlanError):
        oracle.epoch_chunk_rows(ep, 2, 0, 0)


def test_cache_rewind_replays_each_epoch_in_order():
    rng = np.random.default_rng(0)
    z = rng.normal(size=(12, 5))
    y = rng.integers(0, 5, 12)
    m = np.ones(12, np.uint8)
    c = oracle.OldLogprobCache(3, 12)
    for k in range(3):
        c.record(z[4 * k:4 * k + 4], y[4 * k:4 * k + 4], m[4 * k:4 * k + 4])
    with pytest.raises(CacheError):
        c.rewind()                                     # the first walk is not replayed yet
    first = [c.replay(4) for _ in range(3)]
    c.rewind()
    second = [c.replay(4) for _ in range(3)]
    assert all(np.array_equal(a, b) for a, b in zip(first, second))


def test_shuffled_chunk_sources_and_gather():
    off = [0, 3, 3, 8, 10]                  # rows of 3, 0, 5, 2 tokens
    assert oracle.chunk_token_sources(off, [2, 0]) == [3, 4, 5, 6, 7, 0, 1, 2]
    assert oracle.chunk_token_sources(off, [1, 3]) == [8, 9]
    vals = list(range(100, 110))
    assert oracle.gather(vals, oracle.chunk_token_sources(off, [3, 2, 1, 0])) == \
        [108, 109, 103, 104, 105, 106, 107, 100, 101, 102]
    # gathering every row once, in any order, and scattering back restores the batch
    order = [2, 3, 0, 1]
    src = oracle.chunk_token_sources(off, order)
    g = oracle.gather(vals, src)
    back = [None] * 10
    for k, s in enumerate(src):
        back[s] = g[k]
    assert back == vals
