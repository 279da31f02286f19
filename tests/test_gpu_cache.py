"""GPU side of the frozen pi_old machinery ([P1] "pi_old must be frozen
across the window -- the ahead pass"): the old-log-prob cache through the C
ABI (records are the ahead pass, paired by call order), the determinism
probe's compare against the oracle, and the page's claim end to end on the
fused loss kernel -- at n_mini > 1 the cache makes the clip bind, pi_old
recomputed from the drifting policy never does."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import DEV, to_f64, tol_logp
from grpo_token_level_amd import ops

pytestmark = pytest.mark.gpu


def _batch(n_rows, T, V, dtype, seed, std=1.5):
    g = torch.Generator(device="cpu").manual_seed(seed)
    z = (torch.randn((n_rows * T, V), generator=g) * std).to(dtype)
    rng = np.random.default_rng(seed)
    y = rng.integers(0, V, n_rows * T).astype(np.int32)
    mask = (rng.random(n_rows * T) > 0.2).astype(np.uint8)
    return z, y, mask


def test_cache_records_are_the_ahead_pass_and_pair_by_order():
    n_rows, T, V = 8, 64, 1000
    for dtype in (torch.float32, torch.bfloat16):
        z, y, mask = _batch(n_rows, T, V, dtype, seed=1)
        zg, yg, mg = z.to(DEV), torch.from_numpy(y).to(DEV), torch.from_numpy(mask).to(DEV)
        n_mini, n_micro, mini_rows, micro_rows = ops.plan_fixed(n_rows, 2, 4, 2)
        assert ops.needs_ahead_pass(n_mini)
        calls = [(i, j) for i in range(n_mini) for j in range(n_micro)]
        cache = ops.OldLogprobCache(len(calls), torch.empty(n_rows * T, dtype=torch.float32, device=DEV))
        recs = []
        for i, j in calls:
            a, e = ops.plan_chunk(n_rows, mini_rows, micro_rows, i, j)
            recs.append(cache.record(zg[a * T:e * T], yg[a * T:e * T], mg[a * T:e * T]).clone())
        assert cache.recorded == len(calls)
        for k, (i, j) in enumerate(calls):
            a, e = ops.plan_chunk(n_rows, mini_rows, micro_rows, i, j)
            got = cache.replay((e - a) * T)
            assert torch.equal(got, recs[k])
            lp, _, _ = ops.logprob_fwd(zg[a * T:e * T], yg[a * T:e * T], mg[a * T:e * T])
            assert torch.equal(got, lp)                      # the record is the ahead pass itself
            ref = oracle.logprob_fwd(z[a * T:e * T].double().numpy(), y[a * T:e * T], mask[a * T:e * T])["logp"]
            assert np.max(np.abs(to_f64(got) - ref)) <= tol_logp(dtype)
        with pytest.raises(ops.GrpoError) as err:
            cache.replay(micro_rows * T)                     # the walk has no fifth call
        assert err.value.kind == "ESTATE"


def test_cache_capacity_and_divergence_errors():
    z, y, mask = _batch(4, 32, 256, torch.float32, seed=2)
    zg, yg, mg = z.to(DEV), torch.from_numpy(y).to(DEV), torch.from_numpy(mask).to(DEV)
    cache = ops.OldLogprobCache(2, torch.empty(100, dtype=torch.float32, device=DEV))
    cache.record(zg[:64], yg[:64], mg[:64])
    with pytest.raises(ops.GrpoError) as err:
        cache.record(zg[64:128], yg[64:128], mg[64:128])    # 128 > 100 floats
    assert err.value.kind == "ECAPACITY"
    with pytest.raises(ops.GrpoError) as err:
        cache.replay(63)
    assert err.value.kind == "EINVAL"


def test_probe_compare_matches_oracle():
    rng = np.random.default_rng(3)
    n = 5000
    a = rng.normal(-3, 1, n).astype(np.float32)
    b = a.copy()
    idx = rng.choice(n, 40, replace=False)
    b[idx] += rng.choice([-1, 1], 40) * rng.uniform(0.0, 0.2, 40).astype(np.float32)
    b[idx[:3]] = np.nan
    b[idx[3]] = np.inf
    mask = (rng.random(n) > 0.1).astype(np.uint8)
    G = lambda x: torch.from_numpy(x).to(DEV)  # noqa: E731
    for bound in (0.05, 0.0, 0.15):
        got = ops.probe_stats(ops.probe_compare(G(a), G(b), G(mask), bound))
        nv, nm, mx = oracle.probe_compare(a, b, mask, bound)
        assert (got["n_valid"], got["n_moved"]) == (nv, nm)
        assert got["max_abs"] == mx
    ok = ops.probe_stats(ops.probe_compare(G(a), G(a.copy()), G(mask)))
    assert ok["n_moved"] == 0 and ok["max_abs"] == 0.0 and ok["n_valid"] == int(mask.sum())


def test_probe_screens_the_first_ahead_chunk():
    z, y, mask = _batch(4, 128, 4096, torch.bfloat16, seed=4, std=3.0)
    zg, yg, mg = z.to(DEV), torch.from_numpy(y).to(DEV), torch.from_numpy(mask).to(DEV)
    cache = ops.OldLogprobCache(1, torch.empty(512, dtype=torch.float32, device=DEV))
    rec = cache.record(zg, yg, mg)
    # a deterministic re-score at unchanged weights moves nothing: the probe passes
    probe = ops.Probe()
    lp, _, _ = ops.logprob_fwd(zg, yg, mg)
    st = ops.probe_stats(ops.probe_compare(rec, lp, mg))
    assert st["n_moved"] == 0 and probe.finish(st) and not probe.due()
    # a stochastic layer (noise on the logits of the training-mode forward) fails the strict gate
    g = torch.Generator(device="cpu").manual_seed(9)
    noisy = (z.float() + torch.randn(z.shape, generator=g) * 0.5).to(torch.bfloat16).to(DEV)
    lp2, _, _ = ops.logprob_fwd(noisy, yg, mg)
    st2 = ops.probe_stats(ops.probe_compare(rec, lp2, mg))
    assert st2["n_moved"] > 0
    assert ops.Probe().finish(st2) is False


def test_frozen_pi_old_makes_the_clip_bind_on_the_gpu():
    # n_mini = 2 over 16 rows; between the two optimizer steps the policy
    # moves (a logit drift).  With the cache the ratio departs from 1 in
    # mini-batch 1 and the clip binds; with pi_old recomputed from the
    # current policy the ratio is exactly 1 and nothing clips.
    n_rows, T, V = 16, 64, 2048
    z0, y, mask = _batch(n_rows, T, V, torch.float32, seed=6)
    g = torch.Generator(device="cpu").manual_seed(7)
    z1 = z0 + torch.randn(z0.shape, generator=g) * 0.6
    z0g, z1g = z0.to(DEV), z1.to(DEV)
    yg, mg = torch.from_numpy(y).to(DEV), torch.from_numpy(mask).to(DEV)
    n_mini, n_micro, mini_rows, micro_rows = ops.plan_fixed(n_rows, 4, 8, 4)
    assert (n_mini, n_micro) == (2, 2) and ops.needs_ahead_pass(n_mini)
    adv_row = torch.from_numpy(np.where(np.arange(n_rows) % 2 == 0, 1.0, -1.0).astype(np.float32)).to(DEV)
    row_off = torch.arange(0, micro_rows * T + 1, T, dtype=torch.int64, device=DEV)
    tok_row = ops.tok_row(row_off, micro_rows * T)
    calls = [(i, j) for i in range(n_mini) for j in range(n_micro)]
    cache = ops.OldLogprobCache(len(calls), torch.empty(n_rows * T, dtype=torch.float32, device=DEV))
    for i, j in calls:                                        # the ahead walk, policy at rollout
        a, e = ops.plan_chunk(n_rows, mini_rows, micro_rows, i, j)
        cache.record(z0g[a * T:e * T], yg[a * T:e * T], mg[a * T:e * T])
    clipped = {}
    for i, j in calls:                                        # the training walk
        a, e = ops.plan_chunk(n_rows, mini_rows, micro_rows, i, j)
        sl = slice(a * T, e * T)
        z = z0g if i == 0 else z1g
        frozen = cache.replay((e - a) * T)
        recomputed, _, _ = ops.logprob_fwd(z[sl], yg[sl], mg[sl])
        res = {}
        for name, old in (("cache", frozen), ("recomputed", recomputed)):
            ws = ops.loss_fwd_bwd(z[sl], yg[sl], mg[sl], old, tok_row, adv_row[a:e], row_off, scale=1.0)
            res[name] = ops.stats_to_dicts(ws["chunk_stats"])[0]["n_clipped"]
            if name == "cache" and i == 1:
                # per-token parity with the oracle on the drifted policy against the frozen record
                zz = z[sl].double().cpu().numpy()
                ref = oracle.loss_fwd_bwd(zz, y[sl], mask[sl], to_f64(old),
                                          to_f64(adv_row[a:e])[tok_row.cpu().numpy()], 1.0)
                assert res[name] == int(ref["clipped"].sum())
                assert np.max(np.abs(to_f64(ws["loss_tok"]) - ref["loss_tok"])) <= 1e-4
        clipped[(i, j)] = res
    for (i, j), r in clipped.items():
        assert r["recomputed"] == 0
        if i == 0:
            assert r["cache"] == 0
        else:
            assert r["cache"] >= 20, r


def test_paired_record_gives_the_ratio_exactly_one_on_long_rows():
    # Rows of V = 151 936 bf16 (past 1024 vectors, where the plain forward pass
    # streams): pi_old recorded with grpo_old_cache_record_paired and replayed
    # into the fused loss on unchanged logits gives log-ratio 0 on every valid
    # token, so rho = 1 exactly, nothing clips and each token's surrogate loss is -A
    # ([P1] "pi_old must be frozen across the window": the ratio of the policy
    # to its detached copy).  The plain record agrees to float32 summation order.
    n_rows, T, V = 4, 48, 151936
    z, y, mask = _batch(n_rows, T, V, torch.bfloat16, seed=21, std=3.0)
    zg, yg, mg = z.to(DEV), torch.from_numpy(y).to(DEV), torch.from_numpy(mask).to(DEV)
    n = n_rows * T
    adv = torch.tensor([1.0, -1.0, 0.5, -0.25], dtype=torch.float32, device=DEV)
    row_off = torch.arange(0, n + 1, T, dtype=torch.int64, device=DEV)
    tok_row = ops.tok_row(row_off, n)
    recs = {}
    for paired in (False, True):
        cache = ops.OldLogprobCache(1, torch.empty(n, dtype=torch.float32, device=DEV))
        cache.record(zg, yg, mg, paired=paired)
        recs[paired] = cache.replay(n).clone()
    s = 1.0 / float(mask.sum())
    ws = ops.loss_fwd_bwd(zg, yg, mg, recs[True], tok_row, adv, row_off, scale=s)
    torch.cuda.synchronize()
    v = torch.from_numpy(mask.astype(bool)).to(DEV)
    assert torch.equal(ws["logp"][v], recs[True][v])
    assert ops.stats_to_dicts(ws["chunk_stats"])[0]["n_clipped"] == 0
    want = -adv[tok_row.long()]
    assert torch.equal(ws["loss_tok"][v], want[v])
    diff = (recs[False] - recs[True]).abs()[v]
    assert float(diff.max()) <= 2e-5
