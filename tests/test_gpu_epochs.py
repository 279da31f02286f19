"""GPU side of inner epochs and the seeded shuffle ([P3] section 1; [P1]
"What's not done", item 2): chunk token maps and gathers against the oracle,
a shuffled chunk read through tok_src equal bit for bit to the same chunk
copied out contiguously, the cache's rewind across unshuffled epochs, and a
two-epoch shuffled step end to end against the oracle with pi_old frozen at
the ahead pass."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import DEV, assert_tokens_match, to_f64
from grpo_token_level_amd import ops

pytestmark = pytest.mark.gpu

G = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731


def test_chunk_tok_src_matches_oracle():
    lens = np.array([3, 0, 5, 2, 7, 1], np.int64)
    src_off = np.concatenate([[0], np.cumsum(lens)])
    for rows in ([2, 0], [5, 4, 3, 2, 1, 0], [1, 3], [4]):
        dst_off = np.concatenate([[0], np.cumsum(lens[rows])])
        got = ops.chunk_tok_src(G(src_off), G(np.array(rows, np.int64)), G(dst_off)).cpu().numpy()
        assert got.tolist() == oracle.chunk_token_sources(src_off.tolist(), rows)
    # a row index outside the batch maps its tokens to -1
    got = ops.chunk_tok_src(G(src_off), G(np.array([0, 9], np.int64)), G(np.array([0, 3, 5], np.int64)))
    assert got.cpu().numpy().tolist() == [0, 1, 2, -1, -1]


def test_gather_matches_numpy():
    rng = np.random.default_rng(1)
    for dt in (np.uint8, np.int16, np.float32, np.int64):
        src = rng.integers(0, 100, 1000).astype(dt)
        idx = rng.integers(0, 1000, 777).astype(np.int64)
        idx[5] = 1000                       # out of range -> 0
        idx[6] = -3
        got = ops.gather(G(src), G(idx)).cpu().numpy()
        want = np.array(oracle.gather(src.tolist(), np.clip(idx, 0, 999).tolist()), dt)
        want[5] = want[6] = 0
        assert np.array_equal(got, want)


def _batch(n_rows, T, V, dtype, seed, noise=0.3):
    g = torch.Generator(device="cpu").manual_seed(seed)
    z = (torch.randn((n_rows * T, V), generator=g) * 2.0).to(dtype)
    rng = np.random.default_rng(seed)
    y = rng.integers(0, V, n_rows * T).astype(np.int32)
    mask = (rng.random(n_rows * T) > 0.25).astype(np.uint8)
    adv = rng.normal(0, 1, n_rows).astype(np.float32)
    lp = oracle.logprob_fwd(z.double().numpy(), y, np.ones(n_rows * T, np.uint8))["logp"]
    old = (lp + rng.normal(0, noise, n_rows * T)).astype(np.float32)
    return z, y, mask, adv, old


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_shuffled_chunk_through_tok_src_equals_the_copied_chunk(dtype):
    n_rows, T, V = 12, 40, 1000
    z, y, mask, adv, old = _batch(n_rows, T, V, dtype, seed=2)
    rows = [7, 2, 11, 0]
    src_off = np.arange(0, (n_rows + 1) * T, T, dtype=np.int64)
    dst_off = np.arange(0, (len(rows) + 1) * T, T, dtype=np.int64)
    src = np.array(oracle.chunk_token_sources(src_off.tolist(), rows), np.int64)
    tok_src = ops.chunk_tok_src(G(src_off), G(np.array(rows, np.int64)), G(dst_off))
    assert tok_src.cpu().numpy().tolist() == src.tolist()
    tok_row = ops.tok_row(G(dst_off), len(src))
    adv_chunk = ops.gather(G(adv), G(np.array(rows, np.int64)))
    zg = z.to(DEV)
    dl_batch = torch.zeros_like(zg)
    via = ops.loss_fwd_bwd(zg, G(y), G(mask), G(old), tok_row, adv_chunk, G(dst_off), scale=0.01,
                           dlogits=dl_batch, tok_src=tok_src)
    # the same chunk copied out contiguously
    ii = torch.as_tensor(src, device=DEV)
    copy = ops.loss_fwd_bwd(zg[ii].contiguous(), G(y[src]), G(mask[src]), G(old[src]), tok_row, adv_chunk,
                            G(dst_off), scale=0.01)
    torch.cuda.synchronize()
    for k in ("logp", "entropy", "loss_tok", "tok_flags", "row_stats", "chunk_stats"):
        assert torch.equal(via[k][:len(src)] if via[k].dim() == 1 else via[k], copy[k][:len(src)]
                           if copy[k].dim() == 1 else copy[k]), k
    assert torch.equal(dl_batch[ii], copy["dlogits"])
    others = np.setdiff1d(np.arange(n_rows * T), src)
    assert not dl_batch[torch.as_tensor(others, device=DEV)].any()     # untouched rows
    # and the chunk against the oracle
    d = dict(z64=z.double().numpy()[src], target=y[src], mask=mask[src], old=old[src], dtype=dtype)
    ref = oracle.loss_fwd_bwd(d["z64"], d["target"], d["mask"], d["old"].astype(np.float64),
                              adv[np.repeat(rows, T)].astype(np.float64), 0.01)
    assert_tokens_match(copy, ref, d)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 1003), (torch.float32, 1001), (torch.bfloat16, 50257)])
def test_shuffled_chunk_of_misaligned_rows_matches_oracle(dtype, V):
    # Rows off 16-byte alignment (odd V, ld = V), read and written in the
    # batch through tok_src: the register kernel over the aligned vectors that
    # cover each row (dlogits shares the logits' layout).  A row's alignment
    # phase depends on where it sits, so the chunk copied out contiguously is
    # summed in another lane partition; both are checked against the oracle.
    n_rows, T = (6, 8) if V > 10000 else (12, 40)
    z, y, mask, adv, old = _batch(n_rows, T, V, dtype, seed=V)
    rows = [4, 1, 5, 0] if V > 10000 else [7, 2, 11, 0]
    src_off = np.arange(0, (n_rows + 1) * T, T, dtype=np.int64)
    dst_off = np.arange(0, (len(rows) + 1) * T, T, dtype=np.int64)
    src = np.array(oracle.chunk_token_sources(src_off.tolist(), rows), np.int64)
    tok_src = ops.chunk_tok_src(G(src_off), G(np.array(rows, np.int64)), G(dst_off))
    tok_row = ops.tok_row(G(dst_off), len(src))
    adv_chunk = ops.gather(G(adv), G(np.array(rows, np.int64)))
    zg = z.to(DEV)
    dl_batch = torch.full_like(zg, 3.0)
    via = ops.loss_fwd_bwd(zg, G(y), G(mask), G(old), tok_row, adv_chunk, G(dst_off), scale=0.01,
                           dlogits=dl_batch, tok_src=tok_src)
    torch.cuda.synchronize()
    others = np.setdiff1d(np.arange(n_rows * T), src)
    assert torch.all(dl_batch[torch.as_tensor(others, device=DEV)] == 3.0)   # rows outside the chunk untouched
    out = {k: v[:len(src)] for k, v in via.items() if torch.is_tensor(v) and v.dim() == 1}
    out["dlogits"] = dl_batch[torch.as_tensor(src, device=DEV)]
    out["chunk_stats"], out["row_stats"] = via["chunk_stats"], via["row_stats"]
    d = dict(z64=z.double().numpy()[src], target=y[src], mask=mask[src], old=old[src], dtype=dtype)
    ref = oracle.loss_fwd_bwd(d["z64"], d["target"], d["mask"], d["old"].astype(np.float64),
                              adv[np.repeat(rows, T)].astype(np.float64), 0.01)
    assert_tokens_match(out, ref, d)


def test_tok_src_outside_the_batch_poisons_the_token():
    z, y, mask, adv, old = _batch(2, 16, 256, torch.float32, seed=3)
    mask[:] = 1
    tok_src = G(np.array([0, 1, 2, 99, 4], np.int64))            # 99 >= 32 batch tokens
    off = G(np.array([0, 5], np.int64))
    ws = ops.loss_fwd_bwd(z.to(DEV), G(y), G(mask), G(old), ops.tok_row(off, 5), G(adv[:1]), off, scale=1.0,
                          tok_src=tok_src)
    flags = ws["tok_flags"].cpu().numpy()
    assert flags[3] == 5 and np.all(flags[[0, 1, 2, 4]] & 1)
    st = ops.stats_to_dicts(ws["chunk_stats"])[0]
    assert st["n_nonfinite"] >= 1 and ops.Accumulator(1).add(st) == "NONFINITE"


def test_unshuffled_epochs_replay_the_cache_by_call_order():
    n_rows, T, V = 8, 32, 512
    z, y, mask, adv, _ = _batch(n_rows, T, V, torch.bfloat16, seed=4)
    zg, yg, mg = z.to(DEV), G(y), G(mask)
    ep = ops.plan_epochs(n_rows, 2, 4, 2, mu=3, shuffle=False)
    calls = [(i, j) for i in range(ep["n_mini"]) for j in range(ep["n_micro"])]
    cache = ops.OldLogprobCache(len(calls), torch.empty(n_rows * T, dtype=torch.float32, device=DEV))
    recs = []
    for i, j in calls:
        rows = ep["perm"][0][i * ep["mini_rows"] + j * ep["micro_rows"]:][:ep["micro_rows"]]
        a, b = int(rows[0]) * T, (int(rows[-1]) + 1) * T
        recs.append(cache.record(zg[a:b], yg[a:b], mg[a:b]).clone())
    for e in range(3):
        if e:
            cache.rewind()
        for k in range(len(calls)):
            assert torch.equal(cache.replay(ep["micro_rows"] * T), recs[k])


def test_two_shuffled_epochs_end_to_end():
    # pi_old from one ahead walk in batch order (the cache buffer holds the
    # whole batch's log-probs in batch token order); each epoch reshuffles
    # the rows; every chunk reads logits, inputs and pi_old through tok_src.
    n_rows, T, V = 16, 24, 700
    z, y, mask, adv, _ = _batch(n_rows, T, V, torch.float32, seed=5)
    g = torch.Generator(device="cpu").manual_seed(6)
    z_now = z + torch.randn(z.shape, generator=g) * 0.4        # the policy has moved since the rollout
    zg, znow, yg, mg = z.to(DEV), z_now.to(DEV), G(y), G(mask)
    ep = ops.plan_epochs(n_rows, 4, 8, 4, mu=2, shuffle=True, seed=11)
    assert ep["perm"].tolist() == oracle.plan_epochs(n_rows, 4, 8, 4, 2, True, 11)["perm"]
    batch_off = np.arange(0, (n_rows + 1) * T, T, dtype=np.int64)
    # ahead walk in batch order: one record per fixed-plan chunk, records end to end
    n_mini, n_micro, mini_rows, micro_rows = ops.plan_fixed(n_rows, 4, 8, 4)
    cache = ops.OldLogprobCache(n_mini * n_micro, torch.empty(n_rows * T, dtype=torch.float32, device=DEV))
    for i in range(n_mini):
        for j in range(n_micro):
            a, b = ops.plan_chunk(n_rows, mini_rows, micro_rows, i, j)
            cache.record(zg[a * T:b * T], yg[a * T:b * T], mg[a * T:b * T])
    old_batch = cache.buf                                        # pi_old of every batch token
    old_np = to_f64(old_batch)
    dst_off = G(np.arange(0, micro_rows * T + 1, T, dtype=np.int64))
    tok_row = ops.tok_row(dst_off, micro_rows * T)
    for e in range(2):
        for i in range(ep["n_mini"]):
            for j in range(ep["n_micro"]):
                rows = ep["perm"][e][i * mini_rows + j * micro_rows:][:micro_rows]
                rows_g = G(np.asarray(rows, np.int64))
                tok_src = ops.chunk_tok_src(G(batch_off), rows_g, dst_off)
                ws = ops.loss_fwd_bwd(znow, yg, mg, old_batch, tok_row, ops.gather(G(adv), rows_g), dst_off,
                                      scale=1.0, dlogits=None, tok_src=tok_src)
                src = np.array(oracle.chunk_token_sources(batch_off.tolist(), list(rows)), np.int64)
                ref = oracle.loss_fwd_bwd(z_now.double().numpy()[src], y[src], mask[src], old_np[src],
                                          adv[np.repeat(rows, T)].astype(np.float64), 1.0, want_dz=False)
                d = dict(z64=z_now.double().numpy()[src], target=y[src], mask=mask[src], old=old_np[src].astype(np.float32),
                         dtype=torch.float32)
                assert_tokens_match(ws, ref, d, check_dz=False)
                st = ops.stats_to_dicts(ws["chunk_stats"])[0]
                assert st["n_clipped"] == int(ref["clipped"].sum())
