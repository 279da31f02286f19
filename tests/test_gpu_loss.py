"""GPU parity of the fused loss kernel, the forward-only pass and the small
device helpers against the oracle, element by element, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import DEV, assert_tokens_match, make_chunk, rel_l2, run_gpu, run_oracle, to_f64
from grpo_token_level_amd import ops

pytestmark = pytest.mark.gpu


def assert_same_up_to_sum_order(a, b):
    """The forward-only pass streams rows past 1024 vectors in another lane
    partition than the fused kernel, so their outputs agree to rounding (a
    few float32 ulps), with the same non-finite entries."""
    a, b = to_f64(a), to_f64(b)
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb) and np.array_equal(a[~fa], b[~fb])
    assert np.all(np.abs(a[fa] - b[fb]) <= 2e-6 * np.maximum(1.0, np.abs(b[fb])))


def _stats(ws):
    return ops.stats_to_dicts(ws["chunk_stats"])[0], ops.stats_to_dicts(ws["row_stats"])


def _check_stats(ws, ref, d):
    chunk, rows = _stats(ws)
    want_rows = oracle.row_stats(ref, d["row_off"].tolist())
    for g, w in zip(rows, want_rows):
        for k in ("n_valid", "n_valid_rows", "n_nonfinite"):
            assert g[k] == w[k], k
        assert g["loss_sum"] == pytest.approx(w["loss_sum"], rel=1e-4, abs=1e-4)
    want = oracle.chunk_stats(ref, d["row_off"].tolist())
    assert chunk["n_valid"] == want["n_valid"]
    assert chunk["loss_sum"] == pytest.approx(sum(r["loss_sum"] for r in rows), rel=1e-12, abs=1e-12)


# (V, in dtype, out dtype, n_tok): register paths (wave / 256 / 1024 threads
# per row), the generic path (V or stride not a multiple of the vector),
# ragged token counts around the 4-rows-per-block wave path.
CASES = [
    (1024, torch.float32, torch.float32, 203),
    (1024, torch.float32, torch.bfloat16, 61),
    (4096, torch.bfloat16, torch.bfloat16, 130),
    (4096, torch.bfloat16, torch.float32, 67),
    (16384, torch.bfloat16, torch.bfloat16, 37),
    (32000, torch.bfloat16, torch.bfloat16, 21),
    # 256-thread blocks with 16 and 24 vectors per lane
    (24576, torch.bfloat16, torch.float32, 7),
    (40960, torch.bfloat16, torch.bfloat16, 9),
    (20000, torch.float32, torch.float32, 6),
    (151936, torch.bfloat16, torch.bfloat16, 9),
    (151936, torch.bfloat16, torch.float32, 5),
    (8, torch.float32, torch.float32, 33),
    (1, torch.float32, torch.float32, 10),
    (7, torch.bfloat16, torch.bfloat16, 17),
    (1000, torch.bfloat16, torch.bfloat16, 23),
    # rows off 16-byte alignment (V and the row stride odd), dlogits in the
    # same phase: the register kernel over the aligned vectors covering each
    # row (256 threads x 16, 1024 x 8, 1024 x 19 vectors; fp32 256 x 24)
    (50257, torch.bfloat16, torch.bfloat16, 11),
    (32001, torch.bfloat16, torch.bfloat16, 13),
    (151939, torch.bfloat16, torch.bfloat16, 5),
    (20001, torch.float32, torch.float32, 6),
    # 512-thread blocks: 12 and 16 vectors per lane
    (57344, torch.bfloat16, torch.float32, 5),
    (65536, torch.bfloat16, torch.bfloat16, 4),
    (200000, torch.bfloat16, torch.bfloat16, 5),
    # rows past the register file: the tail of each lane's vectors in LDS
    (155656, torch.bfloat16, torch.bfloat16, 5),
    (202048, torch.bfloat16, torch.bfloat16, 6),
    (229376, torch.bfloat16, torch.float32, 3),
    (100000, torch.float32, torch.float32, 4),
    # past registers and LDS: up to 4 more vectors per lane read in both
    # sweeps (one vector past the LDS capacity, a 256k vocabulary, the full
    # capacity of 262 144)
    (229384, torch.bfloat16, torch.bfloat16, 3),
    (256000, torch.bfloat16, torch.bfloat16, 3),
    (256000, torch.bfloat16, torch.float32, 2),
    (262144, torch.bfloat16, torch.bfloat16, 3),
    # one vector past that, fp32 rows past the LDS capacity, rows off 16-byte
    # alignment with an output of another phase: the streaming kernel
    (262152, torch.bfloat16, torch.bfloat16, 2),
    (114696, torch.float32, torch.float32, 2),
    (50257, torch.bfloat16, torch.float32, 9),
    (1003, torch.float32, torch.bfloat16, 31),
]


@pytest.mark.parametrize("V,din,dout,n", CASES)
def test_loss_matches_oracle(V, din, dout, n):
    print(f"loss parity V={V} in={din} out={dout} n={n}", flush=True)
    d = make_chunk(n, V, din, seed=V + n, noise=0.4)
    N = int(d["mask"].sum())
    scale = 1.0 / max(N, 1)
    ws = run_gpu(d, scale=scale, out_dtype=dout)
    ref = run_oracle(d, scale)
    assert_tokens_match(ws, ref, d)
    _check_stats(ws, ref, d)


@pytest.mark.parametrize("din,V,ld,n", [(torch.float32, 1024, 1040, 45), (torch.bfloat16, 1024, 1040, 45),
                                        (torch.bfloat16, 202048, 202064, 4), (torch.bfloat16, 256000, 256016, 3),
                                        (torch.bfloat16, 50257, 50263, 9)])
def test_padded_row_stride_and_inplace(din, V, ld, n):
    # logits rows padded to ld > V: dlogits into a contiguous tensor, into one
    # with the logits' stride, then the same chunk updated in place
    # (202048: part of each row in LDS; 256000: part read again in the
    # gradient sweep; 50257 with an odd stride: rows of every alignment phase,
    # the contiguous output in another phase than its logits row -> the
    # streaming kernel, the strided and in-place ones in the same phase ->
    # the register kernel over aligned vectors)
    d = make_chunk(n, V, din, seed=3, ld=ld)
    scale = 0.01
    ref = run_oracle(d, scale)
    ws = run_gpu(d, scale=scale)
    assert_tokens_match(ws, ref, d)
    strided = torch.full((n, ld), 7.0, dtype=din, device=DEV)
    ws1 = run_gpu(d, scale=scale, dlogits=strided[:, :V])
    assert_tokens_match(ws1, ref, d)
    assert torch.all(strided[:, V:] == 7.0)                  # the padding columns are never written
    ws2 = run_gpu(d, scale=scale, dlogits="inplace")
    assert_tokens_match(ws2, ref, d)
    assert torch.equal(ws2["dlogits"], ws1["dlogits"])
    if V % 8 == 0:
        assert torch.equal(ws2["dlogits"], ws["dlogits"])
    assert torch.equal(d["logits"], ws2["dlogits"])          # the logits buffer now holds dlogits


def test_denominator_from_device_count():
    d = make_chunk(300, 4096, torch.bfloat16, seed=4)
    N = ops.count_valid(d["g"]["mask"])
    assert int(N.item()) == int(d["mask"].sum())
    a = run_gpu(d, scale=1.0, denom=N)
    b = run_gpu(d, scale=1.0 / int(d["mask"].sum()))
    ref = run_oracle(d, 1.0 / int(d["mask"].sum()))
    assert_tokens_match(a, ref, d)
    assert rel_l2(to_f64(a["dlogits"]), to_f64(b["dlogits"])) < 1e-6


def test_all_masked_and_empty():
    d = make_chunk(40, 1024, torch.float32, seed=5)
    d["g"]["mask"].zero_()
    d["mask"][:] = 0
    ws = run_gpu(d, scale=1.0)
    assert not ws["dlogits"].any() and not ws["logp"].any() and not ws["loss_tok"].any()
    chunk, rows = _stats(ws)
    assert chunk["n_valid"] == 0 and chunk["loss_sum"] == 0.0 and chunk["n_valid_rows"] == 0
    # zero tokens: stats still written
    e = make_chunk(0, 64, torch.float32, seed=6, n_rows=1, with_old=False)
    ws = run_gpu(e, scale=1.0)
    chunk, _ = _stats(ws)
    assert chunk["n_valid"] == 0 and chunk["loss_sum"] == 0.0


def test_bad_targets_and_nan_logits_are_flagged_not_read():
    d = make_chunk(20, 1024, torch.float32, seed=7)
    d["mask"][:] = 1
    d["g"]["mask"].fill_(1)
    d["target"][3] = 1024
    d["target"][4] = -5
    d["g"]["target"].copy_(torch.from_numpy(d["target"]))
    d["logits"][9, 17] = float("nan")
    d["z64"][9, 17] = np.nan
    ws = run_gpu(d, scale=1.0)
    flags = ws["tok_flags"].cpu().numpy()
    assert set(np.nonzero(flags & 4)[0].tolist()) == {3, 4, 9}
    chunk, _ = _stats(ws)
    assert chunk["n_nonfinite"] == 3
    acc = ops.Accumulator(2)
    assert acc.add(chunk) == "NONFINITE"          # window of 2 poisoned at position 0
    assert not np.isfinite(chunk["obj_sum"])       # the objective share carries the NaN too
    clean = dict(chunk, n_nonfinite=0, loss_sum=1.0, entropy_sum=1.0, obj_sum=1.0)
    assert acc.add(clean) == "SKIPPED"            # the rest of the poisoned window
    assert acc.add(clean) == "OK"                 # a fresh window


# first: elements held by the first vector of every lane of a row (lanes per
# row x elements per 16-byte vector on that kernel path)
@pytest.mark.parametrize("V,dtype,first", [(151936, torch.bfloat16, 8192), (16384, torch.bfloat16, 2048),
                                           (4096, torch.bfloat16, 512), (1024, torch.float32, 256),
                                           (202048, torch.bfloat16, 8192), (256000, torch.bfloat16, 8192),
                                           (262152, torch.bfloat16, 2056), (50257, torch.bfloat16, 8192),
                                           (32001, torch.bfloat16, 2048), (61440, torch.bfloat16, 4096),
                                           (40960, torch.bfloat16, 2048)])
def test_special_rows(V, dtype, first):
    # Rows the one-sweep sums cannot take and that go through the exact
    # max-shifted sweeps instead: scattered -inf logits, the whole first
    # vector of every lane at -inf, a logit ~150 nats above the rest of its
    # lane, a -inf target logit; plus a constant row and a row shifted down.
    print(f"special rows V={V} {dtype}", flush=True)
    n = 8
    d = make_chunk(n, V, dtype, seed=40 + V, masked_frac=0.0, n_rows=2)
    z = d["logits"].float().cpu()
    rng = np.random.default_rng(V)
    z[1, rng.choice(V, V // 100, replace=False)] = float("-inf")
    z[2, :first] = float("-inf")
    z[3, V // 2 + 3] = 150.0
    z[4].fill_(0.5)
    z[5] -= 30.0
    z[6, int(d["target"][6])] = float("-inf")
    for r in (1, 2):
        if not np.isfinite(float(z[r, int(d["target"][r])])):
            d["target"][r] = int(np.nonzero(np.isfinite(z[r].numpy()))[0][-1])
    zz = z.to(dtype)
    d["logits"].copy_(zz.to(DEV))
    d["z64"] = zz.double().numpy()
    d["g"]["target"].copy_(torch.from_numpy(d["target"]))
    lp = oracle.logprob_fwd(d["z64"], d["target"], np.ones(n, np.uint8))["logp"]
    with np.errstate(invalid="ignore"):
        d["old"] = np.where(np.isfinite(lp), lp + 0.05, 0.0).astype(np.float32)
    d["g"]["old"].copy_(torch.from_numpy(d["old"]))
    ws = run_gpu(d, scale=0.1)
    ref = run_oracle(d, 0.1)
    assert ref["nonfinite"].tolist() == [False] * 6 + [True, False]
    assert_tokens_match(ws, ref, d)
    f_logp, f_lse, f_ent = ops.logprob_fwd(d["logits"], d["g"]["target"], d["g"]["mask"])
    assert_same_up_to_sum_order(f_logp, ws["logp"])
    assert_same_up_to_sum_order(f_ent, ws["entropy"])
    fwd = oracle.logprob_fwd(d["z64"], d["target"], d["mask"])
    fin = np.isfinite(fwd["logp"])
    assert np.max(np.abs(to_f64(f_logp)[fin] - fwd["logp"][fin])) <= (1e-5 if dtype == torch.float32 else 2e-3)
    assert np.max(np.abs(to_f64(f_lse) - fwd["lse"])) <= (1e-5 if dtype == torch.float32 else 2e-3)


@pytest.mark.parametrize("V,n", [(16384, 300), (4096, 1100)])
def test_many_blocks_with_a_periodic_mask(V, n):
    # More blocks than one run of 8 x 16 (the block -> token deal over the
    # XCDs permutes them) plus a ragged tail, with valid and masked tokens
    # alternating: every token is processed exactly once, as the oracle says.
    print(f"periodic mask V={V} n={n}", flush=True)
    d = make_chunk(n, V, torch.bfloat16, seed=50 + n, masked_frac=0.0, n_rows=7)
    d["mask"][1::2] = 0
    d["g"]["mask"].copy_(torch.from_numpy(d["mask"]))
    N = int(d["mask"].sum())
    ws = run_gpu(d, scale=1.0 / N)
    ref = run_oracle(d, 1.0 / N)
    assert_tokens_match(ws, ref, d)
    _check_stats(ws, ref, d)


def test_clip_quadrants_exercised():
    d = make_chunk(400, 1024, torch.float32, seed=8, noise=0.6)
    ref = run_oracle(d, 1.0)
    ws = run_gpu(d, scale=1.0)
    assert_tokens_match(ws, ref, d)
    A = d["adv_row"][d["tok_row"]]
    rho = np.exp(ref["logp"] - d["old"])
    v = ref["valid"]
    for cond in ((A > 0) & (rho > 1.2), (A > 0) & (rho < 0.8), (A < 0) & (rho > 1.2), (A < 0) & (rho < 0.8)):
        assert (cond & v).sum() >= 5


def test_asymmetric_clip():
    d = make_chunk(200, 1024, torch.float32, seed=9, noise=0.5)
    ref = run_oracle(d, 0.5, eps=(0.2, 0.28))
    ws = run_gpu(d, scale=0.5, eps=(0.2, 0.28))
    assert_tokens_match(ws, ref, d, eps=(0.2, 0.28))


def test_runs_are_bit_identical():
    d = make_chunk(64, 151936, torch.bfloat16, seed=10)
    a = run_gpu(d, scale=0.001)
    b = run_gpu(d, scale=0.001)
    for k in ("dlogits", "logp", "entropy", "loss_tok", "row_stats", "chunk_stats"):
        assert torch.equal(a[k], b[k]), k


def test_chunked_equals_unchunked_bit_exact():
    # The same rows run as one chunk and as four: dlogits, per-token outputs and
    # row stats are bit-identical (per-token scale, row-local reductions).
    n_rows, T, V = 16, 24, 4096
    d = make_chunk(n_rows * T, V, torch.bfloat16, seed=11, n_rows=2)
    row_off = np.arange(0, n_rows * T + 1, T).astype(np.int64)
    tok_row = np.repeat(np.arange(n_rows, dtype=np.int32), T)
    adv = np.random.default_rng(1).normal(size=n_rows).astype(np.float32)
    g = d["g"]
    whole = ops.loss_fwd_bwd(d["logits"], g["target"], g["mask"], g["old"], torch.from_numpy(tok_row).to(DEV),
                             torch.from_numpy(adv).to(DEV), torch.from_numpy(row_off).to(DEV), scale=1 / 377.0)
    parts = []
    for c in range(4):
        a, b = c * 4 * T, (c + 1) * 4 * T
        parts.append(ops.loss_fwd_bwd(d["logits"][a:b], g["target"][a:b], g["mask"][a:b], g["old"][a:b],
                                      torch.from_numpy(tok_row[a:b] - 4 * c).to(DEV),
                                      torch.from_numpy(adv[4 * c:4 * c + 4]).to(DEV),
                                      torch.from_numpy(row_off[4 * c:4 * c + 5] - a).to(DEV), scale=1 / 377.0))
    assert torch.equal(torch.cat([p["dlogits"] for p in parts]), whole["dlogits"])
    for k in ("logp", "entropy", "loss_tok", "tok_flags"):
        assert torch.equal(torch.cat([p[k] for p in parts]), whole[k]), k
    assert torch.equal(torch.cat([p["row_stats"][:4] for p in parts]), whole["row_stats"][:n_rows])


@pytest.mark.parametrize("n_rows", [1, 15, 16, 17, 40])
def test_row_stats_independent_of_the_chunk(n_rows):
    """A row's stats are the same bits whether the row is reduced alone or
    inside a chunk of n_rows rows (ragged lengths, an empty row, a short last
    row); the chunk's stats match the oracle."""
    rng = np.random.default_rng(40 + n_rows)
    lens = [int(x) for x in rng.integers(5, 40, n_rows)]
    if n_rows > 2:
        lens[1] = 0
        lens[-1] = 3
    n_tok = sum(lens)
    d = make_chunk(n_tok, 1024, torch.float32, seed=50 + n_rows, n_rows=1)
    row_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    d["row_off"] = row_off
    d["tok_row"] = np.repeat(np.arange(n_rows, dtype=np.int32), lens)
    d["adv_row"] = rng.normal(0, 1, n_rows).astype(np.float32)
    for k in ("row_off", "tok_row", "adv_row"):
        d["g"][k] = torch.from_numpy(d[k]).to(DEV)
    scale = 1.0 / 97.0
    whole = run_gpu(d, scale=scale)
    ref = run_oracle(d, scale)
    assert_tokens_match(whole, ref, d)
    _check_stats(whole, ref, d)
    g = d["g"]
    for r in range(n_rows):
        a, b = int(row_off[r]), int(row_off[r + 1])
        one = ops.loss_fwd_bwd(d["logits"][a:b], g["target"][a:b], g["mask"][a:b], g["old"][a:b],
                               torch.zeros(b - a, dtype=torch.int32, device=DEV), g["adv_row"][r:r + 1],
                               torch.tensor([0, b - a], dtype=torch.int64, device=DEV), scale=scale)
        assert torch.equal(one["row_stats"][0], whole["row_stats"][r]), r
        assert torch.equal(one["loss_tok"], whole["loss_tok"][a:b]), r


@pytest.mark.parametrize("V,dtype,n", [(1024, torch.float32, 130), (151936, torch.bfloat16, 7),
                                       (1000, torch.bfloat16, 19), (4096, torch.bfloat16, 66),
                                       (202048, torch.bfloat16, 5), (100000, torch.float32, 4),
                                       (50257, torch.bfloat16, 6), (256000, torch.bfloat16, 3)])
def test_logprob_fwd_matches_oracle(V, dtype, n):
    d = make_chunk(n, V, dtype, seed=12 + V, with_old=False)
    logp, lse, ent = ops.logprob_fwd(d["logits"], d["g"]["target"], d["g"]["mask"])
    ref = oracle.logprob_fwd(d["z64"], d["target"], d["mask"])
    tol = 1e-5 if dtype == torch.float32 else 2e-3
    assert np.max(np.abs(to_f64(logp) - ref["logp"])) <= tol
    assert np.max(np.abs(to_f64(lse) - ref["lse"])) <= tol
    assert np.max(np.abs(to_f64(ent) - ref["entropy"]) - 1e-5 * np.abs(ref["entropy"])) <= 1e-4
    # the loss kernel's forward outputs are the same numbers up to the order of the sums
    ws = run_gpu(make_chunk(n, V, dtype, seed=12 + V, with_old=False), scale=1.0, dlogits=None)
    assert_same_up_to_sum_order(ws["logp"], logp)
    assert_same_up_to_sum_order(ws["lse"], lse)


def _random_shapes(count=24, seed=2024):
    """Seeded shapes across every dispatch path: V in [1, 262 144], half
    log-uniform up to 4096 and half uniform above (the wave, 256- and
    1024-thread register paths, the LDS tail, the streaming kernel), both
    input dtypes, padded row strides, in-place and mixed-precision outputs,
    ragged token counts."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        if k % 2:
            V = int(rng.integers(4097, 262145))
        else:
            V = max(1, int(np.exp(rng.uniform(0.0, np.log(4096.0)))))
        din = torch.float32 if rng.random() < 0.4 else torch.bfloat16
        n = int(rng.integers(1, 9)) if V > 60000 else int(rng.integers(1, 40))
        pad = int(rng.integers(0, 14)) if rng.random() < 0.5 else 0
        mode = ("inplace", "new_other", "new_same")[int(rng.integers(0, 3))]
        out.append((k, V, din, n, pad, mode))
    return out


@pytest.mark.parametrize("k,V,din,n,pad,mode", _random_shapes())
def test_random_shapes_match_oracle(k, V, din, n, pad, mode):
    d = make_chunk(n, V, din, seed=300 + k, ld=V + pad)
    dout = din
    if mode == "new_other":
        dout = torch.float32 if din == torch.bfloat16 else torch.bfloat16
    ref = run_oracle(d, 1.0 / 50.0)
    if mode == "inplace":
        ws = ops.loss_fwd_bwd(d["logits"], d["g"]["target"], d["g"]["mask"],
                              d["g"]["old"], d["g"]["tok_row"], d["g"]["adv_row"], d["g"]["row_off"],
                              scale=1.0 / 50.0, dlogits="inplace")
    else:
        ws = run_gpu(d, scale=1.0 / 50.0, out_dtype=dout)
    assert_tokens_match(ws, ref, d)
    _check_stats(ws, ref, d)
    if mode != "inplace":
        # the forward-only pass on the same (untouched) logits
        logp, lse, ent = ops.logprob_fwd(d["logits"], d["g"]["target"], d["g"]["mask"])
        fwd = oracle.logprob_fwd(d["z64"], d["target"], d["mask"])
        fin = np.isfinite(fwd["logp"])
        tol = 1e-5 if din == torch.float32 else 2e-3
        assert np.max(np.abs(to_f64(logp)[fin] - fwd["logp"][fin]), initial=0.0) <= tol
        assert np.max(np.abs(to_f64(lse) - fwd["lse"]), initial=0.0) <= tol
        assert_same_up_to_sum_order(logp, ws["logp"])
        # the paired forward pass: the fused call's bits wherever that call keeps
        # aligned rows on chip (logits and dlogits rows both 16-byte aligned, up
        # to 262 144 bf16 / 114 688 fp32 logits)
        vec = 8 if din == torch.bfloat16 else 4
        out_b = 2 if dout == torch.bfloat16 else 4
        if (V % vec == 0 and (V + pad) % vec == 0 and (V * out_b) % 16 == 0
                and V // vec <= (32768 if din == torch.bfloat16 else 28672)):
            p_logp, p_lse, p_ent = ops.logprob_fwd(d["logits"], d["g"]["target"], d["g"]["mask"], paired=True)
            assert torch.equal(p_logp, ws["logp"]) and torch.equal(p_lse, ws["lse"])
            assert torch.equal(p_ent, ws["entropy"])


def test_count_valid_and_tok_row():
    rng = np.random.default_rng(13)
    for n in (0, 1, 15, 16, 17, 1000, 131072 + 5):
        m = (rng.random(n) < 0.6).astype(np.uint8) * rng.integers(1, 255, n).astype(np.uint8)
        t = torch.from_numpy(m).to(DEV)
        assert int(ops.count_valid(t).item()) == int((m != 0).sum())
        if n > 3:   # unaligned start
            assert int(ops.count_valid(t[3:]).item()) == int((m[3:] != 0).sum())
    off = np.array([0, 0, 5, 9, 9, 20], np.int64)
    tr = ops.tok_row(torch.from_numpy(off).to(DEV), 22).cpu().numpy()
    want = [1] * 5 + [2] * 4 + [4] * 11 + [-1, -1]
    assert tr.tolist() == want


def test_deferred_stats_over_several_chunks():
    # Four chunks with the reductions deferred, then one grpo_loss_stats over
    # all their rows: every per-token output and dlogits row is the same as
    # with per-chunk reductions, each row's stats are the same bits, and a
    # chunk's stats are the sum of its rows' (grpo_stats_sum).
    n_rows, T, V = 16, 48, 4096
    d = make_chunk(n_rows * T, V, torch.bfloat16, seed=14, n_rows=2, masked_frac=0.3)
    row_off = np.arange(0, n_rows * T + 1, T).astype(np.int64)
    tok_row = np.repeat(np.arange(n_rows, dtype=np.int32), T)
    adv = np.random.default_rng(2).normal(size=n_rows).astype(np.float32)
    g = d["g"]
    G = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    ws = ops.loss_workspace(n_rows * T, n_rows, DEV)
    dl_def = torch.empty_like(d["logits"])
    per_chunk = []
    for c in range(4):
        a, b = c * 4 * T, (c + 1) * 4 * T
        view = {k: ws[k][a:b] for k in ("logp", "lse", "entropy", "loss_tok", "kl_tok", "tok_flags")}
        ops.loss_fwd_bwd(d["logits"][a:b], g["target"][a:b], g["mask"][a:b], g["old"][a:b],
                         G(tok_row[a:b] - 4 * c), G(adv[4 * c:4 * c + 4]), G(row_off[4 * c:4 * c + 5] - a),
                         scale=1 / 500.0, dlogits=dl_def[a:b], ws=view, defer_stats=True)
        per_chunk.append(ops.loss_fwd_bwd(d["logits"][a:b], g["target"][a:b], g["mask"][a:b], g["old"][a:b],
                                          G(tok_row[a:b] - 4 * c), G(adv[4 * c:4 * c + 4]),
                                          G(row_off[4 * c:4 * c + 5] - a), scale=1 / 500.0))
    ops.loss_stats(ws, G(row_off), scale=1 / 500.0)
    torch.cuda.synchronize()
    assert torch.equal(dl_def, torch.cat([p["dlogits"] for p in per_chunk]))
    for k in ("logp", "entropy", "loss_tok", "tok_flags"):
        assert torch.equal(ws[k], torch.cat([p[k] for p in per_chunk])), k
    assert torch.equal(ws["row_stats"], torch.cat([p["row_stats"][:4] for p in per_chunk]))
    rows = ops.stats_to_dicts(ws["row_stats"])
    for c, p in enumerate(per_chunk):
        want = ops.stats_to_dicts(p["chunk_stats"])[0]
        got = ops.stats_sum(rows[4 * c:4 * c + 4])
        for k in want:
            assert got[k] == pytest.approx(want[k], rel=1e-12, abs=1e-12), k
    whole = ops.stats_to_dicts(ws["chunk_stats"])[0]
    assert whole["n_valid"] == int(d["mask"].sum())
    assert whole["loss_sum"] == pytest.approx(sum(r["loss_sum"] for r in rows), rel=1e-12)
    ref = oracle.loss_fwd_bwd(d["z64"], d["target"], d["mask"], d["old"].astype(np.float64),
                              adv.astype(np.float64)[tok_row], 1 / 500.0, want_dz=False)
    want_rows = oracle.row_stats(ref, row_off.tolist())
    for r, (gr, wr) in enumerate(zip(rows, want_rows)):
        assert gr["n_valid"] == wr["n_valid"] and gr["loss_sum"] == pytest.approx(wr["loss_sum"], rel=1e-4, abs=1e-6)


# (V, dtype, ld, in place): kernel shapes of the fused loss -- one wave per
# row, 512 x 12, 1024 x 19, the LDS tail, the re-read part (bf16), fp32 past
# the register file, and rows off 16-byte alignment updated in place
@pytest.mark.parametrize("V,dtype,ld,inplace", [(1024, torch.float32, 1024, False),
                                                (40960, torch.bfloat16, 40960, False),
                                                (151936, torch.bfloat16, 151936, False),
                                                (202048, torch.bfloat16, 202048, False),
                                                (256000, torch.bfloat16, 256000, False),
                                                (100000, torch.float32, 100000, False),
                                                (50257, torch.bfloat16, 50257, True),
                                                (32001, torch.bfloat16, 32007, True)])
def test_paired_forward_equals_the_fused_loss(V, dtype, ld, inplace):
    # grpo_logprob_fwd_paired runs the sums in the fused loss's lane partition:
    # logp, lse and entropy equal the fused call's bit for bit (the plain
    # forward pass streams rows past 1024 vectors and agrees only to float32
    # summation order).
    print(f"paired forward V={V} {dtype} ld={ld} inplace={inplace}", flush=True)
    n = 6 if V > 60000 else 24
    d = make_chunk(n, V, dtype, seed=V + 5, ld=ld)
    g = d["g"]
    f_logp, f_lse, f_ent = ops.logprob_fwd(d["logits"], g["target"], g["mask"], paired=True)
    ws = run_gpu(d, scale=0.05, dlogits="inplace" if inplace else "new")
    torch.cuda.synchronize()
    assert torch.equal(f_logp, ws["logp"])
    assert torch.equal(f_lse, ws["lse"])
    assert torch.equal(f_ent, ws["entropy"])
