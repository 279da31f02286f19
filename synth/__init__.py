"""Seeded synthetic inputs shaped like the workloads on the pages.

Shared by the tests, the bench and the smoke check.  This module draws
random numbers and lays them out; it holds none of the loss arithmetic (no
softmax, no ratio, no advantage, no packing): those live in the oracle and in
the HIP path, separately.

Workloads (sizes from the pages' GRPO settings: Qwen-family vocabularies,
2048-token completions, groups of 4 or 8, context-compaction rows):

* ``tiny``     8 prompts x group 4 = 32 rows, lengths U{8..64} right-padded to
               64, V = 1024 fp32 logits ~ N(0, 2), ~20 % of response tokens masked
               in spans of 2-6, mini 16 / micro 8.
* ``qwen``     16 x 4 = 64 rows, lengths U{128..2048} right-padded to 2048,
               V = 151936 bf16 logits ~ N(0, 3), micro 8 rows, one mini-batch.
* ``long``     16 x 8 = 128 rows, all 2048 tokens valid, same vocabulary,
               mini 64, micro 4.
* ``dynamic``  256 rows, lengths round(LogNormal(ln 512, 1.0)) clipped to
               [64, 8192], packed, token budget 16384, proxy L + L^2/4096.
* ``compact``  8 x 4 = 32 rollouts with U{1..5} segment rows of U{256..1024}
               tokens, Q = 4, micro 4 rows, hidden 2048 bf16 ~ N(0, 1), LM head
               [151936 x 2048] bf16 ~ N(0, 0.02).

Everywhere: targets U[0, V), rewards Bernoulli(0.5) per rollout, clip
epsilon 0.2, and a log-ratio perturbation N(0, 0.05) that the caller adds to
the current log-probs to form old log-probs.
"""

import math

import numpy as np

WORKLOADS = {
    "tiny": dict(n_prompts=8, group=4, T=64, V=1024, len_lo=8, len_hi=64,
                 logit_std=2.0, dtype="f32", mini=16, micro=8, mask="spans"),
    "qwen": dict(n_prompts=16, group=4, T=2048, V=151936, len_lo=128, len_hi=2048,
                 logit_std=3.0, dtype="bf16", mini=0, micro=8, mask="rightpad"),
    "long": dict(n_prompts=16, group=8, T=2048, V=151936, len_lo=2048, len_hi=2048,
                 logit_std=3.0, dtype="bf16", mini=64, micro=4, mask="rightpad"),
    "dynamic": dict(n_rows=256, V=151936, median=512, sigma=1.0, len_lo=64,
                    len_hi=8192, budget=16384, proxy_div=4096, logit_std=3.0,
                    dtype="bf16", fixed_micro=8, group=4),
    "compact": dict(n_prompts=8, group=4, seg_lo=1, seg_hi=5, tok_lo=256,
                    tok_hi=1024, Q=4, micro=4, H=2048, V=151936, h_std=1.0,
                    w_std=0.02),
}

EPS_CLIP = 0.2
LOGRATIO_STD = 0.05
_WORKLOAD_IDS = {"tiny": 1, "qwen": 2, "long": 3, "dynamic": 4, "compact": 5, "custom": 9}

_MASK64 = (1 << 64) - 1


def _splitmix64(x):
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def row_seed(seed, workload, row, stream=0):
    """Seed of one row's random stream: a function of (seed, workload, row,
    stream) only, so a row's values do not depend on how rows are packed."""
    h = _splitmix64(int(seed) & _MASK64)
    h = _splitmix64(h ^ _WORKLOAD_IDS.get(workload, 9))
    h = _splitmix64(h ^ (int(row) & _MASK64))
    h = _splitmix64(h ^ int(stream))
    return h & ((1 << 63) - 1)


def _span_mask(rng, length, frac=0.2, span_lo=2, span_hi=6):
    """Mask ~frac of a row's positions in random spans: until at least
    round(frac*length) positions are masked, pick a start U[0, length) and a
    span U{span_lo..span_hi} and mask [start, min(start+span, length))."""
    keep = np.ones(length, dtype=np.uint8)
    want = int(round(frac * length))
    while int((keep == 0).sum()) < want:
        start = int(rng.integers(0, length))
        span = int(rng.integers(span_lo, span_hi + 1))
        keep[start:min(start + span, length)] = 0
    return keep


def padded_batch(workload="tiny", seed=0, **over):
    """Host-side description of a right-padded batch.

    Returns a dict with ``n_rows``, ``T``, ``V``, ``lengths`` [rows],
    ``mask`` [rows*T] uint8, ``target`` [rows*T] int32, ``reward`` [rows]
    float32 (one rollout per row), ``logratio_noise`` [rows*T] float64,
    ``group``, ``mini``, ``micro``, ``logit_std``, ``dtype``.
    """
    cfg = dict(WORKLOADS[workload])
    cfg.update(over)
    rng = np.random.default_rng(row_seed(seed, workload, -1, 1))
    n_rows = cfg.get("n_rows", cfg["n_prompts"] * cfg["group"])
    T, V = cfg["T"], cfg["V"]
    lengths = rng.integers(cfg["len_lo"], cfg["len_hi"] + 1, size=n_rows).astype(np.int64)
    mask = np.zeros((n_rows, T), dtype=np.uint8)
    for r in range(n_rows):
        L = int(lengths[r])
        if cfg["mask"] == "spans":
            mask[r, :L] = _span_mask(rng, L)
        else:
            mask[r, :L] = 1
    target = rng.integers(0, V, size=(n_rows, T)).astype(np.int32)
    reward = (rng.random(n_rows) < 0.5).astype(np.float32)
    noise = rng.normal(0.0, LOGRATIO_STD, size=(n_rows, T))
    return dict(workload=workload, seed=seed, n_rows=n_rows, T=T, V=V, lengths=lengths,
                mask=mask.reshape(-1), target=target.reshape(-1), reward=reward,
                logratio_noise=noise.reshape(-1), group=cfg["group"],
                mini=cfg.get("mini", 0), micro=cfg.get("micro", 0),
                logit_std=cfg["logit_std"], dtype=cfg["dtype"])


def dynamic_lengths(seed=0, **over):
    """Row lengths of the dynamic-batching workload: round(LogNormal(ln median,
    sigma)) clipped to [len_lo, len_hi]."""
    cfg = dict(WORKLOADS["dynamic"])
    cfg.update(over)
    rng = np.random.default_rng(row_seed(seed, "dynamic", -1, 1))
    raw = rng.lognormal(math.log(cfg["median"]), cfg["sigma"], size=cfg["n_rows"])
    return np.clip(np.rint(raw), cfg["len_lo"], cfg["len_hi"]).astype(np.int64)


def dynamic_batch(seed=0, **over):
    """Host-side description of the dynamic-batching workload (unpacked: row
    r's tokens are a contiguous run of ``lengths[r]`` positions, all valid)."""
    cfg = dict(WORKLOADS["dynamic"])
    cfg.update(over)
    lengths = dynamic_lengths(seed, **over)
    rng = np.random.default_rng(row_seed(seed, "dynamic", -1, 2))
    n_tok = int(lengths.sum())
    return dict(workload="dynamic", seed=seed, n_rows=cfg["n_rows"], V=cfg["V"],
                lengths=lengths, target=rng.integers(0, cfg["V"], size=n_tok).astype(np.int32),
                mask=np.ones(n_tok, dtype=np.uint8),
                reward=(rng.random(cfg["n_rows"]) < 0.5).astype(np.float32),
                logratio_noise=rng.normal(0.0, LOGRATIO_STD, size=n_tok),
                group=cfg["group"], budget=cfg["budget"], proxy_div=cfg["proxy_div"],
                fixed_micro=cfg["fixed_micro"], logit_std=cfg["logit_std"], dtype=cfg["dtype"])


def compaction_batch(seed=0, **over):
    """Host-side description of the context-compaction workload: segment rows
    per rollout, tokens per segment row, rewards per rollout, targets and the
    log-ratio perturbation per real token (rollout-major segment order)."""
    cfg = dict(WORKLOADS["compact"])
    cfg.update(over)
    rng = np.random.default_rng(row_seed(seed, "compact", -1, 1))
    n_roll = cfg["n_prompts"] * cfg["group"]
    segs = rng.integers(cfg["seg_lo"], cfg["seg_hi"] + 1, size=n_roll).astype(np.int32)
    seg_len = rng.integers(cfg["tok_lo"], cfg["tok_hi"] + 1, size=int(segs.sum())).astype(np.int64)
    n_tok = int(seg_len.sum())
    return dict(workload="compact", seed=seed, n_groups=cfg["n_prompts"], group=cfg["group"],
                rows_per_rollout=segs, seg_len=seg_len,
                reward=(rng.random(n_roll) < 0.5).astype(np.float32),
                target=rng.integers(0, cfg["V"], size=n_tok).astype(np.int32),
                logratio_noise=rng.normal(0.0, LOGRATIO_STD, size=n_tok),
                Q=cfg["Q"], micro=cfg["micro"], H=cfg["H"], V=cfg["V"],
                h_std=cfg["h_std"], w_std=cfg["w_std"])


def fill_normal_rows(out, row_ids, row_start, row_len, std, seed, workload, stream=0):
    """Fill ``out`` (a torch tensor [n_tok, V], any float dtype, any device)
    with N(0, std^2) values drawn row by row: the positions
    ``row_start[k] : row_start[k] + row_len[k]`` get the stream of row
    ``row_ids[k]``, seeded by ``row_seed``.  Values are drawn in float32 and
    rounded to ``out.dtype`` by torch (nearest-even)."""
    import torch
    dev = out.device
    V = out.shape[1]
    for rid, st, ln in zip(row_ids, row_start, row_len):
        st, ln = int(st), int(ln)
        if ln == 0:
            continue
        g = torch.Generator(device=dev)
        g.manual_seed(row_seed(seed, workload, int(rid), stream))
        step = max(1, (1 << 28) // V)       # bound the float32 staging buffer
        for a in range(0, ln, step):
            b = min(ln, a + step)
            vals = torch.randn((b - a, V), generator=g, device=dev, dtype=torch.float32)
            vals.mul_(std)
            out[st + a:st + b].copy_(vals)
    return out
