"""Throughput of one token-level GRPO loss step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload qwen|long|tiny] [--gpus 1]

A step is one pass of the hot path over one collected batch whose logits are
already resident in HBM: the fixed mini/micro plan and the group advantages
(host, libgrpo), the step's valid-token count N (device), then for every
micro-batch chunk the fused log-softmax + clipped-surrogate forward/backward
that reads the chunk's logits once and writes dlogits once (device), and the
token-weighted roll-up of the chunk statistics (host accumulator).

Prints one JSON line: valid tokens/s, the dominant kernel's achieved HBM
bandwidth against the 8 TB/s peak (algorithmic bytes over its launch time,
timed with HIP events on the stream it runs on), and the CPU oracle's
throughput on a bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "valid tokens/s, fused log-softmax+GRPO loss fwd/bwd; % of HBM peak"
HBM_PEAK_GBS = 8000.0
PER_TOKEN_SCALAR_READ = 4 + 4 + 4      # target, old log-prob, row index (valid tokens)
PER_TOKEN_SCALAR_ALL = 1 + 4 * 4 + 1   # mask read; logp, lse, entropy, loss written; flags written

WORKLOAD_TEXT = {
    "qwen": "64 rows (16 prompts x group 4), response lengths U{128..2048} right-padded to 2048, "
            "vocab 151936, bf16 logits ~N(0,3), micro 8 rows -> 8 chunks, one mini-batch",
    "long": "128 rows (16 prompts x group 8) x 2048 tokens all valid, vocab 151936, bf16 logits ~N(0,3), "
            "mini 64 rows (2 optimizer steps), micro 4 rows -> 32 chunks",
    "tiny": "32 rows (8 prompts x group 4), lengths U{8..64} padded to 64, vocab 1024, fp32 logits ~N(0,2), "
            "~20% masked in spans, mini 16 / micro 8 -> 2x2 chunks",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle sample (0 disables the cpu_baseline leg)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for counter calibration)")
    return ap.parse_args()


def build_batch(wl, seed, torch, ops):
    """Resident synthetic batch for workload ``wl`` (logits generated on the GPU)."""
    from synth import fill_normal_rows, padded_batch
    b = padded_batch(wl, seed=seed)
    n_rows, T, V = b["n_rows"], b["T"], b["V"]
    dt = torch.bfloat16 if b["dtype"] == "bf16" else torch.float32
    dev = "cuda"
    n_tok = n_rows * T
    logits = torch.empty((n_tok, V), dtype=dt, device=dev)
    fill_normal_rows(logits, range(n_rows), [r * T for r in range(n_rows)], [T] * n_rows, b["logit_std"], seed, wl)
    G = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    target, mask = G(b["target"]), G(b["mask"])
    # pi_old: the ahead pass over the collected batch, then the log-ratio
    # perturbation that stands in for the policy having moved since rollout
    logp, _, _ = ops.logprob_fwd(logits, target, mask, want_lse=False, want_entropy=False)
    old = (logp.double() + G(b["logratio_noise"])).float()
    del logp
    dlogits = torch.empty_like(logits)
    return dict(b=b, logits=logits, target=target, mask=mask, old=old, dlogits=dlogits, dtype=dt)


class Step:
    """One loss step over the resident batch; the same work every call."""

    def __init__(self, data, torch, ops):
        self.torch, self.ops, self.d = torch, ops, data
        b = data["b"]
        self.n_rows, self.T, self.V = b["n_rows"], b["T"], b["V"]
        self.reward = b["reward"]
        dev = "cuda"
        n_mini, n_micro, mini_rows, micro_rows = ops.plan_fixed(self.n_rows, b["group"], b["mini"], b["micro"])
        self.micro_rows = micro_rows
        self.row_off = torch.arange(0, micro_rows * self.T + 1, self.T, dtype=torch.int64, device=dev)
        self.tok_row = ops.tok_row(self.row_off, micro_rows * self.T)
        self.ws = ops.loss_workspace(micro_rows * self.T, micro_rows, dev)
        self.N = torch.empty(max(n_mini, 1), dtype=torch.int64, device=dev)
        self.adv_host = torch.empty(self.n_rows, dtype=torch.float32).pin_memory()
        self.adv_dev = torch.empty(self.n_rows, dtype=torch.float32, device=dev)
        self.stats_dev = torch.empty((n_mini * n_micro, ops.STATS_BYTES), dtype=torch.uint8, device=dev)
        self.stats_host = torch.empty((n_mini * n_micro, ops.STATS_BYTES), dtype=torch.uint8).pin_memory()
        self.events = []

    def __call__(self, record=False):
        torch, ops, d = self.torch, self.ops, self.d
        b = d["b"]
        T = self.T
        plan = ops.plan_fixed(self.n_rows, b["group"], b["mini"], b["micro"])
        n_mini, n_micro, mini_rows, micro_rows = plan
        adv = ops.group_advantage(self.reward, b["group"])            # one rollout per row here
        self.adv_host.numpy()[:] = adv
        self.adv_dev.copy_(self.adv_host, non_blocking=True)
        results = []
        k = 0
        for i in range(n_mini):
            r0 = i * mini_rows
            ops.count_valid(d["mask"][r0 * T:(r0 + mini_rows) * T], out=self.N[i:i + 1])
            for j in range(n_micro):
                a, e = ops.plan_chunk(self.n_rows, mini_rows, micro_rows, i, j)
                t0, t1 = a * T, e * T
                if record:
                    ev0 = torch.cuda.Event(enable_timing=True)
                    ev1 = torch.cuda.Event(enable_timing=True)
                    ev0.record()
                self.ws["chunk_stats"] = self.stats_dev[k:k + 1]
                ops.loss_fwd_bwd(d["logits"][t0:t1], d["target"][t0:t1], d["mask"][t0:t1], d["old"][t0:t1],
                                 self.tok_row, self.adv_dev[a:e], self.row_off, scale=1.0,
                                 denom=self.N[i:i + 1], dlogits=d["dlogits"][t0:t1], ws=self.ws)
                if record:
                    ev1.record()
                    self.events.append((ev0, ev1, t0, t1))
                k += 1
        self.stats_host.copy_(self.stats_dev, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        stats = ops.stats_to_dicts(self.stats_host.numpy())
        k = 0
        for i in range(n_mini):
            acc = ops.Accumulator(n_micro)
            for j in range(n_micro):
                acc.add(stats[k])
                k += 1
            results.append(acc.finalize())
        return results


def algorithmic_bytes(mask_np, t0, t1, V, b_in, b_out):
    m = mask_np[t0:t1]
    nv = int(m.sum())
    nm = (t1 - t0) - nv
    return nv * (V * (b_in + b_out) + PER_TOKEN_SCALAR_READ) + nm * V * b_out + (t1 - t0) * PER_TOKEN_SCALAR_ALL


def cpu_baseline(data, budget_s):
    """The oracle, as it stands, on the first valid tokens of the batch until
    ``budget_s`` seconds of compute have run (single process)."""
    import oracle
    torch = __import__("torch")
    b = data["b"]
    mask = b["mask"]
    valid = np.nonzero(mask)[0]
    rng = np.random.default_rng(1)
    adv_rows = rng.normal(0, 1, b["n_rows"])
    done, t_used = 0, 0.0
    block = 16
    pos = 0
    while t_used < budget_s and pos < len(valid):
        idx = valid[pos:pos + block]
        pos += block
        z = data["logits"][torch.as_tensor(idx, device="cuda")].double().cpu().numpy()
        y = b["target"][idx]
        m = np.ones(len(idx), np.uint8)
        old = oracle.logprob_fwd(z, y, m)["logp"] + b["logratio_noise"][idx]
        adv = adv_rows[idx // b["T"]]
        t0 = time.perf_counter()
        oracle.loss_fwd_bwd(z, y, m, old, adv, 1.0 / max(1, len(valid)))
        t_used += time.perf_counter() - t0
        done += len(idx)
    return {"value": done / t_used, "unit": "valid tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} valid tokens of the benched batch (V={b['V']}, float64 numpy, one process), "
                      f"{t_used:.1f} s of compute"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from grpo_token_level_amd import ops
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    ops.version()                      # fails loudly if libgrpo.so is missing
    wl = args.workload
    data = build_batch(wl, args.seed, torch, ops)
    step = Step(data, torch, ops)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    step.events.clear()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        res = step(record=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    b = data["b"]
    n_valid = int(np.sum(b["mask"]))
    ms = 1e3 * wall / args.steps
    value = n_valid / (wall / args.steps)
    # dominant kernel: the fused loss launch per chunk (token kernel + two tiny
    # stats reductions inside the same event pair)
    b_in = 2 if data["dtype"] == torch.bfloat16 else 4
    b_out = b_in
    tot_bytes, tot_ms = 0, 0.0
    for ev0, ev1, t0_, t1_ in step.events:
        tot_ms += ev0.elapsed_time(ev1)
        tot_bytes += algorithmic_bytes(b["mask"], t0_, t1_, b["V"], b_in, b_out)
    launches = len(step.events)
    achieved = (tot_bytes / launches) / (tot_ms / launches * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "valid tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{wl}: {WORKLOAD_TEXT[wl]}", "logits_dtype": "bf16" if b_in == 2 else "fp32",
                   "rows": b["n_rows"], "T": b["T"], "V": b["V"], "valid_tokens": n_valid,
                   "chunks_per_step": launches // args.steps, "step_loss": res[0]["loss"] if res[0] else None},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "tok_reg_kernel (fused loss fwd+bwd), per chunk launch",
                     "algorithmic_bytes_per_launch": tot_bytes // launches,
                     "avg_launch_ms": round(tot_ms / launches, 4)},
    }
    # context: a plain device-to-device copy of one chunk's bytes (read V*2 +
    # write V*2 per token), timed the same way, after the timed region
    t0_, t1_ = step.events[0][2], step.events[0][3]
    src, dst = data["logits"][t0_:t1_], data["dlogits"][t0_:t1_]
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    c0.record()
    for _ in range(3):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    out["roofline"]["device_copy_GBs"] = round(3 * 2 * src.numel() * src.element_size() / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)
    if wl == "qwen":
        from grpo_token_level_amd.prof_summary import load_traffic
        rec = load_traffic(os.path.join(ROOT, "profiles", "fused_loss_qwen_pmc.txt"))
        if rec is not None:
            out["roofline"]["traffic"] = rec["traffic_bytes_per_launch"]
    if args.copy_calibration:
        # known-size plain copy for the byte counters: 1 GiB read, 1 GiB written
        x = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
        y = torch.empty_like(x)
        torch.bitwise_not(x, out=y)
        torch.cuda.synchronize()
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(data, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
