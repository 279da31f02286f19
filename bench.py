"""Throughput of one token-level GRPO loss step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload long|qwen|tiny|dynamic|compact] [--gpus 1]

A step is one pass of the hot path over one collected batch whose inputs are
already resident in HBM:

* padded workloads (long = default: the largest configuration, 128 rows x
  2048 tokens at group 8; qwen; tiny): the fixed mini/micro plan and
  the group advantages (host, libgrpo), N per mini-batch (device), then per
  micro-batch chunk the fused log-softmax + clipped-surrogate forward/backward
  that reads the chunk's logits once and writes dlogits once (device), and the
  token-weighted roll-up of the chunk statistics (host accumulator);
* dynamic: the same with the token-budget packing plan (host) and its boxes;
* compact: the context-compaction plan, advantages copied to segment rows,
  W^T, then per 4-row chunk the fused LM-head loss (bf16 MFMA GEMMs) with dW
  accumulated over the chunks.

Prints one JSON line: valid tokens/s, the dominant kernel's achieved
bandwidth (or MFMA rate) against the chip's published peak, measured with HIP
events on the stream the kernels run on, and the CPU oracle's throughput on
a bounded sample of the same workload.
"""

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "valid tokens/s, fused log-softmax+GRPO loss fwd/bwd; % of HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PER_TOKEN_SCALAR_READ = 4 + 4 + 4      # target, old log-prob, row index (valid tokens)
PER_TOKEN_SCALAR_ALL = 1 + 4 * 4 + 1   # mask read; logp, lse, entropy, loss written; flags written

WORKLOAD_TEXT = {
    "qwen": "64 rows (16 prompts x group 4), response lengths U{128..2048} right-padded to 2048, "
            "vocab 151936, bf16 logits ~N(0,3), micro 8 rows -> 8 chunks, one mini-batch",
    "long": "128 rows (16 prompts x group 8) x 2048 tokens all valid, vocab 151936, bf16 logits ~N(0,3), "
            "mini 64 rows (2 optimizer steps), micro 4 rows -> 32 chunks",
    "tiny": "32 rows (8 prompts x group 4), lengths U{8..64} padded to 64, vocab 1024, fp32 logits ~N(0,2), "
            "~20% masked in spans, mini 16 / micro 8 -> 2x2 chunks",
    "dynamic": "256 rows, lengths round(LogNormal(ln 512, 1.0)) clipped to [64, 8192], all valid, packed, "
               "vocab 151936 bf16 ~N(0,3), token budget 16384 per micro-batch, proxy L + L^2/4096",
    "compact": "8 prompts x group 4 rollouts, U{1..5} segment rows of U{256..1024} tokens, groups padded to a "
               "multiple of Q=4 with masked copies, micro 4 rows, hidden 2048 bf16 ~N(0,1), "
               "LM head [151936 x 2048] bf16 ~N(0,0.02)",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle sample (0 disables the cpu_baseline leg)")
    ap.add_argument("--terms", action="store_true",
                    help="padded workloads: seq-mean-token-mean aggregation with an entropy bonus (0.01) and a k3 "
                         "KL term (0.05) against a reference log-prob (the step's extra-term variant)")
    ap.add_argument("--paired", action="store_true",
                    help="with --ahead: record pi_old with the paired forward pass (the fused loss's lane "
                         "partition: the ratio is exactly 1 on unchanged logits)")
    ap.add_argument("--ahead", action="store_true",
                    help="padded workloads: when the batch drives more than one optimizer step, run the ahead "
                         "pass (pi_old recorded per chunk into the old-log-prob cache) inside the timed step and "
                         "train against the replayed records")
    ap.add_argument("--epochs", type=int, default=1,
                    help="padded workloads: inner epochs (mu) over the collected batch in one timed step")
    ap.add_argument("--shuffle", action="store_true",
                    help="padded workloads: reshuffle the rows every epoch (seeded); chunks read the batch through "
                         "tok_src")
    ap.add_argument("--cpu-pool-seconds", type=float, default=8.0,
                    help="wall seconds of the oracle over a process pool (0: skip)")
    ap.add_argument("--vocab", type=int, default=0,
                    help="padded workloads: vocabulary size in place of the workload's own (rows past the register "
                         "file take the LDS-tail configuration, beyond 229 376 or off 16-byte alignment the "
                         "streaming kernel)")
    ap.add_argument("--replicate", type=int, default=1,
                    help="tiny workload: the same row shape and distributions replicated R times as one batch in "
                         "one launch (the HBM reading of the launch-bound workload)")
    ap.add_argument("--graph", action="store_true",
                    help="padded workloads: capture the step's device work in a HIP graph once and replay it "
                         "(the launch-bound tiny step); the roofline then uses graph replay time / launches")
    ap.add_argument("--keep-z", action="store_true",
                    help="compact workload: the LM head keeps each chunk's fp32 logits for pass 2 "
                         "(GRPO_LMHEAD_KEEP_Z: one [tokens x V] matrix per chunk in place of the recompute)")
    ap.add_argument("--defer-dw", action="store_true",
                    help="compact workload: each chunk appends h^T and dz^T to a dW window and one GEMM per step "
                         "adds the step's dW (GRPO_LMHEAD_DEFER_DW + grpo_lmhead_dw_flush)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for counter calibration)")
    return ap.parse_args()


def _g(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


class Timed:
    """HIP-event brackets around the dominant launches of the timed steps."""

    def __init__(self, torch):
        self.torch = torch
        self.rec = []
        self.on = False
        self.pending = None

    def begin(self):
        if not self.on:
            return None
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def end(self, e0, units, launches=1):
        if e0 is None:
            return
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.rec.append((e0, e1, units, launches))

    # The binding calls mark() (its on_launch hook) after marshalling a call's
    # arguments, right before the library call, so that the window brackets
    # the launch and not the Python work before it (when the GPU has drained
    # its queue, as ahead of the single launch of a replicated tiny step, that
    # work would otherwise count as kernel time).
    def mark(self):
        self.pending = self.begin()

    def end_marked(self, units, launches=1):
        self.end(self.pending, units, launches)
        self.pending = None

    def totals(self):
        ms = sum(a.elapsed_time(b) for a, b, _, _ in self.rec)
        units = sum(u for _, _, u, _ in self.rec)
        return ms, units, sum(n for _, _, _, n in self.rec)


# ---------------------------------------------------------------- padded / dynamic: fused loss

def chunk_bytes(mask_np, V, b_in, b_out, extra_per_valid=0):
    """Algorithmic bytes of one fused launch: valid tokens read V*b_in and write
    V*b_out, masked tokens write V*b_out (zeros), plus the per-token scalars
    (``extra_per_valid``: the reference log-prob read and KL write of the
    extra-term variant)."""
    nv = int(mask_np.sum())
    nm = len(mask_np) - nv
    return (nv * (V * (b_in + b_out) + PER_TOKEN_SCALAR_READ + extra_per_valid) + nm * V * b_out
            + len(mask_np) * PER_TOKEN_SCALAR_ALL)


class PaddedStep:
    """Fixed-plan step over a right-padded batch: mu inner epochs (1 by
    default) of n_mini optimizer windows of n_micro chunks, optionally
    reshuffled per epoch (the chunks then read the batch through tok_src),
    optionally with the ahead pass and the extra loss terms."""

    ENT_COEF, KL_COEF = 0.01, 0.05

    def __init__(self, wl, seed, torch, ops, timed, terms=False, ahead=False, paired=False, epochs=1, shuffle=False,
                 over=None, graph=False):
        from synth import fill_normal_rows, padded_batch
        self.torch, self.ops, self.timed = torch, ops, timed
        self.terms = terms
        self.graph, self.graph_obj = graph, None
        self.ahead_timed = Timed(torch)
        b = self.b = padded_batch(wl, seed=seed, **(over or {}))
        n_rows, T, V = b["n_rows"], b["T"], b["V"]
        self.V = V
        self.dt = torch.bfloat16 if b["dtype"] == "bf16" else torch.float32
        n_tok = n_rows * T
        self.logits = torch.empty((n_tok, V), dtype=self.dt, device="cuda")
        fill_normal_rows(self.logits, range(n_rows), [r * T for r in range(n_rows)], [T] * n_rows, b["logit_std"],
                         seed, wl)
        self.target, self.mask = _g(torch, b["target"]), _g(torch, b["mask"])
        # pi_old: the ahead pass over the collected batch, then the log-ratio
        # perturbation that stands in for the policy having moved since rollout
        logp, _, _ = ops.logprob_fwd(self.logits, self.target, self.mask, want_lse=False, want_entropy=False)
        self.old = (logp.double() + _g(torch, b["logratio_noise"])).float()
        if terms:
            # a reference policy a little further away: old log-probs plus the same noise again
            self.ref = (self.old.double() + _g(torch, b["logratio_noise"])).float()
        del logp
        self.dlogits = torch.empty_like(self.logits)
        ep = ops.plan_epochs(n_rows, b["group"], b["mini"], b["micro"], mu=epochs, shuffle=shuffle, seed=seed + 1)
        self.ep, self.mu, self.shuffle = ep, epochs, shuffle
        n_mini, n_micro, mini_rows, micro_rows = ep["n_mini"], ep["n_micro"], ep["mini_rows"], ep["micro_rows"]
        self.perm_dev = _g(torch, ep["perm"])
        self.batch_off = torch.arange(0, n_tok + 1, T, dtype=torch.int64, device="cuda")
        self.row_off = torch.arange(0, micro_rows * T + 1, T, dtype=torch.int64, device="cuda")
        self.mini_off = torch.arange(0, mini_rows * T + 1, T, dtype=torch.int64, device="cuda")
        self.n_seq = torch.empty(n_mini, dtype=torch.int64, device="cuda")
        self.w_row = torch.empty(mini_rows, dtype=torch.float32, device="cuda")
        self.tok_row = ops.tok_row(self.row_off, micro_rows * T)
        # per-token outputs of a whole mini-batch: the chunks write views of it
        # with their row reductions deferred, and one grpo_loss_stats call per
        # optimizer window reduces every row of the window
        self.ws = ops.loss_workspace(mini_rows * T, mini_rows, "cuda")
        self.mini_rows, self.micro_rows, self.n_micro = mini_rows, micro_rows, n_micro
        self.chunk_tokens = micro_rows * T
        self.N = torch.empty(n_mini, dtype=torch.int64, device="cuda")
        self.adv_host = torch.empty(n_rows, dtype=torch.float32).pin_memory()
        self.adv_dev = torch.empty(n_rows, dtype=torch.float32, device="cuda")
        if shuffle:
            self.mini_src = torch.empty(mini_rows * T, dtype=torch.int64, device="cuda")
            self.mini_mask = torch.empty(mini_rows * T, dtype=torch.uint8, device="cuda")
            self.tok_src = torch.empty(micro_rows * T, dtype=torch.int64, device="cuda")
            self.adv_chunk = torch.empty(micro_rows, dtype=torch.float32, device="cuda")
        n_win = epochs * n_mini
        self.stats_dev = torch.empty((n_win * mini_rows, ops.STATS_BYTES), dtype=torch.uint8, device="cuda")
        self.stats_host = torch.empty((n_win * mini_rows, ops.STATS_BYTES), dtype=torch.uint8).pin_memory()
        self.win_stats = torch.empty((n_win, ops.STATS_BYTES), dtype=torch.uint8, device="cuda")
        b_in = 2 if self.dt == torch.bfloat16 else 4
        self.chunk_units = {}
        for e in range(epochs):
            for i in range(n_mini):
                for j in range(n_micro):
                    rows = ep["perm"][e][i * mini_rows + j * micro_rows:][:micro_rows]
                    m = np.concatenate([b["mask"][r * T:(r + 1) * T] for r in rows])
                    self.chunk_units[(e, i, j)] = chunk_bytes(m, V, b_in, b_in, 8 if terms else 0)
        self.n_valid = int(np.sum(b["mask"])) * epochs
        self.logits_dtype = "bf16" if b_in == 2 else "fp32"
        self.graph_units = sum(self.chunk_units.values())
        self.graph_launches = len(self.chunk_units)
        # the ahead pass runs only where the gate asks for it (more than one
        # optimizer step per collected batch: n_mini windows per epoch, mu epochs)
        self.ahead = ahead and ops.needs_ahead_pass(n_mini * epochs)
        self.paired = paired
        if self.ahead:
            self.cache = ops.OldLogprobCache(n_mini * n_micro,
                                             torch.empty(n_rows * T, dtype=torch.float32, device="cuda"))
            self.ahead_units = {}
            for i in range(n_mini):
                for j in range(n_micro):
                    a, e_ = ops.plan_chunk(n_rows, mini_rows, micro_rows, i, j)
                    self.ahead_units[(i, j)] = int(np.sum(b["mask"][a * T:e_ * T])) * V * b_in

    def __call__(self):
        self._host_prep()
        if not self.graph:
            self._device()
        elif self.graph_obj is None:
            # first call: run eagerly (warm-up), then capture the device work once
            self._device()
            self.torch.cuda.synchronize()
            self.graph_obj = self.torch.cuda.CUDAGraph()
            with self.torch.cuda.graph(self.graph_obj):
                self._device()
            self.torch.cuda.synchronize()
        else:
            ev = self.timed.begin()
            self.graph_obj.replay()
            self.timed.end(ev, self.graph_units, self.graph_launches)
        return self._finish()

    def _host_prep(self):
        b = self.b
        self.adv_host.numpy()[:] = self.ops.group_advantage(b["reward"], b["group"])    # one rollout per row
        self.adv_dev.copy_(self.adv_host, non_blocking=True)

    def _device(self):
        torch, ops, b, T = self.torch, self.ops, self.b, self.b["T"]
        n_rows = b["n_rows"]
        n_mini, n_micro, mini_rows, micro_rows = ops.plan_fixed(n_rows, b["group"], b["mini"], b["micro"])
        if self.ahead:
            # [P1] the ahead walk: pi_old of every chunk, recorded before training (batch order)
            self.cache.reset()
            for i in range(n_mini):
                for j in range(n_micro):
                    a, e = ops.plan_chunk(n_rows, mini_rows, micro_rows, i, j)
                    self.cache.record(self.logits[a * T:e * T], self.target[a * T:e * T], self.mask[a * T:e * T],
                                      paired=self.paired, on_launch=self.ahead_timed.mark)
                    self.ahead_timed.end_marked(self.ahead_units[(i, j)])
        k = 0
        for ep in range(self.mu):
            if self.ahead and not self.shuffle and ep > 0:
                self.cache.rewind()                      # the next epoch replays the records in order
            for i in range(n_mini):
                if self.shuffle:
                    rows_mini = self.perm_dev[ep, i * mini_rows:(i + 1) * mini_rows]
                    ops.chunk_tok_src(self.batch_off, rows_mini, self.mini_off, out=self.mini_src)
                    mini_mask = ops.gather(self.mask, self.mini_src, out=self.mini_mask)
                else:
                    mini_mask = self.mask[i * mini_rows * T:(i + 1) * mini_rows * T]
                ops.count_valid(mini_mask, out=self.N[i:i + 1])
                if self.terms:
                    ops.count_rows(mini_mask, self.mini_off, out=self.n_seq[i:i + 1])
                    ops.row_weights(mini_mask, self.mini_off, ops.C.AGG_SEQ_MEAN_TOKEN_MEAN, self.n_seq[i:i + 1],
                                    out=self.w_row)
                w = ep * n_mini + i
                for j in range(n_micro):
                    r0 = j * micro_rows                      # the chunk's rows within the mini-batch
                    view = {key: self.ws[key][r0 * T:(r0 + micro_rows) * T]
                            for key in ("logp", "lse", "entropy", "loss_tok", "kl_tok", "tok_flags")}
                    if self.terms:
                        kw = dict(scale=1.0, row_weight=self.w_row[r0:r0 + micro_rows],
                                  ent_coef=self.ENT_COEF, kl_coef=self.KL_COEF, kl_type=ops.C.KL_K3)
                    else:
                        kw = dict(scale=1.0, denom=self.N[i:i + 1])
                    if self.shuffle:
                        rows = self.perm_dev[ep, i * mini_rows + r0:i * mini_rows + r0 + micro_rows]
                        ops.chunk_tok_src(self.batch_off, rows, self.row_off, out=self.tok_src)
                        ops.gather(self.adv_dev, rows, out=self.adv_chunk)
                        old = self.cache.buf if self.ahead else self.old
                        if self.terms:
                            kw["ref_logp"] = self.ref
                        ops.loss_fwd_bwd(self.logits, self.target, self.mask, old, self.tok_row, self.adv_chunk,
                                         self.row_off, dlogits=self.dlogits, ws=view, tok_src=self.tok_src,
                                         defer_stats=True, on_launch=self.timed.mark, **kw)
                    else:
                        a, e = ops.plan_chunk(n_rows, mini_rows, micro_rows, i, j)
                        t0, t1 = a * T, e * T
                        old = self.cache.replay(t1 - t0) if self.ahead else self.old[t0:t1]
                        if self.terms:
                            kw["ref_logp"] = self.ref[t0:t1]
                        ops.loss_fwd_bwd(self.logits[t0:t1], self.target[t0:t1], self.mask[t0:t1], old,
                                         self.tok_row, self.adv_dev[a:e], self.row_off, dlogits=self.dlogits[t0:t1],
                                         ws=view, defer_stats=True, on_launch=self.timed.mark, **kw)
                    self.timed.end_marked(self.chunk_units[(ep, i, j)])
                    k += 1
                # the window's row reductions in one call (rows in mini-batch order)
                self.ws["row_stats"] = self.stats_dev[w * mini_rows:(w + 1) * mini_rows]
                self.ws["chunk_stats"] = self.win_stats[w:w + 1]
                if self.terms:
                    ops.loss_stats(self.ws, self.mini_off, scale=1.0, row_weight=self.w_row, with_kl=True,
                                   ent_coef=self.ENT_COEF, kl_coef=self.KL_COEF)
                else:
                    ops.loss_stats(self.ws, self.mini_off, scale=1.0, denom=self.N[i:i + 1])

    def _finish(self):
        torch, ops, b = self.torch, self.ops, self.b
        n_mini, n_micro, _, _ = ops.plan_fixed(b["n_rows"], b["group"], b["mini"], b["micro"])
        self.stats_host.copy_(self.stats_dev, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        base = self.stats_host.data_ptr()
        m, u, sb = self.mini_rows, self.micro_rows, ops.STATS_BYTES
        out = []
        for w in range(self.mu * n_mini):
            acc = ops.Accumulator(n_micro)
            for j in range(n_micro):              # a chunk's stats: the sum of its rows'
                acc.add_rows_at(base + (w * m + j * u) * sb, u)
            out.append(acc.finalize())
        return out

    def llc_note(self):
        ws = self.logits.numel() * self.logits.element_size() * 2
        if ws > 256e6:
            return f"cold: a step touches {ws / 1e9:.1f} GB of logits and dlogits, beyond the 256 MB last-level cache"
        return f"warm: a step touches {ws / 1e6:.1f} MB of logits and dlogits, within the 256 MB last-level cache"

    def copy_context(self):
        """The yardstick's streaming copy of one chunk's bytes, timed like the
        kernel: the bandwidth a plain copy of the same bytes gets."""
        import yardstick
        return self._stream_rate(yardstick.COPY)

    def read_context(self):
        """The same for a plain read of one chunk's logits (the ahead pass's yardstick)."""
        import yardstick
        return self._stream_rate(yardstick.READ)

    def _stream_rate(self, mode):
        import yardstick
        torch = self.torch
        n = self.chunk_tokens
        src = self.logits[:n]
        dst = self.dlogits[:n] if mode == yardstick.COPY else None
        nbytes = src.numel() * src.element_size()
        dst = yardstick.stream(mode, src, dst, nbytes)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(3):
            yardstick.stream(mode, src, dst, nbytes)
        c1.record()
        torch.cuda.synchronize()
        moved = nbytes * (2 if mode == yardstick.COPY else 1)
        return 3 * moved / (c0.elapsed_time(c1) * 1e-3) / 1e9

    def sample(self, n, start=0):
        """(z float64 [n, V], target, drift, advantage) of valid tokens start .. start+n."""
        torch, b = self.torch, self.b
        idx = np.nonzero(b["mask"])[0][start:start + n]
        z = self.logits[torch.as_tensor(idx, device="cuda")].double().cpu().numpy()
        adv = np.random.default_rng(1).normal(0, 1, b["n_rows"])[idx // b["T"]]
        return z, b["target"][idx], b["logratio_noise"][idx], adv


class DynamicStep(PaddedStep):
    """Token-budget packing: rows laid out box by box, one launch per box."""

    def __init__(self, wl, seed, torch, ops, timed):
        from synth import dynamic_batch, fill_normal_rows
        self.torch, self.ops, self.timed = torch, ops, timed
        b = self.b = dynamic_batch(seed=seed)
        L = b["lengths"].astype(np.int64)
        V = self.V = b["V"]
        self.dt = torch.bfloat16
        plan = ops.plan_dynamic(L, b["budget"], b["proxy_div"])
        order = plan["order"]
        offB = ops.row_offsets(L, order)
        offA = np.concatenate([[0], np.cumsum(L)])
        perm = np.concatenate([np.arange(offA[r], offA[r + 1]) for r in order])
        n_tok = int(offA[-1])
        self.logits = torch.empty((n_tok, V), dtype=self.dt, device="cuda")
        fill_normal_rows(self.logits, order, offB[:-1], L[order], b["logit_std"], seed, "dynamic")
        self.target = _g(torch, b["target"][perm])
        self.mask = _g(torch, b["mask"][perm])
        logp, _, _ = ops.logprob_fwd(self.logits, self.target, self.mask, want_lse=False, want_entropy=False)
        self.old = (logp.double() + _g(torch, b["logratio_noise"][perm])).float()
        del logp
        self.dlogits = torch.empty_like(self.logits)
        bin_tok = [int(offB[plan["bin_off"][k + 1]] - offB[plan["bin_off"][k]]) for k in range(plan["n_bins"])]
        # per-token outputs of the whole batch (one optimizer window): the boxes
        # write views of it with their row reductions deferred, then one
        # grpo_loss_stats call reduces every row (packed order)
        self.ws = ops.loss_workspace(n_tok, len(L), "cuda")
        self.chunk_tokens = max(bin_tok)
        self.tok_row = torch.empty(max(bin_tok), dtype=torch.int32, device="cuda")
        self.N = torch.empty(1, dtype=torch.int64, device="cuda")
        n_rows = len(L)
        self.meta_host = torch.empty(n_rows + plan["n_bins"] + 8, dtype=torch.int64).pin_memory()
        self.meta_dev = torch.empty(n_rows + plan["n_bins"] + 8, dtype=torch.int64, device="cuda")
        self.adv_host = torch.empty(n_rows, dtype=torch.float32).pin_memory()
        self.adv_dev = torch.empty(n_rows, dtype=torch.float32, device="cuda")
        self.stats_dev = torch.empty((n_rows, ops.STATS_BYTES), dtype=torch.uint8, device="cuda")
        self.stats_host = torch.empty((n_rows, ops.STATS_BYTES), dtype=torch.uint8).pin_memory()
        self.win_stats = torch.empty((1, ops.STATS_BYTES), dtype=torch.uint8, device="cuda")
        self.offB_host = torch.empty(n_rows + 1, dtype=torch.int64).pin_memory()
        self.offB_dev = torch.empty(n_rows + 1, dtype=torch.int64, device="cuda")
        self.mask_np = b["mask"][perm]
        self.n_valid = int(np.sum(b["mask"]))
        self.logits_dtype = "bf16"

    def __call__(self):
        torch, ops, b = self.torch, self.ops, self.b
        L = b["lengths"].astype(np.int64)
        n_rows = len(L)
        plan = ops.plan_dynamic(L, b["budget"], b["proxy_div"])
        order, bin_off = plan["order"], plan["bin_off"]
        offB = ops.row_offsets(L, order)
        # per box: its rows' token offsets relative to the box start
        local = np.empty(n_rows + plan["n_bins"], np.int64)
        starts = []
        p = 0
        for k in range(plan["n_bins"]):
            a, e = int(bin_off[k]), int(bin_off[k + 1])
            starts.append(p)
            local[p:p + e - a + 1] = offB[a:e + 1] - offB[a]
            p += e - a + 1
        self.meta_host.numpy()[:p] = local[:p]
        self.meta_dev[:p].copy_(self.meta_host[:p], non_blocking=True)
        adv = ops.group_advantage(b["reward"], b["group"])
        self.adv_host.numpy()[:] = adv[order]
        self.adv_dev.copy_(self.adv_host, non_blocking=True)
        self.offB_host.numpy()[:] = offB
        self.offB_dev.copy_(self.offB_host, non_blocking=True)
        ops.count_valid(self.mask, out=self.N)
        for k in range(plan["n_bins"]):
            a, e = int(bin_off[k]), int(bin_off[k + 1])
            t0, t1 = int(offB[a]), int(offB[e])
            ro = self.meta_dev[starts[k]:starts[k] + e - a + 1]
            tr = ops.tok_row(ro, t1 - t0, out=self.tok_row[:t1 - t0])
            ws = {kk: self.ws[kk][t0:t1] for kk in ("logp", "lse", "entropy", "loss_tok", "kl_tok", "tok_flags")}
            ops.loss_fwd_bwd(self.logits[t0:t1], self.target[t0:t1], self.mask[t0:t1], self.old[t0:t1], tr,
                             self.adv_dev[a:e], ro, scale=1.0, denom=self.N, dlogits=self.dlogits[t0:t1], ws=ws,
                             defer_stats=True, on_launch=self.timed.mark)
            self.timed.end_marked(chunk_bytes(self.mask_np[t0:t1], b["V"], 2, 2))
        self.ws["row_stats"] = self.stats_dev
        self.ws["chunk_stats"] = self.win_stats
        ops.loss_stats(self.ws, self.offB_dev, scale=1.0, denom=self.N)
        self.stats_host.copy_(self.stats_dev, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        raw = self.stats_host.numpy()
        nb = plan["n_bins"]
        acc = ops.Accumulator(nb)
        for k in range(nb):                       # a box's stats: the sum of its rows'
            acc.add_rows(raw, int(bin_off[k]), int(bin_off[k + 1] - bin_off[k]))
        return [acc.finalize()]

    def sample(self, n, start=0):
        torch = self.torch
        idx = np.arange(start, min(start + n, self.logits.shape[0]))
        z = self.logits[torch.as_tensor(idx, device="cuda")].double().cpu().numpy()
        adv = np.random.default_rng(1).normal(0, 1, len(idx))
        return z, self.target[:len(idx)].cpu().numpy(), np.zeros(len(idx)), adv


# ---------------------------------------------------------------- compaction: fused LM head

class CompactStep:
    def __init__(self, wl, seed, torch, ops, timed, keep_z=False, defer_dw=False):
        from synth import compaction_batch
        self.torch, self.ops, self.timed = torch, ops, timed
        b = self.b = compaction_batch(seed=seed)
        plan = ops.plan_compaction(b["rows_per_rollout"], b["n_groups"], b["group"], b["Q"],
                                   b["n_groups"] * b["group"])
        H, V = b["H"], b["V"]
        seg_len = b["seg_len"]
        seg_off = np.concatenate([[0], np.cumsum(seg_len)])
        row_len = np.array([seg_len[s] for s in plan["row_src"]], np.int64)
        self.off = np.concatenate([[0], np.cumsum(row_len)])
        src_tok = np.concatenate([np.arange(seg_off[s], seg_off[s] + seg_len[s]) for s in plan["row_src"]])
        n_tok = int(self.off[-1])
        mask = np.repeat(1 - plan["is_pad"].astype(np.uint8), row_len).astype(np.uint8)
        gen = torch.Generator(device="cuda").manual_seed(seed + 11)
        self.W = (torch.randn((V, H), generator=gen, device="cuda") * b["w_std"]).to(torch.bfloat16)
        h_seg = (torch.randn((int(seg_off[-1]), H), generator=gen, device="cuda") * b["h_std"]).to(torch.bfloat16)
        self.h = h_seg[torch.as_tensor(src_tok, device="cuda")].contiguous()   # pads copy a real row
        del h_seg
        self.target = _g(torch, b["target"][src_tok])
        self.mask = _g(torch, mask)
        self.mask_np = mask
        # pi_old from a plain fp32 recompute, 1024 tokens at a time, plus the drift
        old = torch.empty(n_tok, dtype=torch.float32, device="cuda")
        Wf = self.W.float()
        for a in range(0, n_tok, 1024):
            e = min(a + 1024, n_tok)
            z = self.h[a:e].float() @ Wf.t()
            old[a:e] = torch.log_softmax(z, -1).gather(1, self.target[a:e].long()[:, None])[:, 0]
            del z
        del Wf
        self.old = old + _g(torch, b["logratio_noise"][src_tok]).float()
        self.Wt = torch.empty((H, V), dtype=torch.bfloat16, device="cuda")
        self.dW = torch.zeros((V, H), dtype=torch.float32, device="cuda")
        self.dh = torch.empty((n_tok, H), dtype=torch.float32, device="cuda")
        self.N = torch.empty(1, dtype=torch.int64, device="cuda")
        self.chunks = [(a, min(a + b["micro"], plan["n_rows"])) for a in range(0, plan["n_rows"], b["micro"])]
        max_tok = int(max(self.off[e] - self.off[a] for a, e in self.chunks))
        self.keep_z = keep_z
        self.defer_dw = defer_dw
        self.workspace = torch.empty(ops.lmhead_workspace_bytes(max_tok, H, V, keep_z, defer_dw), dtype=torch.uint8,
                                     device="cuda")
        # the dW window holds every chunk's columns (its tokens rounded up to 64)
        self.window = (ops.LmheadDwWindow(sum(-(-int(self.off[e] - self.off[a]) // 64) * 64 for a, e in self.chunks),
                                          H, V, device="cuda") if defer_dw else None)
        self.ws = ops.loss_workspace(max_tok, b["micro"], "cuda")
        self.tok_row = torch.empty(max_tok, dtype=torch.int32, device="cuda")
        self.row_off_dev = _g(torch, np.concatenate([self.off[a:e + 1] - self.off[a] for a, e in self.chunks]))
        self.adv_host = torch.empty(plan["n_rows"], dtype=torch.float32).pin_memory()
        self.adv_dev = torch.empty(plan["n_rows"], dtype=torch.float32, device="cuda")
        self.stats_dev = torch.empty((len(self.chunks), ops.STATS_BYTES), dtype=torch.uint8, device="cuda")
        self.stats_host = torch.empty((len(self.chunks), ops.STATS_BYTES), dtype=torch.uint8).pin_memory()
        self.n_valid = int(mask.sum())
        self.H, self.V = H, V
        self.logits_dtype = ("fp32 logits of one chunk kept for pass 2 (GRPO_LMHEAD_KEEP_Z)" if keep_z else
                             "none (h and W bf16; logits never materialised)")

    def __call__(self):
        torch, ops, b = self.torch, self.ops, self.b
        plan = ops.plan_compaction(b["rows_per_rollout"], b["n_groups"], b["group"], b["Q"],
                                   b["n_groups"] * b["group"])
        adv_roll = ops.group_advantage(b["reward"], b["group"])
        self.adv_host.numpy()[:] = ops.rows_advantage(adv_roll, plan["row_rollout"])
        self.adv_dev.copy_(self.adv_host, non_blocking=True)
        self.dW.zero_()
        ops.transpose_bf16(self.W, out=self.Wt)
        ops.count_valid(self.mask, out=self.N)
        ro_at = 0
        for k, (a, e) in enumerate(self.chunks):
            t0, t1 = int(self.off[a]), int(self.off[e])
            ro = self.row_off_dev[ro_at:ro_at + e - a + 1]
            ro_at += e - a + 1
            tr = ops.tok_row(ro, t1 - t0, out=self.tok_row[:t1 - t0])
            ws = {kk: (v[:t1 - t0] if kk in ("logp", "lse", "entropy", "loss_tok", "tok_flags") else v)
                  for kk, v in self.ws.items()}
            ws["row_stats"] = self.ws["row_stats"][:e - a]
            ws["chunk_stats"] = self.stats_dev[k:k + 1]
            ops.lmhead_fwd_bwd(self.h[t0:t1], self.W, self.Wt, self.target[t0:t1], self.mask[t0:t1],
                               self.old[t0:t1], tr, self.adv_dev[a:e], ro, None if self.defer_dw else self.dW,
                               denom=self.N, dh=self.dh[t0:t1], ws=ws, workspace=self.workspace,
                               keep_z=self.keep_z, dw_window=self.window, on_launch=self.timed.mark)
            # logits, dh and (unless deferred) dW: 2VH each per valid token
            self.timed.end_marked((4.0 if self.defer_dw else 6.0) * self.V * self.H
                                  * int(self.mask_np[t0:t1].sum()))
        if self.defer_dw:
            self.window.flush(self.dW, on_launch=self.timed.mark)
            self.timed.end_marked(2.0 * self.V * self.H * self.n_valid)
        self.stats_host.copy_(self.stats_dev, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        acc = ops.Accumulator(len(self.chunks))
        for s in ops.stats_to_dicts(self.stats_host.numpy()):
            acc.add(s)
        return [acc.finalize()]


# ---------------------------------------------------------------- CPU baseline

def _oracle_block(z, y, drift, adv):
    """The oracle on one block of tokens; returns (tokens, seconds of compute)."""
    import oracle
    m = np.ones(len(y), np.uint8)
    old = oracle.logprob_fwd(z, y, m)["logp"] + drift
    t0 = time.perf_counter()
    oracle.loss_fwd_bwd(z, y, m, old, adv, 1e-5)
    return len(y), time.perf_counter() - t0


_SHM = {}


def _oracle_pool_worker(args):
    """One pool task: tokens [a, b) of the shared float64 logits block."""
    from multiprocessing import shared_memory
    name, shape, a, b, y, drift, adv = args
    if name not in _SHM:
        for old in list(_SHM):
            _SHM.pop(old).close()
        _SHM[name] = shared_memory.SharedMemory(name=name)
    z = np.ndarray(shape, dtype=np.float64, buffer=_SHM[name].buf)
    return _oracle_block(z[a:b], y, drift, adv)


def cpu_baseline(step, budget_s, block=1024):
    """The oracle, as it stands, on the benched batch's valid tokens, streamed
    to the host 1024 at a time (float64), until ``budget_s`` seconds of
    compute have run (one process)."""
    done, t_used, pos = 0, 0.0, 0
    V = None
    while t_used < budget_s:
        z_all, y_all, drift, adv_all = step.sample(block, pos)
        if len(y_all) == 0:
            break
        V = z_all.shape[1]
        for a in range(0, len(y_all), 16):
            n, dt = _oracle_block(z_all[a:a + 16], y_all[a:a + 16], drift[a:a + 16], adv_all[a:a + 16])
            done += n
            t_used += dt
            if t_used >= budget_s:
                break
        pos += block
        del z_all
    return {"value": round(done / t_used, 1), "unit": "valid tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {done} valid tokens of the benched batch (V={V}, float64 numpy, one process), "
                      f"{t_used:.1f} s of compute"}


def cpu_baseline_pool(step, budget_s, block=1024):
    """The same oracle over a multiprocessing pool on the cores this process
    may run on (at most 16), blocks of 16 tokens per task; wall time of the
    pool's compute.  Spawned workers: they never touch the GPU."""
    import multiprocessing as mp
    cores = min(len(os.sched_getaffinity(0)), 16)
    done, wall, pos = 0, 0.0, 0
    ctx = mp.get_context("spawn")
    from multiprocessing import shared_memory
    with ctx.Pool(cores) as pool:
        while wall < budget_s:
            z_all, y_all, drift, adv_all = step.sample(block, pos)
            if len(y_all) == 0:
                break
            shm = shared_memory.SharedMemory(create=True, size=z_all.nbytes)
            try:
                np.ndarray(z_all.shape, dtype=np.float64, buffer=shm.buf)[:] = z_all
                tasks = [(shm.name, z_all.shape, a, a + 16, y_all[a:a + 16], drift[a:a + 16], adv_all[a:a + 16])
                         for a in range(0, len(y_all), 16)]
                t0 = time.perf_counter()
                done += sum(n for n, _ in pool.map(_oracle_pool_worker, tasks))
                wall += time.perf_counter() - t0
            finally:
                shm.close()
                shm.unlink()
            pos += block
            del z_all
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(done / wall, 1), "unit": "valid tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} valid tokens of the benched batch, blocks of 1024 in shared memory, 16-token "
                      f"tasks over a {cores}-process pool, {wall:.1f} s wall" + (f" ({model})" if model else "")}


def fused_kernel_label(V, dtype):
    """Which fused-loss kernel a contiguous [tokens x V] chunk of this dtype takes
    (the library's dispatch: 1024 threads x 19 register vectors, plus 9 LDS
    vectors per lane past that, plus up to 4 vectors per lane read in both
    sweeps for bf16, else the streaming kernel; rows off 16-byte alignment,
    whose dlogits rows here share their phase, take the register kernel over
    the aligned vectors covering them, at most V / vec + 1 of them)."""
    vec = 8 if dtype == "bf16" else 4
    if V % vec:
        nvec = (V + 2 * vec - 2) // vec
        return "tok_reg_kernel (rows off alignment)" if nvec <= 1024 * 19 else "tok_stream_kernel"
    if V // vec <= 1024 * 19:
        return "tok_reg_kernel"
    if V // vec <= 1024 * 28:
        return "tok_reg_kernel (LDS tail)"
    if dtype == "bf16" and V // vec <= 1024 * 32:
        return "tok_reg_kernel (LDS tail, part of the row read twice)"
    return "tok_stream_kernel"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from grpo_token_level_amd import ops
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    ops.version()                      # fails loudly if libgrpo.so is missing
    wl = args.workload
    timed = Timed(torch)
    cls = {"qwen": PaddedStep, "long": PaddedStep, "tiny": PaddedStep, "dynamic": DynamicStep,
           "compact": CompactStep}[wl]
    if (args.terms or args.ahead or args.epochs != 1 or args.shuffle or args.graph) and cls is not PaddedStep:
        print("--terms, --ahead, --epochs, --shuffle and --graph apply to the padded workloads (qwen, long, tiny)",
              file=sys.stderr)
        sys.exit(2)
    extra = {}
    if args.terms:
        extra["terms"] = True
    if args.ahead:
        extra["ahead"] = True
    if args.paired:
        if not args.ahead:
            print("--paired applies to --ahead", file=sys.stderr)
            sys.exit(2)
        extra["paired"] = True
    if args.epochs != 1 or args.shuffle:
        extra["epochs"] = args.epochs
        extra["shuffle"] = args.shuffle
    if args.graph:
        if args.ahead:
            print("--graph does not combine with --ahead (the cache's host bookkeeping runs per call)",
                  file=sys.stderr)
            sys.exit(2)
        extra["graph"] = True
    if args.replicate != 1:
        if wl != "tiny":
            print("--replicate applies to the tiny workload", file=sys.stderr)
            sys.exit(2)
        from synth import WORKLOADS
        extra["over"] = dict(n_prompts=WORKLOADS["tiny"]["n_prompts"] * args.replicate, mini=0, micro=0)
    if args.keep_z:
        if cls is not CompactStep:
            print("--keep-z applies to the compact workload", file=sys.stderr)
            sys.exit(2)
        extra["keep_z"] = True
    if args.defer_dw:
        if cls is not CompactStep:
            print("--defer-dw applies to the compact workload", file=sys.stderr)
            sys.exit(2)
        extra["defer_dw"] = True
    if args.vocab:
        if cls is not PaddedStep or args.vocab < 1:
            print("--vocab applies to the padded workloads (qwen, long, tiny) and must be positive", file=sys.stderr)
            sys.exit(2)
        extra.setdefault("over", {})["V"] = args.vocab
    step = cls(wl, args.seed, torch, ops, timed, **extra)
    # device memory of the steps alone (the set-up's own peak is left out)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    # A full garbage collection walks every tracked Python object, most of them
    # torch's own (~170 k): tens of milliseconds on one host thread.  Inside the
    # timed steps such a pause can fall between a launch's start event and the
    # launch itself while the GPU has drained its queue, and the idle time would
    # be booked to that launch.  The set-up's objects are collected once and
    # frozen out of later collections; the steps' own garbage is still collected.
    gc.collect()
    gc.freeze()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timed.on = True
    if getattr(step, "ahead", False):
        step.ahead_timed.on = True
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    marks[0].record()
    for k in range(args.steps):
        res = step()
        marks[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = sorted(marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps))
    median_ms = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    ms = 1e3 * wall / args.steps
    value = step.n_valid / (wall / args.steps)
    tot_ms, units, launches = timed.totals()
    cfg = {"workload": f"{wl}: {WORKLOAD_TEXT[wl]}"
                       + ("; seq-mean-token-mean aggregation, entropy bonus 0.01, k3 KL 0.05" if args.terms else "")
                       + ("; ahead pass (pi_old cache) in the step" if args.ahead else "")
                       + (f"; {args.epochs} inner epochs" if args.epochs != 1 else "")
                       + ("; rows reshuffled every epoch (seeded)" if args.shuffle else "")
                       + (f"; replicated x{args.replicate} as one batch, one launch" if args.replicate != 1 else "")
                       + ("; device work replayed from a HIP graph" if args.graph else "")
                       + (f"; vocabulary {args.vocab} in place of the workload's" if args.vocab else "")
                       + ("; dW of the step's chunks as one GEMM from a dW window" if args.defer_dw else ""),
           "logits_dtype": step.logits_dtype,
           "valid_tokens": step.n_valid, "launches_per_step": launches // args.steps,
           "step_loss": res[0]["loss"] if res and res[0] else None}
    if args.terms and res and res[0]:
        cfg["step_objective"] = res[0]["obj_sum"]
    if args.ahead:
        cfg["ahead_pass"] = bool(getattr(step, "ahead", False))
        if cfg["ahead_pass"]:
            a_ms, a_units, a_n = step.ahead_timed.totals()
            cfg["ahead_ms_per_step"] = round(a_ms / args.steps, 4)
            cfg["ahead_read_GBs"] = round(a_units / (a_ms * 1e-3) / 1e9, 1)
            cfg["device_read_GBs"] = round(step.read_context(), 1)
            cfg["ahead_paired"] = bool(getattr(step, "paired", False))
    if wl == "compact":
        achieved = (units / launches) / (tot_ms / launches * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "grpo_lmhead_fwd_bwd per 4-row chunk (bf16 MFMA GEMMs + epilogues"
                          + ("; pass 2 from the kept fp32 logits" if getattr(step, "keep_z", False) else
                             "; pass 2 recomputes the logits")
                          + ("; dW deferred to one grpo_lmhead_dw_flush GEMM per step, counted as a launch)"
                             if getattr(step, "defer_dw", False) else ")"),
                "algorithmic_flops_per_launch": int(units // launches), "avg_launch_ms": round(tot_ms / launches, 4)}
    else:
        achieved = (units / launches) / (tot_ms / launches * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": fused_kernel_label(step.V, step.logits_dtype) + " (fused loss fwd+bwd), per chunk launch; "
                          "the row and chunk reductions run once per optimizer window, outside these windows"
                          + ("; graph replay time (reductions included) divided by the chunk launches"
                             if args.graph else ""),
                "algorithmic_bytes_per_launch": int(units // launches), "avg_launch_ms": round(tot_ms / launches, 4)}
        roof["device_copy_GBs"] = round(step.copy_context(), 1)
        if wl in ("qwen", "long", "dynamic") and not (args.terms or args.ahead or args.epochs != 1 or args.shuffle
                                                     or args.vocab):
            from yardstick.prof_summary import load_traffic
            rec = load_traffic(os.path.join(ROOT, "profiles", f"fused_loss_{wl}_pmc.txt"))
            if rec is not None:
                roof["traffic"] = rec["traffic_bytes_per_launch"]
    cfg["llc"] = step.llc_note() if hasattr(step, "llc_note") else None
    if wl == "compact":
        # the LM head's memory claim: the default path never holds a [tokens x V]
        # matrix (the kept logits and the dW window do, on request)
        cfg["peak_device_GB"] = round(torch.cuda.max_memory_allocated() / 1e9, 2)
        cfg["tokens_x_V_bf16_GB"] = round(int(step.off[-1]) * step.V * 2 / 1e9, 2)
    out = {"metric": METRIC, "value": round(value, 1), "unit": "valid tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "ms_per_step_median": round(median_ms, 4),
           "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if wl == "compact" else "f32", "data": "synthetic", "config": cfg,
           "roofline": roof}
    if args.copy_calibration:
        # known-size plain copy for the byte counters: 1 GiB read, 1 GiB written
        x = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
        y = torch.empty_like(x)
        torch.bitwise_not(x, out=y)
        torch.cuda.synchronize()
    if args.cpu_seconds > 0 and hasattr(step, "sample"):
        out["cpu_baseline"] = cpu_baseline(step, args.cpu_seconds)
        if args.cpu_pool_seconds > 0:
            out["cpu_baseline_pool"] = cpu_baseline_pool(step, args.cpu_pool_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
