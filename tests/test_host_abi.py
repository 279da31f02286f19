"""CPU tests of libgrpo's host half through the C ABI: every declared symbol
is exported, the ctypes structs match the C layout, and the host plans,
advantages and accumulator agree with the oracle (plans bit-exact)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from oracle import PlanError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grpo.h")

C = pytest.importorskip("grpo_token_level_amd._capi")
try:
    C.lib()
except ImportError as e:  # pragma: no cover - the driver builds before testing
    pytest.skip(str(e), allow_module_level=True)
from grpo_token_level_amd import ops  # noqa: E402
from grpo_token_level_amd.ops import GrpoError  # noqa: E402


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(grpo_\w+)\s*\(", text)))


@pytest.mark.skipif(C.HOST_ONLY, reason="the host-only sanitizer build carries no device entry points")
def test_every_declared_function_is_exported():
    names = _declared_functions()
    assert len(names) >= 15
    lib = ctypes.CDLL(C.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares a prototype for each of them
    assert sorted(C.PROTOTYPES) == names


def test_struct_layouts_match_the_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "grpo.h"
#define F(T, f) printf(#T "." #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("grpo_stats %zu\n", sizeof(grpo_stats));
  printf("grpo_loss_args %zu\n", sizeof(grpo_loss_args));
  printf("grpo_step_result %zu\n", sizeof(grpo_step_result));
  printf("grpo_lmhead_args %zu\n", sizeof(grpo_lmhead_args));
  F(grpo_loss_args, logits) F(grpo_loss_args, n_rows) F(grpo_loss_args, eps_low) F(grpo_loss_args, denom)
  F(grpo_loss_args, dlogits) F(grpo_loss_args, chunk_stats)
  F(grpo_lmhead_args, Wt) F(grpo_lmhead_args, n_rows) F(grpo_lmhead_args, denom) F(grpo_lmhead_args, workspace_bytes)
  F(grpo_loss_args, row_weight) F(grpo_loss_args, kl_tok) F(grpo_loss_args, kl_type)
  F(grpo_lmhead_args, row_weight) F(grpo_lmhead_args, ent_coef) F(grpo_lmhead_args, kl_type)
  F(grpo_lmhead_args, flags) F(grpo_lmhead_args, dw_window)
  printf("grpo_lmhead_dw_window %zu\n", sizeof(grpo_lmhead_dw_window));
  F(grpo_lmhead_dw_window, bytes) F(grpo_lmhead_dw_window, cap_tok) F(grpo_lmhead_dw_window, V)
  F(grpo_lmhead_dw_window, reserved)
  F(grpo_stats, kl_sum) F(grpo_stats, obj_sum) F(grpo_stats, n_valid_rows)
  F(grpo_step_result, kl) F(grpo_step_result, obj_sum) F(grpo_step_result, n_clipped)
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines())
    assert int(got["grpo_stats"]) == ctypes.sizeof(C.Stats) == C.STATS_BYTES
    assert int(got["grpo_loss_args"]) == ctypes.sizeof(C.LossArgs)
    assert int(got["grpo_step_result"]) == ctypes.sizeof(C.StepResult)
    assert int(got["grpo_lmhead_args"]) == ctypes.sizeof(C.LmheadArgs)
    assert int(got["grpo_lmhead_dw_window"]) == ctypes.sizeof(C.DwWindow)
    for key, v in got.items():
        if "." in key:
            struct, field = key.split(".")
            cls = {"grpo_loss_args": C.LossArgs, "grpo_lmhead_args": C.LmheadArgs,
                   "grpo_stats": C.Stats, "grpo_step_result": C.StepResult,
                   "grpo_lmhead_dw_window": C.DwWindow}[struct]
            assert getattr(cls, field).offset == int(v), key


# ---------------------------------------------------------------- plans vs oracle

def _kind(fn, *a, **k):
    try:
        return fn(*a, **k), None
    except PlanError as e:
        return None, e.kind
    except GrpoError as e:
        return None, e.kind
    except ValueError:
        return None, "EINVAL"


def test_fixed_plan_matches_oracle():
    rng = np.random.default_rng(0)
    cases = [(32, 4, 16, 8), (32, 4, 0, 0), (30, 4, 0, 0), (64, 4, 0, 8), (128, 8, 64, 4), (32, 4, 12, 0),
             (32, 4, 16, 5), (0, 4, 0, 0), (32, 0, 0, 0), (32, 4, -1, 0)]
    for _ in range(300):
        cases.append(tuple(int(x) for x in (rng.integers(0, 70), rng.integers(0, 9), rng.integers(0, 70), rng.integers(0, 40))))
    for c in cases:
        want, wk = _kind(oracle.plan_fixed, *c)
        got, gk = _kind(ops.plan_fixed, *c)
        assert (got, gk) == (want, wk), c
        if want:
            for i, j in oracle.train_calls(want):
                assert ops.plan_chunk(c[0], want[2], want[3], i, j) == oracle.chunk_rows(want, i, j)


def test_plan_chunk_rejects_out_of_range():
    with pytest.raises(GrpoError) as e:
        ops.plan_chunk(32, 16, 8, 2, 0)
    assert e.value.kind == "EINVAL"


def test_dynamic_plan_matches_oracle_bit_exact():
    rng = np.random.default_rng(1)
    for _ in range(200):
        n = int(rng.integers(0, 60))
        budget = int(rng.integers(8, 300))
        lengths = rng.integers(0, budget + (1 if rng.random() < 0.9 else 40), size=n).tolist()
        pd = int(rng.integers(1, 5000))
        want, wk = _kind(oracle.plan_dynamic, lengths, budget, pd)
        got, gk = _kind(ops.plan_dynamic, lengths, budget, pd)
        assert gk == wk
        if want:
            assert got["n_bins"] == want["n_bins"]
            assert got["bin_off"].tolist() == want["bin_off"]
            assert got["order"].tolist() == want["order"]
            assert got["restore"].tolist() == want["restore"]


def test_dynamic_plan_on_the_lognormal_workload():
    from synth import dynamic_lengths
    for seed in range(3):
        L = dynamic_lengths(seed=seed).tolist()
        want = oracle.plan_dynamic(L, 16384, 4096)
        got = ops.plan_dynamic(L, 16384, 4096)
        assert got["order"].tolist() == want["order"] and got["bin_off"].tolist() == want["bin_off"]


def test_dynamic_capacity_error_reports_need():
    nb = ctypes.c_int64()
    L = np.array([8] * 10, np.int64)
    off = np.zeros(3, np.int64)
    order = np.zeros(10, np.int64)
    rest = np.zeros(10, np.int64)
    code = C.lib().grpo_plan_dynamic(C.ptr64(L), 10, 8, 4, 2, ctypes.byref(nb), C.ptr64(off), C.ptr64(order), C.ptr64(rest))
    assert code == -7 and nb.value == 10


def test_compaction_plan_matches_oracle():
    rng = np.random.default_rng(2)
    cases = [([1, 3, 2, 5, 1, 1], 3, 2, 4, 6, False), ([1, 3, 2, 5, 1, 1], 3, 2, 4, 8, False),
             ([1, 3, 2, 5], 3, 2, 4, 6, False), ([1, 0, 2, 5, 1, 1], 3, 2, 4, 6, False),
             ([1, 3, 2, 5, 1, 1], 3, 2, 4, 6, True), ([1, 3, 2, 5, 1, 1], 3, 2, 0, 6, False)]
    for _ in range(200):
        G, ng, Q = int(rng.integers(1, 6)), int(rng.integers(1, 8)), int(rng.integers(1, 9))
        seg = rng.integers(1, 6, size=ng * G).tolist()
        cases.append((seg, ng, G, Q, ng * G, False))
    for seg, ng, G, Q, exp, dyn in cases:
        want, wk = _kind(oracle.plan_compaction, seg, ng, G, Q, exp, dynamic=dyn)
        got, gk = _kind(ops.plan_compaction, seg, ng, G, Q, exp, dynamic=dyn)
        assert gk == wk, (seg, ng, G, Q, exp, dyn)
        if want:
            for k in ("row_rollout", "row_seg", "row_src", "is_pad", "group_pad"):
                assert got[k].tolist() == want[k], k
            assert got["n_rows"] == want["n_rows"]


def test_row_offsets():
    L = np.array([3, 0, 5, 2])
    assert ops.row_offsets(L).tolist() == [0, 3, 3, 8, 10]
    assert ops.row_offsets(L, [2, 0, 3, 1]).tolist() == [0, 5, 8, 10, 10]


# ---------------------------------------------------------------- advantage vs oracle

def test_group_advantage_matches_oracle():
    rng = np.random.default_rng(3)
    for G in (1, 2, 4, 8):
        for norm in (True, False):
            r = (rng.random(8 * G) < 0.5).astype(np.float32) + rng.normal(0, 0.1, 8 * G).astype(np.float32)
            got = ops.group_advantage(r, G, 1e-6, norm)
            want = oracle.group_advantage(r.astype(np.float64), G, 1e-6, norm)
            # host accumulates in double and rounds once to float32
            assert np.allclose(got, want, rtol=2 ** -23, atol=1e-12)
    with pytest.raises(GrpoError):
        ops.group_advantage([1, 0, 1], 2)


def test_rows_advantage_matches_oracle():
    p = oracle.plan_compaction([1, 3, 2, 5, 1, 1], 3, 2, 4, 6)
    A = np.array([1.0, -1.0, 0.5, -0.5, 2.0, -2.0], np.float32)
    assert ops.rows_advantage(A, p["row_rollout"]).tolist() == oracle.rows_advantage(A, p["row_rollout"]).tolist()
    with pytest.raises(GrpoError):
        ops.rows_advantage(A, [0, 6])


# ---------------------------------------------------------------- accumulator vs oracle

def test_accumulator_matches_oracle_on_random_sequences():
    rng = np.random.default_rng(4)
    for _ in range(100):
        n_micro = int(rng.integers(1, 6))
        a, b = oracle.Accumulator(n_micro), ops.Accumulator(n_micro)
        for _ in range(int(rng.integers(1, 40))):
            if rng.random() < 0.3:
                fa, fb = a.finalize(), b.finalize()
                assert (fa is None) == (fb is None)
                if fa:
                    for k in fa:
                        assert fb[k] == pytest.approx(fa[k], rel=1e-15, abs=0), k
                continue
            bad = rng.random() < 0.15
            st = {"loss_sum": float("nan") if bad and rng.random() < 0.5 else float(rng.normal()),
                  "entropy_sum": float(rng.random()), "kl_sum": float(rng.random()),
                  "obj_sum": float("inf") if bad and rng.random() < 0.3 else float(rng.normal()),
                  "n_valid": int(rng.integers(0, 50)),
                  "n_clipped": int(rng.integers(0, 3)), "n_nonfinite": 1 if bad else 0,
                  "n_valid_rows": int(rng.integers(0, 4))}
            assert b.add(st) == a.add(st)


def test_accumulator_is_opaque_and_refuses_unprepared_bytes():
    L = C.lib()
    n = int(L.grpo_accum_size())
    assert 0 < n <= 4096
    raw = (ctypes.c_int64 * ((n + 7) // 8))()
    s = C.Stats(n_valid=3, loss_sum=1.5)
    r = C.StepResult()
    stepped = ctypes.c_int32(7)
    assert L.grpo_accum_add(raw, ctypes.byref(s)) == -1                  # never prepared
    assert L.grpo_accum_finalize(raw, ctypes.byref(r), ctypes.byref(stepped)) == -1
    assert stepped.value == 7                                            # nothing written on an error
    assert L.grpo_accum_init(raw, 0) == -1
    assert L.grpo_accum_init(raw, 1) == 0
    assert L.grpo_accum_add(raw, ctypes.byref(s)) == 0
    copy = (ctypes.c_int64 * len(raw))(*raw)                             # plain bytes: a copy is a copy
    for acc in (raw, copy):
        assert L.grpo_accum_finalize(acc, ctypes.byref(r), ctypes.byref(stepped)) == 0
        assert stepped.value == 1 and r.n_valid == 3 and r.loss == 0.5


def test_stats_sum_adds_rows_in_order():
    rng = np.random.default_rng(9)
    for n in (0, 1, 7, 300):
        rows = [{"loss_sum": float(rng.normal()), "entropy_sum": float(rng.random()), "kl_sum": float(rng.normal()),
                 "obj_sum": float(rng.normal()), "n_valid": int(rng.integers(0, 100)),
                 "n_clipped": int(rng.integers(0, 3)), "n_nonfinite": int(rng.integers(0, 2)),
                 "n_valid_rows": int(rng.integers(0, 2))} for _ in range(n)]
        want = {k: 0.0 if k.endswith("_sum") else 0 for k in oracle.STAT_KEYS}
        for r in rows:                               # the oracle's chunk roll-up: rows in row order
            for k in want:
                want[k] += r[k]
        assert ops.stats_sum(rows) == want


# ---------------------------------------------------------------- ahead pass, cache, probe (host parts)

def test_ahead_pass_gate_matches_oracle():
    for n_mini in (0, 1, 2, 7):
        for rollout in (False, True):
            for consumes in (False, True):
                assert ops.needs_ahead_pass(n_mini, rollout, consumes) == oracle.needs_ahead_pass(n_mini, rollout,
                                                                                                  consumes)


def test_probe_verdict_matches_oracle():
    rng = np.random.default_rng(5)
    for _ in range(200):
        bound, frac = float(rng.random() * 0.1), float(rng.choice([0.0, 0.05, 0.1, 0.5, 1.0]))
        n_valid = int(rng.integers(0, 100))
        n_moved = int(rng.integers(0, n_valid + 1))
        a, b = ops.Probe(bound, frac), oracle.Probe(bound, frac)
        st = {"n_valid": n_valid, "n_moved": n_moved, "max_abs": 0.0}
        assert a.finish(st) == b.finish(n_valid, n_moved)
        with pytest.raises(GrpoError) as e:
            a.finish(st)
        assert e.value.kind == "ESTATE"
    with pytest.raises(GrpoError):
        ops.Probe(-1.0, 0.0)
    with pytest.raises(GrpoError):
        ops.Probe(0.05, 1.5)


def test_old_cache_state_machine_without_device_work():
    # zero-token records never launch a kernel, so the bookkeeping runs on the CPU
    c = C.OldCache()
    off = np.zeros(4, np.int64)
    L = C.lib()
    assert L.grpo_old_cache_init(ctypes.byref(c), None, 0, C.ptr64(off), 3) == 0
    ptr = ctypes.c_void_p()
    assert L.grpo_old_cache_replay(ctypes.byref(c), 0, ctypes.byref(ptr)) == -9          # nothing recorded
    for _ in range(3):
        assert L.grpo_old_cache_record(None, ctypes.byref(c), 1, None, 8, 0, 8, None, None, None) == 0
    assert L.grpo_old_cache_record(None, ctypes.byref(c), 1, None, 8, 0, 8, None, None, None) == -9  # walk complete
    assert L.grpo_old_cache_replay(ctypes.byref(c), 5, ctypes.byref(ptr)) == -1          # token count differs
    assert L.grpo_old_cache_replay(ctypes.byref(c), 0, ctypes.byref(ptr)) == 0
    assert L.grpo_old_cache_record(None, ctypes.byref(c), 1, None, 8, 0, 8, None, None, None) == -9  # replay began
    assert L.grpo_old_cache_reset(ctypes.byref(c)) == 0 and c.recorded == 0 and c.replayed == 0
    # a record that does not fit is refused before any launch
    assert L.grpo_old_cache_record(None, ctypes.byref(c), 1, ctypes.c_void_p(16), 8, 4, 8, ctypes.c_void_p(16),
                                   ctypes.c_void_p(16), None) == -7
    assert L.grpo_old_cache_init(ctypes.byref(c), None, 0, C.ptr64(off), 0) == -1


def test_paired_old_cache_record_keeps_the_same_bookkeeping():
    # grpo_old_cache_record_paired differs only in the forward pass it runs:
    # zero-token records exercise its bookkeeping on the CPU, interleaved with
    # plain records in one walk
    c = C.OldCache()
    off = np.zeros(4, np.int64)
    L = C.lib()
    assert L.grpo_old_cache_init(ctypes.byref(c), None, 0, C.ptr64(off), 3) == 0
    assert L.grpo_old_cache_record_paired(None, ctypes.byref(c), 1, None, 8, 0, 8, None, None, None) == 0
    assert L.grpo_old_cache_record(None, ctypes.byref(c), 1, None, 8, 0, 8, None, None, None) == 0
    assert L.grpo_old_cache_record_paired(None, ctypes.byref(c), 1, None, 8, 0, 8, None, None, None) == 0
    assert c.recorded == 3
    assert L.grpo_old_cache_record_paired(None, ctypes.byref(c), 1, None, 8, 0, 8, None, None, None) == -9
    assert L.grpo_old_cache_reset(ctypes.byref(c)) == 0
    assert L.grpo_old_cache_record_paired(None, ctypes.byref(c), 1, ctypes.c_void_p(16), 8, 4, 8,
                                          ctypes.c_void_p(16), ctypes.c_void_p(16), None) == -7   # does not fit
    assert L.grpo_old_cache_record_paired(None, None, 1, None, 8, 0, 8, None, None, None) == -1


def test_epoch_plan_matches_oracle_bit_exact():
    rng = np.random.default_rng(6)
    cases = [(32, 4, 16, 8, 3, True, 7), (32, 4, 16, 8, 2, False, 7), (8, 2, 4, 2, 1, True, 0),
             (1, 1, 0, 0, 4, True, 2 ** 64 - 1), (30, 3, 10, 5, 2, True, 12345)]
    for _ in range(60):
        G = int(rng.integers(1, 5))
        B = G * int(rng.integers(1, 20))
        cases.append((B, G, 0, 0, int(rng.integers(1, 4)), bool(rng.integers(0, 2)), int(rng.integers(0, 2 ** 63))))
    for B, G, mini, micro, mu, sh, seed in cases:
        want = oracle.plan_epochs(B, G, mini, micro, mu, sh, seed)
        got = ops.plan_epochs(B, G, mini, micro, mu, sh, seed)
        for k in ("n_mini", "n_micro", "mini_rows", "micro_rows"):
            assert got[k] == want[k]
        assert got["perm"].tolist() == want["perm"], (B, mu, sh, seed)
    for bad in ((32, 4, 16, 8, 0, True, 1), (32, 4, 12, 0, 2, True, 1), (0, 4, 0, 0, 1, False, 1)):
        w, wk = _kind(oracle.plan_epochs, *bad)
        g, gk = _kind(ops.plan_epochs, *bad)
        assert gk == wk, bad


def test_old_cache_rewind_without_device_work():
    c = C.OldCache()
    off = np.zeros(3, np.int64)
    L = C.lib()
    assert L.grpo_old_cache_init(ctypes.byref(c), None, 0, C.ptr64(off), 2) == 0
    for _ in range(2):
        assert L.grpo_old_cache_record(None, ctypes.byref(c), 1, None, 8, 0, 8, None, None, None) == 0
    assert L.grpo_old_cache_rewind(ctypes.byref(c)) == -9          # not replayed yet
    ptr = ctypes.c_void_p()
    for _ in range(2):
        assert L.grpo_old_cache_replay(ctypes.byref(c), 0, ctypes.byref(ptr)) == 0
    assert L.grpo_old_cache_rewind(ctypes.byref(c)) == 0 and c.replayed == 0
    assert L.grpo_old_cache_replay(ctypes.byref(c), 0, ctypes.byref(ptr)) == 0


@pytest.mark.skipif(C.HOST_ONLY, reason="the host-only sanitizer build carries no device entry points")
def test_lmhead_workspace_sizes():
    # The default path never holds a [tokens x V] matrix: past one
    # 65536-column chunk its workspace grows with the vocabulary only by the
    # log-softmax slice partials (16 bytes per token per 64 columns);
    # GRPO_LMHEAD_KEEP_Z adds the fp32 logits and dz over the whole
    # vocabulary (8 bytes per token and column).
    L = C.lib()
    n, H, V = 2700, 2048, 151936
    base = L.grpo_lmhead_workspace_size(n, H, V)
    assert base == L.grpo_lmhead_workspace_size_flags(n, H, V, 0)
    grow = L.grpo_lmhead_workspace_size(n, H, 2 * V) - base
    assert grow <= n * V // 4 + 4096
    keep = L.grpo_lmhead_workspace_size_flags(n, H, V, C.LMHEAD_KEEP_Z)
    assert keep >= base + 8 * n * V - 4 * n * 65536
    grow_keep = L.grpo_lmhead_workspace_size_flags(n, H, 2 * V, C.LMHEAD_KEEP_Z) - keep
    assert grow_keep >= 8 * n * V
    # GRPO_LMHEAD_DEFER_DW: h^T and the chunk of dz^T leave the workspace, and dz
    # spans up to the whole vocabulary
    n_pad = (n + 63) // 64 * 64
    defer = L.grpo_lmhead_workspace_size_flags(n, H, V, C.LMHEAD_DEFER_DW)
    assert defer >= 2 * n * V
    assert defer <= base + 2 * n * ((V + 255) // 256 * 256) - 2 * n_pad * (H + 65536) + 4096
    both = L.grpo_lmhead_workspace_size_flags(n, H, V, C.LMHEAD_KEEP_Z | C.LMHEAD_DEFER_DW)
    assert keep - both >= 2 * n_pad * (H + V) - 512
    assert L.grpo_lmhead_workspace_size_flags(n, H, V, 4) == 0           # unknown flag
    assert L.grpo_lmhead_workspace_size_flags(-1, H, V, 0) == 0
    assert L.grpo_lmhead_workspace_size_flags(0, H, V, C.LMHEAD_KEEP_Z) > 0


def _lmhead_args(n, H, V, flags=0, window=None):
    """grpo_lmhead_args with stand-in device addresses: every call below is
    refused by the host checks before anything touches them."""
    a = C.LmheadArgs()
    a.struct_size = ctypes.sizeof(C.LmheadArgs)
    fake = 1 << 40
    a.h, a.ldh, a.W, a.Wt, a.dW = fake, H, fake, fake, fake
    a.n_tok, a.H, a.V = n, H, V
    for f in ("target", "mask", "old_logp", "tok_row", "adv_row", "row_off", "dh", "logp", "entropy", "loss_tok",
              "tok_flags", "row_stats", "chunk_stats", "workspace"):
        setattr(a, f, fake)
    a.n_rows, a.eps_low, a.eps_high, a.scale = 1, 0.2, 0.2, 1.0
    a.workspace_bytes = 1 << 50
    a.flags = flags
    a.dw_window = ctypes.addressof(window) if window is not None else None
    return a


@pytest.mark.skipif(C.HOST_ONLY, reason="the host-only sanitizer build carries no device entry points")
def test_lmhead_dw_window_sizes_and_refusals():
    L = C.lib()
    kind = lambda rc: C.CODES[rc]  # noqa: E731
    H, V = 2048, 151936
    cap = (1000 + 63) // 64 * 64
    r256 = lambda b: (b + 255) // 256 * 256  # noqa: E731
    need = L.grpo_lmhead_dw_window_size(1000, H, V)
    assert need == 256 + r256(2 * H * cap) + r256(2 * V * cap)
    for bad in ((0, H, V), ((1 << 30) + 1, H, V), (64, 7, V), (64, H, 0), (64, H, 12)):
        assert L.grpo_lmhead_dw_window_size(*bad) == 0
    # set-up refusals (no kernel is launched before these checks)
    w = C.DwWindow()
    fake = 1 << 40
    assert kind(L.grpo_lmhead_dw_window_init(None, None, fake, need, 1000, H, V)) == "EINVAL"
    assert kind(L.grpo_lmhead_dw_window_init(None, ctypes.byref(w), fake + 16, need, 1000, H, V)) == "EINVAL"
    assert kind(L.grpo_lmhead_dw_window_init(None, ctypes.byref(w), fake, need, 1000, H, 12)) == "EINVAL"
    assert kind(L.grpo_lmhead_dw_window_init(None, ctypes.byref(w), fake, need - 1, 1000, H, V)) == "ECAPACITY"
    # a window as init leaves it, filled by hand (host fields only)
    w.buf, w.bytes, w.cap_tok, w.H, w.V, w.reserved = fake, need, 1000, H, V, 0
    assert kind(L.grpo_lmhead_dw_flush(None, None, fake)) == "EINVAL"
    assert kind(L.grpo_lmhead_dw_flush(None, ctypes.byref(w), None)) == "EINVAL"
    assert kind(L.grpo_lmhead_dw_flush(None, ctypes.byref(w), fake)) == "OK"        # empty: nothing to launch
    w.reserved = 100                                                                # not a multiple of 64
    assert kind(L.grpo_lmhead_dw_flush(None, ctypes.byref(w), fake)) == "EINVAL"
    w.reserved = 0
    # the loss call: the flag and the window go together, sizes must match,
    # the window must have room, and the fixed-scratch entry point refuses it
    D = C.LMHEAD_DEFER_DW
    call = lambda a: kind(L.grpo_lmhead_fwd_bwd(None, ctypes.byref(a)))  # noqa: E731
    assert call(_lmhead_args(100, H, V, D, None)) == "EINVAL"
    assert call(_lmhead_args(100, H, V, 0, w)) == "EINVAL"
    assert call(_lmhead_args(100, H, V - 8, D, w)) == "EINVAL"
    assert call(_lmhead_args(1025, H, V, D, w)) == "ECAPACITY"       # 1088 columns > the window's 1024
    w.reserved = 960
    assert call(_lmhead_args(65, H, V, D, w)) == "ECAPACITY"         # 960 + 128 > 1024
    assert w.reserved == 960                                           # a refused call reserves nothing
    a = _lmhead_args(100, H, V, D, w)
    assert kind(L.grpo_lmhead_fwd_bwd_noalloc(None, ctypes.byref(a))) == "EINVAL"
    a = _lmhead_args(100, H, V, C.LMHEAD_KEEP_Z, None)
    a.dW = None                                                        # dW is required unless deferred
    assert call(a) == "EINVAL"
