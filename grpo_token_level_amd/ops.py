"""Python face of libgrpo: the same calls as include/grpo.h, taking numpy
arrays (host calls) and torch tensors (device calls).

Marshalling only.  PyTorch supplies device memory and the current HIP stream;
every computation runs in libgrpo (host C++ or gfx950 kernels).  Device calls
insist on GPU tensors and never fall back to a CPU path.
"""

import ctypes

import numpy as np

from . import _capi as C
from ._capi import GrpoError, STATS_DTYPE, STATS_BYTES  # noqa: F401  (re-exported)

# ---------------------------------------------------------------- host calls


def version():
    return C.lib().grpo_version().decode()


def plan_fixed(batch, group_size, mini=0, micro=0):
    """-> (n_mini, n_micro, mini_rows, micro_rows).  See grpo_plan_fixed."""
    o = [ctypes.c_int64() for _ in range(4)]
    C.check(C.lib().grpo_plan_fixed(batch, group_size, mini, micro, *[ctypes.byref(x) for x in o]))
    return tuple(x.value for x in o)


def plan_chunk(batch, mini_rows, micro_rows, i_mini, j_micro):
    """-> (row_begin, row_end) of chunk (i, j)."""
    b, e = ctypes.c_int64(), ctypes.c_int64()
    C.check(C.lib().grpo_plan_chunk(batch, mini_rows, micro_rows, i_mini, j_micro, ctypes.byref(b), ctypes.byref(e)))
    return b.value, e.value


def plan_epochs(batch, group_size, mini=0, micro=0, mu=1, shuffle=False, seed=0):
    """Inner epochs with an optional seeded shuffle -> dict(n_mini, n_micro,
    mini_rows, micro_rows, mu, perm [mu x batch] int64).  See grpo_plan_epochs."""
    o = [ctypes.c_int64() for _ in range(4)]
    perm = np.zeros(max(mu, 1) * max(batch, 1), np.int64)
    C.check(C.lib().grpo_plan_epochs(batch, group_size, mini, micro, mu, 1 if shuffle else 0, seed & (2 ** 64 - 1),
                                     *[ctypes.byref(x) for x in o], C.ptr64(perm)))
    return {"n_mini": o[0].value, "n_micro": o[1].value, "mini_rows": o[2].value, "micro_rows": o[3].value,
            "mu": mu, "perm": perm[:mu * batch].reshape(mu, batch)}


def plan_dynamic(lengths, token_budget, proxy_div=4096):
    """Token-budget packing -> dict(n_bins, bin_off, order, restore) (int64 arrays)."""
    L = np.ascontiguousarray(lengths, dtype=np.int64)
    n = L.shape[0]
    order = np.zeros(max(n, 1), np.int64)
    restore = np.zeros(max(n, 1), np.int64)
    cap = 8
    while True:
        nb = ctypes.c_int64()
        off = np.zeros(cap + 1, np.int64)
        code = C.lib().grpo_plan_dynamic(C.ptr64(L), n, token_budget, proxy_div, cap, ctypes.byref(nb),
                                         C.ptr64(off), C.ptr64(order), C.ptr64(restore))
        if code == -7:           # ECAPACITY: grow to the reported need
            cap = nb.value
            continue
        C.check(code)
        k = nb.value
        return {"n_bins": k, "bin_off": off[:k + 1].copy(), "order": order[:n].copy(),
                "restore": restore[:n].copy()}


def plan_compaction(rows_per_rollout, n_groups, group_size, Q, expected_rollouts, dynamic=False):
    """Context-compaction rows -> dict of int arrays (see grpo_plan_compaction)."""
    R = np.ascontiguousarray(rows_per_rollout, dtype=np.int32)
    n = R.shape[0]
    cap = max(1, int(R.sum()) + n_groups * max(Q - 1, 0)) if n else 1
    out_n = ctypes.c_int64()
    rr = np.zeros(cap, np.int32)
    rs = np.zeros(cap, np.int32)
    src = np.zeros(cap, np.int32)
    pad = np.zeros(cap, np.uint8)
    gp = np.zeros(max(n_groups, 1), np.int32)
    C.check(C.lib().grpo_plan_compaction(C.ptr32(R), n, n_groups, group_size, Q, expected_rollouts,
                                         1 if dynamic else 0, cap, ctypes.byref(out_n), C.ptr32(rr),
                                         C.ptr32(rs), C.ptr32(src), C.ptru8(pad), C.ptr32(gp)))
    k = out_n.value
    return {"n_rows": k, "row_rollout": rr[:k].copy(), "row_seg": rs[:k].copy(), "row_src": src[:k].copy(),
            "is_pad": pad[:k].copy(), "group_pad": gp[:n_groups].copy()}


def row_offsets(lengths, order=None):
    L = np.ascontiguousarray(lengths, dtype=np.int64)
    n = L.shape[0]
    off = np.zeros(n + 1, np.int64)
    if order is None:
        C.check(C.lib().grpo_row_offsets(C.ptr64(L), None, n, C.ptr64(off)))
    else:
        O = np.ascontiguousarray(order, dtype=np.int64)
        C.check(C.lib().grpo_row_offsets(C.ptr64(L), C.ptr64(O), n, C.ptr64(off)))
    return off


def plan_trace(stage, calls, call_step, row_len, row_valid, row_uid, row_traj, V, T=0, dtype="bf16",
               row_seg=None, row_is_pad=None):
    """Trace of a plan (grpo_plan_trace) -> list of dicts, one per JSON line.

    ``calls``: the rows of each training call in visiting order (a list of
    int sequences); ``call_step``: the optimizer step of each call; per-row
    arrays over the batch's rows."""
    import json
    n_rows = len(row_len)
    a64 = lambda x: np.ascontiguousarray(x, dtype=np.int64)  # noqa: E731
    a32 = lambda x: np.ascontiguousarray(x, dtype=np.int32)  # noqa: E731
    off = a64(np.concatenate([[0], np.cumsum([len(c) for c in calls])]))
    rows = a64(np.concatenate([np.asarray(c, np.int64) for c in calls]) if calls else np.zeros(0))
    keep = [a64(row_len), a64(row_valid), a32(row_uid), a32(row_traj), a64(call_step), off, rows]
    seg = a32(row_seg) if row_seg is not None else None
    pad = np.ascontiguousarray(row_is_pad, dtype=np.uint8) if row_is_pad is not None else None
    vp = lambda x: x.ctypes.data if x is not None and x.size else None  # noqa: E731
    plan = C.TracePlan(struct_size=ctypes.sizeof(C.TracePlan), dtype=C.GRPO_BF16 if dtype == "bf16" else C.GRPO_F32,
                       stage=stage.encode(), n_rows=n_rows, T=T, V=V, row_len=vp(keep[0]), row_valid=vp(keep[1]),
                       row_uid=vp(keep[2]), row_traj=vp(keep[3]), row_seg=vp(seg), row_is_pad=vp(pad),
                       n_calls=len(calls), call_off=vp(off), call_rows=vp(rows), call_step=vp(keep[4]))
    need = ctypes.c_size_t()
    code = C.lib().grpo_plan_trace(ctypes.byref(plan), None, 0, ctypes.byref(need))
    if code != -7:
        C.check(code)
    buf = ctypes.create_string_buffer(need.value)
    C.check(C.lib().grpo_plan_trace(ctypes.byref(plan), buf, need.value, ctypes.byref(need)))
    return [json.loads(line) for line in buf.value.decode().splitlines()]


def group_advantage(reward, group_size, eps=1e-6, norm_by_std=True):
    r = np.ascontiguousarray(reward, dtype=np.float32)
    out = np.zeros(max(r.shape[0], 1), np.float32)
    C.check(C.lib().grpo_group_advantage(C.ptrf32(r), r.shape[0], group_size, eps, 1 if norm_by_std else 0,
                                         C.ptrf32(out)))
    return out[:r.shape[0]]


def rows_advantage(adv_rollout, row_rollout):
    a = np.ascontiguousarray(adv_rollout, dtype=np.float32)
    rr = np.ascontiguousarray(row_rollout, dtype=np.int32)
    out = np.zeros(max(rr.shape[0], 1), np.float32)
    C.check(C.lib().grpo_rows_advantage(C.ptrf32(a), a.shape[0], C.ptr32(rr), rr.shape[0], C.ptrf32(out)))
    return out[:rr.shape[0]]


class Accumulator:
    """Host step accumulator (grpo_accum_*): add() returns 'OK', 'NONFINITE' or
    'SKIPPED'; finalize() returns a dict or None."""

    def __init__(self, n_micro):
        self._L = C.lib()
        n = int(self._L.grpo_accum_size())
        self._a = (ctypes.c_int64 * ((n + 7) // 8))()     # opaque bytes, 8-byte aligned
        self._s = C.Stats()
        self._s_ref = ctypes.byref(self._s)
        C.check(self._L.grpo_accum_init(self._a, n_micro))

    def add(self, stats):
        s = C.Stats(**{k: stats.get(k, 0) for k in STATS_DTYPE.names})
        return self._add(s)

    def add_rows(self, raw, start, n):
        """Adds one chunk given as rows start .. start+n of a host array of
        grpo_stats (uint8 bytes, STATS_BYTES per row): the rows are summed in
        order by grpo_stats_sum, no Python arithmetic."""
        if not isinstance(raw, np.ndarray) or not raw.flags.c_contiguous or raw.dtype != np.uint8:
            raise ValueError("raw must be a C-contiguous uint8 array of grpo_stats")
        if start < 0 or n < 0 or (start + n) * STATS_BYTES > raw.nbytes:
            raise ValueError("rows outside the stats array")
        return self.add_rows_at(raw.ctypes.data + start * STATS_BYTES, n)

    def add_rows_at(self, addr, n):
        """add_rows on n grpo_stats at host address ``addr`` (the caller keeps
        them alive and in bounds)."""
        C.check(self._L.grpo_stats_sum(addr, n, self._s_ref))
        return self._add_ref()

    def _add(self, s):
        ctypes.memmove(ctypes.byref(self._s), ctypes.byref(s), ctypes.sizeof(C.Stats))
        return self._add_ref()

    def _add_ref(self):
        code = self._L.grpo_accum_add(self._a, self._s_ref)
        if code == 0:
            return "OK"
        if code == -5:
            return "NONFINITE"
        if code == -6:
            return "SKIPPED"
        if code == -9:
            return "STATE"
        C.check(code)

    def finalize(self):
        r = C.StepResult()
        stepped = ctypes.c_int32()
        C.check(C.lib().grpo_accum_finalize(self._a, ctypes.byref(r), ctypes.byref(stepped)))
        if not stepped.value:
            return None
        return {k: getattr(r, k) for k, _ in C.StepResult._fields_}


def needs_ahead_pass(n_mini, use_rollout_logprobs=False, consumes_old_logprobs=True):
    return bool(C.lib().grpo_needs_ahead_pass(n_mini, 1 if use_rollout_logprobs else 0,
                                              1 if consumes_old_logprobs else 0))


class OldLogprobCache:
    """grpo_old_cache: pi_old records of one collected batch keyed by call
    order, in a caller-owned device buffer (a float32 torch tensor)."""

    def __init__(self, n_calls, buf):
        torch = _torch()
        if buf.dtype != torch.float32 or not buf.is_cuda or not buf.is_contiguous():
            raise ValueError("buf must be a contiguous float32 GPU tensor")
        self.buf = buf
        self.off = np.zeros(n_calls + 1, np.int64)
        self.c = C.OldCache()
        C.check(C.lib().grpo_old_cache_init(ctypes.byref(self.c), ctypes.c_void_p(buf.data_ptr()), buf.numel(),
                                            C.ptr64(self.off), n_calls))

    def reset(self):
        C.check(C.lib().grpo_old_cache_reset(ctypes.byref(self.c)))

    def _view(self, addr, n):
        start = (addr - self.buf.data_ptr()) // 4 if n else 0
        return self.buf[start:start + n]

    def record(self, logits, target, mask, paired=False, on_launch=None):
        """Ahead pass of one chunk into the next record; returns its view.
        ``paired``: grpo_old_cache_record_paired (the record equals the fused
        loss's log-probs bit for bit on unchanged logits).  ``on_launch``: as
        in loss_fwd_bwd."""
        n, V = logits.shape
        ld = _matrix(logits, "logits", n, V)
        slot = ctypes.c_void_p()
        entry = C.lib().grpo_old_cache_record_paired if paired else C.lib().grpo_old_cache_record
        args = (_stream(), ctypes.byref(self.c), _dtype_code(logits), logits.data_ptr(), ld, n, V,
                _need(target, "target", "int32", n), _need(mask, "mask", "byte", n), ctypes.byref(slot))
        if on_launch is not None:
            on_launch()
        C.check(entry(*args))
        return self._view(slot.value or 0, n)

    def rewind(self):
        """Replay the records again from call 0 (the next unshuffled epoch)."""
        C.check(C.lib().grpo_old_cache_rewind(ctypes.byref(self.c)))

    def replay(self, n_tok):
        """pi_old of the next training call (a view of the buffer)."""
        ptr = ctypes.c_void_p()
        C.check(C.lib().grpo_old_cache_replay(ctypes.byref(self.c), n_tok, ctypes.byref(ptr)))
        return self._view(ptr.value or 0, n_tok)

    @property
    def recorded(self):
        return self.c.recorded

    @property
    def replayed(self):
        return self.c.replayed


PROBE_STATS_BYTES = ctypes.sizeof(C.ProbeStats)


def probe_compare(recorded, rescored, mask, bound=C.PROBE_STRICT_BOUND, out=None):
    """Device compare of two log-prob arrays -> uint8 device tensor holding a
    grpo_probe_stats (see probe_stats)."""
    torch = _torch()
    if out is None:
        out = torch.empty(PROBE_STATS_BYTES, dtype=torch.uint8, device=recorded.device)
    n = mask.numel()
    C.check(C.lib().grpo_probe_compare(_stream(), _need(recorded, "recorded", "float32", n),
                                       _need(rescored, "rescored", "float32", n), _need(mask, "mask", "byte", n),
                                       n, bound, _need(out, "out", "byte", PROBE_STATS_BYTES)))
    return out


def probe_stats(raw):
    b = raw.cpu().numpy().tobytes() if hasattr(raw, "cpu") else bytes(raw)
    s = C.ProbeStats.from_buffer_copy(b)
    return {"n_valid": s.n_valid, "n_moved": s.n_moved, "max_abs": s.max_abs}


class Probe:
    """grpo_probe: the one-shot determinism screen of a run."""

    def __init__(self, bound=C.PROBE_STRICT_BOUND, max_fraction=C.PROBE_STRICT_FRACTION):
        self.p = C.Probe()
        C.check(C.lib().grpo_probe_init(ctypes.byref(self.p), bound, max_fraction))

    def due(self):
        return not self.p.done

    def finish(self, stats):
        s = C.ProbeStats(stats["n_valid"], stats["n_moved"], stats["max_abs"])
        passed = ctypes.c_int32()
        C.check(C.lib().grpo_probe_finish(ctypes.byref(self.p), ctypes.byref(s), ctypes.byref(passed)))
        return bool(passed.value)


def stats_to_dicts(raw):
    """uint8 bytes of a grpo_stats array (numpy or torch) -> list of dicts."""
    if hasattr(raw, "cpu"):
        raw = raw.cpu().numpy()
    arr = np.ascontiguousarray(raw).view(STATS_DTYPE).reshape(-1)
    return [{k: (float(a[k]) if k.endswith("_sum") else int(a[k])) for k in STATS_DTYPE.names} for a in arr]


# ---------------------------------------------------------------- device calls

def _torch():
    import torch
    return torch


def _need(t, name, dtype, n, optional=False):
    """Device address of ``t``: a contiguous GPU tensor of element type
    ``dtype`` ("int32", "int64", "float32", "bfloat16", or "byte" for uint8 or
    bool) holding at least ``n`` elements; None for an absent optional one.
    libgrpo sees only addresses, so every length it will read or write is
    checked here, before the call."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libgrpo has no CPU path)")
    kind = str(t.dtype).removeprefix("torch.")
    if kind not in (("uint8", "bool") if dtype == "byte" else (dtype,)):
        raise ValueError(f"{name} must hold {dtype} elements, not {kind}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements; the call uses {n}")
    return t.data_ptr()


def _matrix(t, name, rows, cols, dtypes=("bfloat16", "float32"), dense=False):
    """Row stride of a GPU matrix of at least ``rows`` rows and exactly
    ``cols`` columns with unit stride along a row (``dense``: no row padding)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libgrpo has no CPU path)")
    kind = str(t.dtype).removeprefix("torch.")
    if kind not in dtypes:
        raise ValueError(f"{name} must hold {' or '.join(dtypes)} elements, not {kind}")
    ld = _rows2d(t, name)
    if t.shape[0] < rows or t.shape[1] != cols:
        raise ValueError(f"{name} is {tuple(t.shape)}; the call needs at least {rows} rows of {cols}")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ld


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return C.GRPO_BF16
    if t.dtype == torch.float32:
        return C.GRPO_F32
    raise ValueError(f"unsupported logits dtype {t.dtype} (bf16 or fp32)")


def _rows2d(x, name):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit stride along the vocabulary")
    return x.stride(0)


def count_valid(mask, out=None):
    """Device int64 [1] tensor holding the number of non-zero mask bytes."""
    torch = _torch()
    if out is None:
        out = torch.empty(1, dtype=torch.int64, device=mask.device)
    C.check(C.lib().grpo_count_valid(_stream(), _need(mask, "mask", "byte", 0), mask.numel(),
                                     _need(out, "out", "int64", 1)))
    return out


def count_rows(mask, row_off, out=None):
    """Device int64 [1] tensor: rows holding a valid token (grpo_count_rows)."""
    torch = _torch()
    if out is None:
        out = torch.empty(1, dtype=torch.int64, device=mask.device)
    C.check(C.lib().grpo_count_rows(_stream(), _need(mask, "mask", "byte", 0), _need(row_off, "row_off", "int64", 1),
                                    row_off.numel() - 1, mask.numel(), _need(out, "out", "int64", 1)))
    return out


def row_weights(mask, row_off, mode, n_seq, out=None):
    """Per-row float32 gradient factors of an aggregation mode (grpo_row_weights);
    ``n_seq`` is the device int64 count from count_rows over the mini-batch."""
    torch = _torch()
    n_rows = row_off.numel() - 1
    if out is None:
        out = torch.empty(max(n_rows, 1), dtype=torch.float32, device=mask.device)
    C.check(C.lib().grpo_row_weights(_stream(), _need(mask, "mask", "byte", 0), _need(row_off, "row_off", "int64", 1),
                                     n_rows, mask.numel(), mode, _need(n_seq, "n_seq", "int64", 1),
                                     _need(out, "w_row", "float32", n_rows)))
    return out


def chunk_tok_src(src_row_off, rows, dst_row_off, out=None):
    """Batch token index of each token of a chunk of batch ``rows`` (device
    int64 tensors), grpo_chunk_tok_src."""
    torch = _torch()
    n_tok = int(dst_row_off[-1].item()) if out is None else out.numel()
    if out is None:
        out = torch.empty(max(n_tok, 1), dtype=torch.int64, device=rows.device)
    C.check(C.lib().grpo_chunk_tok_src(_stream(), _need(src_row_off, "src_row_off", "int64", 1),
                                       src_row_off.numel() - 1, _need(rows, "rows", "int64", 0), rows.numel(),
                                       _need(dst_row_off, "dst_row_off", "int64", rows.numel() + 1), n_tok,
                                       _need(out, "tok_src", "int64", n_tok)))
    return out[:n_tok]


def gather(src, idx, out=None):
    """dst[k] = src[idx[k]] on the device (grpo_gather); 1-, 2-, 4- or 8-byte elements."""
    torch = _torch()
    if out is None:
        out = torch.empty(idx.numel(), dtype=src.dtype, device=src.device)
    if out.dtype != src.dtype:
        raise ValueError(f"out must hold {src.dtype} elements like src, not {out.dtype}")
    kind = str(src.dtype).removeprefix("torch.")
    C.check(C.lib().grpo_gather(_stream(), _need(src, "src", kind, 0), src.numel(),
                                _need(idx, "idx", "int64", 0), idx.numel(), src.element_size(),
                                _need(out, "dst", kind, idx.numel())))
    return out


def tok_row(row_off, n_tok, out=None):
    torch = _torch()
    if out is None:
        out = torch.empty(n_tok, dtype=torch.int32, device=row_off.device)
    C.check(C.lib().grpo_tok_row(_stream(), _need(row_off, "row_off", "int64", 1), row_off.numel() - 1, n_tok,
                                 _need(out, "tok_row", "int32", n_tok)))
    return out


def logprob_fwd(logits, target, mask, want_lse=True, want_entropy=True, paired=False, out=None):
    """Forward-only per-token (logp, lse, entropy) float32 tensors.

    ``paired``: grpo_logprob_fwd_paired, whose sums run in the fused loss's
    lane partition, so the results equal loss_fwd_bwd's bit for bit where the
    fused loss keeps the row on chip.  ``out``: a float32 tensor of n_tok
    elements that receives logp (for instance a slice of a pi_old cache)."""
    torch = _torch()
    n, V = logits.shape
    ld = _matrix(logits, "logits", n, V)
    if out is not None:
        _need(out, "out", "float32", n)
        logp = out
    else:
        logp = torch.empty(n, dtype=torch.float32, device=logits.device)
    lse = torch.empty(n, dtype=torch.float32, device=logits.device) if want_lse else None
    ent = torch.empty(n, dtype=torch.float32, device=logits.device) if want_entropy else None
    entry = C.lib().grpo_logprob_fwd_paired if paired else C.lib().grpo_logprob_fwd
    C.check(entry(_stream(), _dtype_code(logits), logits.data_ptr(), ld, n, V,
                                     _need(target, "target", "int32", n), _need(mask, "mask", "byte", n),
                                     logp.data_ptr(), lse.data_ptr() if lse is not None else None,
                                     ent.data_ptr() if ent is not None else None))
    return logp, lse, ent


def loss_workspace(n_tok, n_rows, device):
    """Per-token and per-row output buffers for loss_fwd_bwd."""
    torch = _torch()
    f = dict(dtype=torch.float32, device=device)
    return {"logp": torch.empty(n_tok, **f), "lse": torch.empty(n_tok, **f), "entropy": torch.empty(n_tok, **f),
            "loss_tok": torch.empty(n_tok, **f), "kl_tok": torch.empty(n_tok, **f),
            "tok_flags": torch.empty(n_tok, dtype=torch.uint8, device=device),
            "row_stats": torch.empty((max(n_rows, 1), STATS_BYTES), dtype=torch.uint8, device=device),
            "chunk_stats": torch.empty((1, STATS_BYTES), dtype=torch.uint8, device=device)}


def _set_terms(a, row_weight, ref_logp, ent_coef, kl_coef, kl_type, ws, n_rows, n_tok, n_src):
    a.row_weight = _need(row_weight, "row_weight", "float32", n_rows, optional=True)
    a.ref_logp = _need(ref_logp, "ref_logp", "float32", n_src, optional=True)
    a.kl_tok = _need(ws.get("kl_tok"), "kl_tok", "float32", n_tok) if ref_logp is not None else None
    a.ent_coef, a.kl_coef, a.kl_type = ent_coef, kl_coef, kl_type


def _set_common(a, target, mask, old_logp, tok_row_, adv_row, row_off, denom, ws, n, n_src, stats=True):
    """The per-token inputs (``n_src`` tokens behind them), the chunk-local row
    arrays and the per-token / per-row outputs shared by both loss calls
    (``stats`` False: the row and chunk reductions are deferred)."""
    n_rows = row_off.numel() - 1
    a.target = _need(target, "target", "int32", n_src)
    a.mask = _need(mask, "mask", "byte", n_src)
    a.old_logp = _need(old_logp, "old_logp", "float32", n_src)
    a.tok_row = _need(tok_row_, "tok_row", "int32", n)
    a.adv_row = _need(adv_row, "adv_row", "float32", n_rows)
    a.row_off = _need(row_off, "row_off", "int64", 1)
    a.n_rows = n_rows
    a.denom = _need(denom, "denom", "int64", 1, optional=True)
    for k in ("logp", "entropy", "loss_tok"):
        setattr(a, k, _need(ws.get(k), k, "float32", n))
    a.lse = _need(ws.get("lse"), "lse", "float32", n, optional=True)
    a.tok_flags = _need(ws.get("tok_flags"), "tok_flags", "byte", n)
    if stats:
        a.row_stats = _need(ws.get("row_stats"), "row_stats", "byte", n_rows * STATS_BYTES)
        a.chunk_stats = _need(ws.get("chunk_stats"), "chunk_stats", "byte", STATS_BYTES)
    if not n:                       # nothing per token is touched
        a.target = a.mask = a.old_logp = a.tok_row = None
        a.logp = a.lse = a.entropy = a.loss_tok = a.tok_flags = None
    if not n_rows:
        a.adv_row = None


def loss_fwd_bwd(logits, target, mask, old_logp, tok_row_, adv_row, row_off, *, scale=1.0, denom=None,
                 eps_low=0.2, eps_high=0.2, dlogits="new", out_dtype=None, ws=None, row_weight=None,
                 ref_logp=None, ent_coef=0.0, kl_coef=0.0, kl_type=C.KL_K3, tok_src=None, defer_stats=False,
                 on_launch=None):
    """Fused GRPO loss forward/backward over one chunk (grpo_loss_fwd_bwd).

    ``defer_stats``: leave the row and chunk reductions to a later
    ``loss_stats`` call (GRPO_LOSS_DEFER_STATS).

    ``dlogits``: "new" (allocate, dtype ``out_dtype`` or the logits dtype),
    "inplace" (overwrite ``logits``), None (no gradient), or a tensor.
    ``row_weight`` / ``ref_logp`` / ``ent_coef`` / ``kl_coef`` / ``kl_type``:
    the aggregation weights and extra terms (``ws["kl_tok"]`` receives the
    per-token KL when ``ref_logp`` is given).
    ``tok_src``: a chunk of batch rows in any order -- ``logits``,
    ``target``, ``mask``, ``old_logp``, ``ref_logp`` and ``dlogits`` are then
    the whole batch's, read and written at tok_src[t]; the chunk's token count
    is tok_src's length.
    Every tensor's device, element type and length are checked against what
    the call will touch before anything is launched (ValueError).
    ``on_launch``: called with no arguments after the arguments are checked
    and marshalled, right before the library call (a timing hook: an event
    recorded there brackets the launch, not the Python work before it).
    Returns the workspace dict with ``dlogits`` added."""
    torch = _torch()
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [tokens x V]")
    n_src, V = logits.shape
    ld = _matrix(logits, "logits", n_src, V)
    n = n_src
    if tok_src is not None:
        _need(tok_src, "tok_src", "int64", 0)
        n = tok_src.numel()
    n_rows = row_off.numel() - 1
    if ws is None:
        ws = loss_workspace(n, n_rows, logits.device)
    if isinstance(dlogits, str) and dlogits == "new":
        dl = torch.empty((n_src, V), dtype=out_dtype or logits.dtype, device=logits.device)
    elif isinstance(dlogits, str) and dlogits == "inplace":
        dl = logits
    else:
        dl = dlogits
    a = C.LossArgs()
    a.struct_size = ctypes.sizeof(C.LossArgs)
    a.in_dtype = _dtype_code(logits)
    a.out_dtype = _dtype_code(dl) if dl is not None else a.in_dtype
    a.logits = logits.data_ptr() if n else None
    a.ld, a.n_tok, a.V = ld, n, V
    _set_common(a, target, mask, old_logp, tok_row_, adv_row, row_off, denom, ws, n, n_src, stats=not defer_stats)
    a.flags = C.LOSS_DEFER_STATS if defer_stats else 0
    a.eps_low, a.eps_high, a.scale = eps_low, eps_high, scale
    if dl is not None:
        a.ld_out = _matrix(dl, "dlogits", n_src, V)
        a.dlogits = dl.data_ptr() if n else None
    _set_terms(a, row_weight, ref_logp, ent_coef, kl_coef, kl_type, ws, n_rows, n, n_src)
    if tok_src is not None:
        a.tok_src = tok_src.data_ptr() if n else None
        a.n_src = n_src
    if on_launch is not None:
        on_launch()
    C.check(C.lib().grpo_loss_fwd_bwd(_stream(), ctypes.byref(a)))
    ws["dlogits"] = dl
    return ws


def loss_stats(ws, row_off, *, scale=1.0, denom=None, row_weight=None, with_kl=False, ent_coef=0.0, kl_coef=0.0):
    """Row and chunk reductions (grpo_loss_stats) over the per-token outputs in
    ``ws`` (loss_tok, entropy, tok_flags, and kl_tok with ``with_kl``) of the
    rows ``row_off``, into ws["row_stats"] and ws["chunk_stats"]; the factor
    fields are the ones the tokens were computed with."""
    n_rows = row_off.numel() - 1
    n = ws["loss_tok"].numel()
    a = C.LossArgs()
    a.struct_size = ctypes.sizeof(C.LossArgs)
    a.n_tok, a.n_rows = n, n_rows
    a.row_off = _need(row_off, "row_off", "int64", n_rows + 1)
    for k in ("entropy", "loss_tok"):
        setattr(a, k, _need(ws.get(k), k, "float32", n))
    a.tok_flags = _need(ws.get("tok_flags"), "tok_flags", "byte", n)
    a.row_stats = _need(ws.get("row_stats"), "row_stats", "byte", n_rows * STATS_BYTES)
    a.chunk_stats = _need(ws.get("chunk_stats"), "chunk_stats", "byte", STATS_BYTES)
    a.denom = _need(denom, "denom", "int64", 1, optional=True)
    a.row_weight = _need(row_weight, "row_weight", "float32", n_rows, optional=True)
    if with_kl:
        a.kl_tok = _need(ws.get("kl_tok"), "kl_tok", "float32", n)
        a.ref_logp = a.kl_tok          # marks the KL term as present; not read
    a.scale, a.ent_coef, a.kl_coef = scale, ent_coef, kl_coef
    C.check(C.lib().grpo_loss_stats(_stream(), ctypes.byref(a)))
    return ws


def stats_sum(rows):
    """Sum of grpo_stats dicts in order (grpo_stats_sum) -> dict."""
    n = len(rows)
    arr = (C.Stats * max(n, 1))()
    for i, r in enumerate(rows):
        arr[i] = C.Stats(**{k: r.get(k, 0) for k in STATS_DTYPE.names})
    out = C.Stats()
    C.check(C.lib().grpo_stats_sum(ctypes.addressof(arr), n, ctypes.byref(out)))
    return {k: (float(getattr(out, k)) if k.endswith("_sum") else int(getattr(out, k))) for k in STATS_DTYPE.names}


def transpose_bf16(x, out=None):
    """bf16 [rows x cols] -> its transpose [cols x rows] (grpo_transpose_bf16)."""
    torch = _torch()
    if x.dtype != torch.bfloat16:
        raise ValueError("transpose_bf16 takes a bf16 matrix")
    rows, cols = x.shape
    ld = _matrix(x, "x", rows, cols, ("bfloat16",))
    if out is None:
        out = torch.empty((cols, rows), dtype=torch.bfloat16, device=x.device)
    ld_out = _matrix(out, "out", cols, rows, ("bfloat16",))
    C.check(C.lib().grpo_transpose_bf16(_stream(), x.data_ptr(), rows, cols, ld, out.data_ptr(), ld_out))
    return out


def lmhead_workspace_bytes(n_tok, H, V, keep_z=False, defer_dw=False):
    flags = (C.LMHEAD_KEEP_Z if keep_z else 0) | (C.LMHEAD_DEFER_DW if defer_dw else 0)
    if flags:
        return int(C.lib().grpo_lmhead_workspace_size_flags(n_tok, H, V, flags))
    return int(C.lib().grpo_lmhead_workspace_size(n_tok, H, V))


def lmhead_dw_window_bytes(cap_tok, H, V):
    return int(C.lib().grpo_lmhead_dw_window_size(cap_tok, H, V))


class LmheadDwWindow:
    """grpo_lmhead_dw_window: h^T and dz^T of several LM-head chunks, so that
    dW takes one GEMM per flush instead of one per chunk.  ``buf``: a
    contiguous uint8 GPU tensor of at least lmhead_dw_window_bytes bytes
    (allocated here when None)."""

    def __init__(self, cap_tok, H, V, device=None, buf=None):
        torch = _torch()
        if buf is None:
            buf = torch.empty(max(lmhead_dw_window_bytes(cap_tok, H, V), 1), dtype=torch.uint8, device=device)
        if buf.dtype != torch.uint8 or not buf.is_cuda or not buf.is_contiguous():
            raise ValueError("buf must be a contiguous uint8 GPU tensor")
        self.buf = buf
        self.w = C.DwWindow()
        C.check(C.lib().grpo_lmhead_dw_window_init(_stream(), ctypes.byref(self.w), ctypes.c_void_p(buf.data_ptr()),
                                                   buf.numel(), cap_tok, H, V))

    def flush(self, dW, on_launch=None):
        """dW (fp32 [V x H]) += the window's dz^T h; empties the window."""
        _matrix(dW, "dW", self.w.V, self.w.H, ("float32",), dense=True)
        if dW.shape[0] != self.w.V:
            raise ValueError(f"dW must be [{self.w.V} x {self.w.H}]")
        if on_launch is not None:
            on_launch()
        C.check(C.lib().grpo_lmhead_dw_flush(_stream(), ctypes.byref(self.w), ctypes.c_void_p(dW.data_ptr())))

    @property
    def reserved(self):
        return self.w.reserved


def lmhead_fwd_bwd(h, W, Wt, target, mask, old_logp, tok_row_, adv_row, row_off, dW, *, scale=1.0, denom=None,
                   eps_low=0.2, eps_high=0.2, dh=None, ws=None, workspace=None, row_weight=None,
                   ref_logp=None, ent_coef=0.0, kl_coef=0.0, kl_type=C.KL_K3, noalloc=False, keep_z=False,
                   dw_window=None, on_launch=None):
    """Fused LM-head GRPO loss over one chunk (grpo_lmhead_fwd_bwd).

    ``dW`` (fp32 [V x H]) is accumulated into; ``dh`` (fp32 [n_tok x H]) is
    written.  Shapes, element types and lengths are checked before the call
    (ValueError).  Returns the per-token workspace dict with ``dh`` added.
    ``noalloc``: call grpo_lmhead_fwd_bwd_noalloc, which uses the library's
    fixed scratch (no workspace is passed; the caller still provides every
    input and output).  ``keep_z``: GRPO_LMHEAD_KEEP_Z (pass 1 keeps the
    chunk's fp32 logits in the workspace and pass 2 reads them back instead
    of recomputing them).  ``dw_window`` (an LmheadDwWindow): GRPO_LMHEAD_DEFER_DW,
    the chunk's h^T and dz^T go to the window and dW (which may then be None)
    is left for the window's flush.  ``on_launch``: as in loss_fwd_bwd."""
    torch = _torch()
    if h.dim() != 2 or W.dim() != 2:
        raise ValueError("h and W must be 2-D")
    n, H = h.shape
    V = W.shape[0]
    n_rows = row_off.numel() - 1
    if ws is None:
        ws = loss_workspace(n, n_rows, h.device)
    if dh is None:
        dh = torch.empty((n, H), dtype=torch.float32, device=h.device)
    if workspace is None and not noalloc:
        workspace = torch.empty(max(lmhead_workspace_bytes(n, H, V, keep_z, dw_window is not None), 1),
                                dtype=torch.uint8, device=h.device)
    a = C.LmheadArgs()
    a.struct_size = ctypes.sizeof(C.LmheadArgs)
    a.flags = (C.LMHEAD_KEEP_Z if keep_z else 0) | (C.LMHEAD_DEFER_DW if dw_window is not None else 0)
    a.dw_window = ctypes.addressof(dw_window.w) if dw_window is not None else None
    a.ldh = _matrix(h, "h", n, H, ("bfloat16",))
    a.h = h.data_ptr() if n else None
    _matrix(W, "W", V, H, ("bfloat16",), dense=True)
    _matrix(Wt, "Wt", H, V, ("bfloat16",), dense=True)
    if W.shape[0] != V or Wt.shape[0] != H:
        raise ValueError(f"W must be [{V} x {H}] and Wt [{H} x {V}]")
    a.W, a.Wt = W.data_ptr(), Wt.data_ptr()
    a.n_tok, a.H, a.V = n, H, V
    _set_common(a, target, mask, old_logp, tok_row_, adv_row, row_off, denom, ws, n, n)
    a.eps_low, a.eps_high, a.scale = eps_low, eps_high, scale
    _matrix(dh, "dh", n, H, ("float32",), dense=True)
    a.dh = dh.data_ptr() if n else None
    if dW is None:
        if dw_window is None:
            raise ValueError("dW is required unless a dW window takes the chunk")
        a.dW = None
    else:
        _matrix(dW, "dW", V, H, ("float32",), dense=True)
        if dW.shape[0] != V:
            raise ValueError(f"dW must be [{V} x {H}]")
        a.dW = dW.data_ptr()
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc calls take no workspace")
        a.workspace, a.workspace_bytes = None, 0
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    _set_terms(a, row_weight, ref_logp, ent_coef, kl_coef, kl_type, ws, n_rows, n, n)
    entry = C.lib().grpo_lmhead_fwd_bwd_noalloc if noalloc else C.lib().grpo_lmhead_fwd_bwd
    if on_launch is not None:
        on_launch()
    C.check(entry(_stream(), ctypes.byref(a)))
    ws["dh"] = dh
    ws["workspace"] = workspace
    return ws
