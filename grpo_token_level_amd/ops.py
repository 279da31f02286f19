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
from ._capi import STREAM_COPY, STREAM_READ, STREAM_FILL  # noqa: F401  (re-exported)

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
        self._a = C.Accum()
        C.check(C.lib().grpo_accum_init(ctypes.byref(self._a), n_micro))

    def add(self, stats):
        s = C.Stats(**{k: stats.get(k, 0) for k in STATS_DTYPE.names})
        code = C.lib().grpo_accum_add(ctypes.byref(self._a), ctypes.byref(s))
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
        C.check(C.lib().grpo_accum_finalize(ctypes.byref(self._a), ctypes.byref(r), ctypes.byref(stepped)))
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

    def record(self, logits, target, mask):
        """Ahead pass of one chunk into the next record; returns its view."""
        ld = _rows2d(logits, "logits")
        n, V = logits.shape
        slot = ctypes.c_void_p()
        C.check(C.lib().grpo_old_cache_record(_stream(), ctypes.byref(self.c), _dtype_code(logits),
                                              _dev(logits, "logits"), ld, n, V, _dev(target, "target"),
                                              _dev(mask, "mask"), ctypes.byref(slot)))
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
    C.check(C.lib().grpo_probe_compare(_stream(), _dev(recorded, "recorded"), _dev(rescored, "rescored"),
                                       _dev(mask, "mask"), mask.numel(), bound, _dev(out, "out")))
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


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libgrpo has no CPU path)")
    if not t.is_contiguous() and t.dim() == 1:
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


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


def stream_probe(mode, src=None, dst=None, nbytes=None):
    """The measurement yardstick (grpo_stream_probe): a plain copy
    (STREAM_COPY, src -> dst), read (STREAM_READ, src; dst is 16 bytes of
    scratch) or zero fill (STREAM_FILL, dst) of ``nbytes`` bytes (default: the
    whole src, or dst for a fill).  Returns dst."""
    torch = _torch()
    if mode == C.STREAM_READ and dst is None:
        dst = torch.empty(16, dtype=torch.uint8, device=src.device)
    if mode not in (C.STREAM_COPY, C.STREAM_READ, C.STREAM_FILL):
        raise ValueError(f"unknown stream mode {mode}")
    size = lambda t: t.numel() * t.element_size()  # noqa: E731
    if nbytes is None:
        nbytes = size(dst if mode == C.STREAM_FILL else src)
    for t, name, need in ((src, "src", nbytes if mode != C.STREAM_FILL else 0),
                          (dst, "dst", 16 if mode == C.STREAM_READ else nbytes)):
        if need and (t is None or not t.is_cuda or not t.is_contiguous() or size(t) < need):
            raise ValueError(f"{name} must be a contiguous GPU tensor of at least {need} bytes")
    C.check(C.lib().grpo_stream_probe(_stream(), mode, ctypes.c_void_p(src.data_ptr()) if src is not None else None,
                                      ctypes.c_void_p(dst.data_ptr()), nbytes))
    return dst


def count_valid(mask, out=None):
    """Device int64 [1] tensor holding the number of non-zero mask bytes."""
    torch = _torch()
    if out is None:
        out = torch.empty(1, dtype=torch.int64, device=mask.device)
    C.check(C.lib().grpo_count_valid(_stream(), _dev(mask, "mask"), mask.numel(), _dev(out, "out")))
    return out


def count_rows(mask, row_off, out=None):
    """Device int64 [1] tensor: rows holding a valid token (grpo_count_rows)."""
    torch = _torch()
    if out is None:
        out = torch.empty(1, dtype=torch.int64, device=mask.device)
    C.check(C.lib().grpo_count_rows(_stream(), _dev(mask, "mask"), _dev(row_off, "row_off"), row_off.numel() - 1,
                                    mask.numel(), _dev(out, "out")))
    return out


def row_weights(mask, row_off, mode, n_seq, out=None):
    """Per-row float32 gradient factors of an aggregation mode (grpo_row_weights);
    ``n_seq`` is the device int64 count from count_rows over the mini-batch."""
    torch = _torch()
    n_rows = row_off.numel() - 1
    if out is None:
        out = torch.empty(max(n_rows, 1), dtype=torch.float32, device=mask.device)
    C.check(C.lib().grpo_row_weights(_stream(), _dev(mask, "mask"), _dev(row_off, "row_off"), n_rows, mask.numel(),
                                     mode, _dev(n_seq, "n_seq"), _dev(out, "w_row")))
    return out


def chunk_tok_src(src_row_off, rows, dst_row_off, out=None):
    """Batch token index of each token of a chunk of batch ``rows`` (device
    int64 tensors), grpo_chunk_tok_src."""
    torch = _torch()
    n_tok = int(dst_row_off[-1].item()) if out is None else out.numel()
    if out is None:
        out = torch.empty(max(n_tok, 1), dtype=torch.int64, device=rows.device)
    C.check(C.lib().grpo_chunk_tok_src(_stream(), _dev(src_row_off, "src_row_off"), src_row_off.numel() - 1,
                                       _dev(rows, "rows"), rows.numel(), _dev(dst_row_off, "dst_row_off"), n_tok,
                                       _dev(out, "tok_src")))
    return out[:n_tok]


def gather(src, idx, out=None):
    """dst[k] = src[idx[k]] on the device (grpo_gather); 1-, 2-, 4- or 8-byte elements."""
    torch = _torch()
    if out is None:
        out = torch.empty(idx.numel(), dtype=src.dtype, device=src.device)
    C.check(C.lib().grpo_gather(_stream(), _dev(src, "src"), src.numel(), _dev(idx, "idx"), idx.numel(),
                                src.element_size(), _dev(out, "dst")))
    return out


def tok_row(row_off, n_tok, out=None):
    torch = _torch()
    if out is None:
        out = torch.empty(n_tok, dtype=torch.int32, device=row_off.device)
    C.check(C.lib().grpo_tok_row(_stream(), _dev(row_off, "row_off"), row_off.numel() - 1, n_tok,
                                 _dev(out, "tok_row")))
    return out


def logprob_fwd(logits, target, mask, want_lse=True, want_entropy=True):
    """Forward-only per-token (logp, lse, entropy) float32 tensors."""
    torch = _torch()
    ld = _rows2d(logits, "logits")
    n, V = logits.shape
    logp = torch.empty(n, dtype=torch.float32, device=logits.device)
    lse = torch.empty_like(logp) if want_lse else None
    ent = torch.empty_like(logp) if want_entropy else None
    C.check(C.lib().grpo_logprob_fwd(_stream(), _dtype_code(logits), _dev(logits, "logits"), ld, n, V,
                                     _dev(target, "target"), _dev(mask, "mask"), _dev(logp, "logp"),
                                     _dev(lse, "lse"), _dev(ent, "entropy")))
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


def _set_terms(a, row_weight, ref_logp, ent_coef, kl_coef, kl_type, ws):
    for name, t in (("row_weight", row_weight), ("ref_logp", ref_logp)):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (libgrpo has no CPU path)")
    a.row_weight = row_weight.data_ptr() if row_weight is not None else None
    a.ref_logp = ref_logp.data_ptr() if ref_logp is not None else None
    a.kl_tok = ws["kl_tok"].data_ptr() if ref_logp is not None else None
    a.ent_coef, a.kl_coef, a.kl_type = ent_coef, kl_coef, kl_type


def loss_fwd_bwd(logits, target, mask, old_logp, tok_row_, adv_row, row_off, *, scale=1.0, denom=None,
                 eps_low=0.2, eps_high=0.2, dlogits="new", out_dtype=None, ws=None, row_weight=None,
                 ref_logp=None, ent_coef=0.0, kl_coef=0.0, kl_type=C.KL_K3, tok_src=None):
    """Fused GRPO loss forward/backward over one chunk (grpo_loss_fwd_bwd).

    ``dlogits``: "new" (allocate, dtype ``out_dtype`` or the logits dtype),
    "inplace" (overwrite ``logits``), None (no gradient), or a tensor.
    ``row_weight`` / ``ref_logp`` / ``ent_coef`` / ``kl_coef`` / ``kl_type``:
    the aggregation weights and extra terms (``ws["kl_tok"]`` receives the
    per-token KL when ``ref_logp`` is given).
    ``tok_src``: a chunk of batch rows in any order -- ``logits``,
    ``target``, ``mask``, ``old_logp``, ``ref_logp`` and ``dlogits`` are then
    the whole batch's, read and written at tok_src[t]; the chunk's token count
    is tok_src's length.
    Returns the workspace dict with ``dlogits`` added."""
    torch = _torch()
    ld = _rows2d(logits, "logits")
    n_src, V = logits.shape
    n = tok_src.numel() if tok_src is not None else n_src
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
    a.target = target.data_ptr() if n else None
    a.mask = mask.data_ptr() if n else None
    a.old_logp = old_logp.data_ptr() if n else None
    a.tok_row = tok_row_.data_ptr() if n else None
    a.adv_row = adv_row.data_ptr() if n_rows else None
    a.row_off = row_off.data_ptr()
    a.n_rows = n_rows
    a.eps_low, a.eps_high, a.scale = eps_low, eps_high, scale
    a.denom = denom.data_ptr() if denom is not None else None
    if dl is not None:
        a.dlogits = dl.data_ptr() if n else None
        a.ld_out = _rows2d(dl, "dlogits")
    for k in ("logp", "lse", "entropy", "loss_tok", "tok_flags", "row_stats", "chunk_stats"):
        t = ws[k]
        if t is not None and not t.is_cuda:
            raise ValueError(f"{k} must be a GPU tensor")
        setattr(a, k, t.data_ptr() if t is not None else None)
    for name, t in (("logits", logits), ("target", target), ("mask", mask), ("old_logp", old_logp),
                    ("tok_row", tok_row_), ("adv_row", adv_row), ("row_off", row_off)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (libgrpo has no CPU path)")
    _set_terms(a, row_weight, ref_logp, ent_coef, kl_coef, kl_type, ws)
    if tok_src is not None:
        if not tok_src.is_cuda or tok_src.dtype != torch.int64:
            raise ValueError("tok_src must be an int64 GPU tensor")
        a.tok_src = tok_src.data_ptr() if n else None
        a.n_src = n_src
    C.check(C.lib().grpo_loss_fwd_bwd(_stream(), ctypes.byref(a)))
    ws["dlogits"] = dl
    return ws


def transpose_bf16(x, out=None):
    """bf16 [rows x cols] -> its transpose [cols x rows] (grpo_transpose_bf16)."""
    torch = _torch()
    if x.dtype != torch.bfloat16:
        raise ValueError("transpose_bf16 takes a bf16 matrix")
    ld = _rows2d(x, "x")
    rows, cols = x.shape
    if out is None:
        out = torch.empty((cols, rows), dtype=torch.bfloat16, device=x.device)
    C.check(C.lib().grpo_transpose_bf16(_stream(), _dev(x, "x"), rows, cols, ld, _dev(out, "out"), _rows2d(out, "out")))
    return out


def lmhead_workspace_bytes(n_tok, H, V):
    return int(C.lib().grpo_lmhead_workspace_size(n_tok, H, V))


def lmhead_fwd_bwd(h, W, Wt, target, mask, old_logp, tok_row_, adv_row, row_off, dW, *, scale=1.0, denom=None,
                   eps_low=0.2, eps_high=0.2, dh=None, ws=None, workspace=None, row_weight=None,
                   ref_logp=None, ent_coef=0.0, kl_coef=0.0, kl_type=C.KL_K3):
    """Fused LM-head GRPO loss over one chunk (grpo_lmhead_fwd_bwd).

    ``dW`` (fp32 [V x H]) is accumulated into; ``dh`` (fp32 [n_tok x H]) is
    written.  Returns the per-token workspace dict with ``dh`` added."""
    torch = _torch()
    n, H = h.shape
    V = W.shape[0]
    n_rows = row_off.numel() - 1
    if ws is None:
        ws = loss_workspace(n, n_rows, h.device)
    if dh is None:
        dh = torch.empty((n, H), dtype=torch.float32, device=h.device)
    if workspace is None:
        workspace = torch.empty(max(lmhead_workspace_bytes(n, H, V), 1), dtype=torch.uint8, device=h.device)
    for name, t in (("h", h), ("W", W), ("Wt", Wt), ("target", target), ("mask", mask), ("old_logp", old_logp),
                    ("tok_row", tok_row_), ("adv_row", adv_row), ("row_off", row_off), ("dW", dW), ("dh", dh)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (libgrpo has no CPU path)")
    a = C.LmheadArgs()
    a.struct_size = ctypes.sizeof(C.LmheadArgs)
    a.h = h.data_ptr() if n else None
    a.ldh = _rows2d(h, "h")
    a.W, a.Wt = W.data_ptr(), Wt.data_ptr()
    a.n_tok, a.H, a.V = n, H, V
    a.target = target.data_ptr() if n else None
    a.mask = mask.data_ptr() if n else None
    a.old_logp = old_logp.data_ptr() if n else None
    a.tok_row = tok_row_.data_ptr() if n else None
    a.adv_row = adv_row.data_ptr() if n_rows else None
    a.row_off = row_off.data_ptr()
    a.n_rows = n_rows
    a.eps_low, a.eps_high, a.scale = eps_low, eps_high, scale
    a.denom = denom.data_ptr() if denom is not None else None
    a.dh = dh.data_ptr() if n else None
    a.dW = dW.data_ptr()
    for k in ("logp", "lse", "entropy", "loss_tok", "tok_flags", "row_stats", "chunk_stats"):
        t = ws[k]
        setattr(a, k, t.data_ptr() if t is not None else None)
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel()
    _set_terms(a, row_weight, ref_logp, ent_coef, kl_coef, kl_type, ws)
    C.check(C.lib().grpo_lmhead_fwd_bwd(_stream(), ctypes.byref(a)))
    ws["dh"] = dh
    ws["workspace"] = workspace
    return ws
