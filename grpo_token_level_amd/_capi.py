"""ctypes view of the C ABI declared in include/grpo.h (libgrpo.so).

Argument marshalling only: this module declares the entry points and the
plain-data structs, loads the in-tree library and turns status codes into
exceptions.  It never computes anything itself and has no fallback: without
the built library every call raises.
"""

import ctypes
import os

import numpy as np

# GRPO_LIB names another build of the same ABI (the host-only sanitizer build).
LIB_PATH = os.environ.get("GRPO_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgrpo.so")
HOST_ONLY = os.path.basename(LIB_PATH) == "libgrpo_host_san.so"

GRPO_F32 = 0
GRPO_BF16 = 1

CODES = {0: "OK", -1: "EINVAL", -2: "EDIVISIBLE", -3: "ETOOLONG", -4: "ECOUNT", -5: "ENONFINITE",
         -6: "ESKIPPED", -7: "ECAPACITY", -8: "EDEVICE", -9: "ESTATE"}


class GrpoError(RuntimeError):
    """A libgrpo call returned a negative status; ``kind`` is its name."""

    def __init__(self, code, msg):
        self.code = code
        self.kind = CODES.get(code, str(code))
        super().__init__(f"{self.kind}: {msg}")


KL_K1, KL_K2, KL_K3 = 1, 2, 3
LOSS_DEFER_STATS = 1
AGG_TOKEN_MEAN, AGG_SEQ_MEAN_TOKEN_SUM, AGG_SEQ_MEAN_TOKEN_MEAN = 0, 1, 2


class Stats(ctypes.Structure):
    _fields_ = [("loss_sum", ctypes.c_double), ("entropy_sum", ctypes.c_double),
                ("kl_sum", ctypes.c_double), ("obj_sum", ctypes.c_double),
                ("n_valid", ctypes.c_int64), ("n_clipped", ctypes.c_int64),
                ("n_nonfinite", ctypes.c_int64), ("n_valid_rows", ctypes.c_int64)]


# numpy view of an array of grpo_stats (64 bytes each)
STATS_DTYPE = np.dtype([("loss_sum", "<f8"), ("entropy_sum", "<f8"), ("kl_sum", "<f8"), ("obj_sum", "<f8"),
                        ("n_valid", "<i8"),
                        ("n_clipped", "<i8"), ("n_nonfinite", "<i8"), ("n_valid_rows", "<i8")])
STATS_BYTES = STATS_DTYPE.itemsize

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float


class LossArgs(ctypes.Structure):
    _fields_ = [("struct_size", _i32), ("in_dtype", _i32), ("out_dtype", _i32), ("reserved0", _i32),
                ("logits", _p), ("ld", _i64), ("n_tok", _i64), ("V", _i64),
                ("target", _p), ("mask", _p), ("old_logp", _p), ("tok_row", _p), ("adv_row", _p),
                ("row_off", _p), ("n_rows", _i64),
                ("eps_low", _f32), ("eps_high", _f32), ("scale", _f32), ("flags", _i32),
                ("denom", _p), ("dlogits", _p), ("ld_out", _i64),
                ("logp", _p), ("lse", _p), ("entropy", _p), ("loss_tok", _p), ("tok_flags", _p),
                ("row_stats", _p), ("chunk_stats", _p),
                ("row_weight", _p), ("ref_logp", _p), ("kl_tok", _p),
                ("ent_coef", _f32), ("kl_coef", _f32), ("kl_type", _i32), ("reserved2", _i32),
                ("tok_src", _p), ("n_src", _i64)]


class LmheadArgs(ctypes.Structure):
    _fields_ = [("struct_size", _i32), ("reserved0", _i32), ("h", _p), ("ldh", _i64), ("W", _p), ("Wt", _p),
                ("n_tok", _i64), ("H", _i64), ("V", _i64),
                ("target", _p), ("mask", _p), ("old_logp", _p), ("tok_row", _p), ("adv_row", _p),
                ("row_off", _p), ("n_rows", _i64),
                ("eps_low", _f32), ("eps_high", _f32), ("scale", _f32), ("flags", _i32),
                ("denom", _p), ("dh", _p), ("dW", _p),
                ("logp", _p), ("lse", _p), ("entropy", _p), ("loss_tok", _p), ("tok_flags", _p),
                ("row_stats", _p), ("chunk_stats", _p), ("workspace", _p), ("workspace_bytes", ctypes.c_size_t),
                ("row_weight", _p), ("ref_logp", _p), ("kl_tok", _p),
                ("ent_coef", _f32), ("kl_coef", _f32), ("kl_type", _i32), ("reserved2", _i32),
                ("dw_window", _p)]


class DwWindow(ctypes.Structure):
    _fields_ = [("buf", _p), ("bytes", ctypes.c_size_t), ("cap_tok", _i64), ("H", _i64), ("V", _i64),
                ("reserved", _i64)]


class TracePlan(ctypes.Structure):
    _fields_ = [("struct_size", _i32), ("dtype", _i32), ("stage", ctypes.c_char_p), ("n_rows", _i64), ("T", _i64),
                ("V", _i64), ("row_len", _p), ("row_valid", _p), ("row_uid", _p), ("row_traj", _p),
                ("row_seg", _p), ("row_is_pad", _p), ("n_calls", _i64), ("call_off", _p), ("call_rows", _p),
                ("call_step", _p)]


class StepResult(ctypes.Structure):
    _fields_ = [("loss", ctypes.c_double), ("entropy", ctypes.c_double), ("kl", ctypes.c_double),
                ("obj_sum", ctypes.c_double), ("grad_scale", ctypes.c_double),
                ("n_valid", _i64), ("n_valid_rows", _i64), ("n_clipped", _i64)]


class OldCache(ctypes.Structure):
    _fields_ = [("buf", _p), ("capacity", _i64), ("off", ctypes.POINTER(ctypes.c_int64)), ("n_calls", _i64),
                ("recorded", _i64), ("replayed", _i64)]


class ProbeStats(ctypes.Structure):
    _fields_ = [("n_valid", _i64), ("n_moved", _i64), ("max_abs", ctypes.c_double)]


class Probe(ctypes.Structure):
    _fields_ = [("bound", ctypes.c_double), ("max_fraction", ctypes.c_double), ("done", _i32), ("passed", _i32)]


LMHEAD_KEEP_Z = 1
LMHEAD_DEFER_DW = 2
LMHEAD_NOALLOC_SCRATCH_BYTES = 256 << 20

PROBE_STRICT_BOUND = 0.05
PROBE_STRICT_FRACTION = 0.0

_P64 = ctypes.POINTER(ctypes.c_int64)
_P32 = ctypes.POINTER(ctypes.c_int32)
_PU8 = ctypes.POINTER(ctypes.c_uint8)
_PF32 = ctypes.POINTER(ctypes.c_float)

# name -> (restype, argtypes)
PROTOTYPES = {
    "grpo_last_error": (ctypes.c_char_p, []),
    "grpo_version": (ctypes.c_char_p, []),
    "grpo_plan_fixed": (ctypes.c_int, [_i64, _i64, _i64, _i64, _P64, _P64, _P64, _P64]),
    "grpo_plan_chunk": (ctypes.c_int, [_i64, _i64, _i64, _i64, _i64, _P64, _P64]),
    "grpo_plan_dynamic": (ctypes.c_int, [_P64, _i64, _i64, _i64, _i64, _P64, _P64, _P64, _P64]),
    "grpo_plan_epochs": (ctypes.c_int, [_i64, _i64, _i64, _i64, _i64, _i32, ctypes.c_uint64, _P64, _P64, _P64, _P64,
                                        _P64]),
    "grpo_plan_compaction": (ctypes.c_int, [_P32, _i64, _i64, _i64, _i64, _i64, _i32, _i64, _P64,
                                            _P32, _P32, _P32, _PU8, _P32]),
    "grpo_row_offsets": (ctypes.c_int, [_P64, _P64, _i64, _P64]),
    "grpo_plan_trace": (ctypes.c_int, [ctypes.POINTER(TracePlan), ctypes.c_char_p, ctypes.c_size_t,
                                       ctypes.POINTER(ctypes.c_size_t)]),
    "grpo_group_advantage": (ctypes.c_int, [_PF32, _i64, _i64, _f32, _i32, _PF32]),
    "grpo_rows_advantage": (ctypes.c_int, [_PF32, _i64, _P32, _i64, _PF32]),
    "grpo_count_valid": (ctypes.c_int, [_p, _p, _i64, _p]),
    "grpo_count_rows": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _p]),
    "grpo_row_weights": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i32, _p, _p]),
    "grpo_tok_row": (ctypes.c_int, [_p, _p, _i64, _i64, _p]),
    "grpo_chunk_tok_src": (ctypes.c_int, [_p, _p, _i64, _p, _i64, _p, _i64, _p]),
    "grpo_gather": (ctypes.c_int, [_p, _p, _i64, _p, _i64, _i64, _p]),
    "grpo_logprob_fwd": (ctypes.c_int, [_p, _i32, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    "grpo_logprob_fwd_paired": (ctypes.c_int, [_p, _i32, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    "grpo_loss_fwd_bwd": (ctypes.c_int, [_p, ctypes.POINTER(LossArgs)]),
    "grpo_loss_stats": (ctypes.c_int, [_p, ctypes.POINTER(LossArgs)]),
    "grpo_stats_sum": (ctypes.c_int, [_p, _i64, ctypes.POINTER(Stats)]),
    "grpo_transpose_bf16": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _p, _i64]),
    "grpo_lmhead_workspace_size": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "grpo_lmhead_workspace_size_flags": (ctypes.c_size_t, [_i64, _i64, _i64, _i32]),
    "grpo_lmhead_fwd_bwd": (ctypes.c_int, [_p, ctypes.POINTER(LmheadArgs)]),
    "grpo_lmhead_fwd_bwd_noalloc": (ctypes.c_int, [_p, ctypes.POINTER(LmheadArgs)]),
    "grpo_lmhead_dw_window_size": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "grpo_lmhead_dw_window_init": (ctypes.c_int, [_p, ctypes.POINTER(DwWindow), _p, ctypes.c_size_t, _i64, _i64,
                                                  _i64]),
    "grpo_lmhead_dw_flush": (ctypes.c_int, [_p, ctypes.POINTER(DwWindow), _p]),
    "grpo_needs_ahead_pass": (ctypes.c_int32, [_i64, _i32, _i32]),
    "grpo_old_cache_init": (ctypes.c_int, [ctypes.POINTER(OldCache), _p, _i64, _P64, _i64]),
    "grpo_old_cache_reset": (ctypes.c_int, [ctypes.POINTER(OldCache)]),
    "grpo_old_cache_rewind": (ctypes.c_int, [ctypes.POINTER(OldCache)]),
    "grpo_old_cache_record": (ctypes.c_int, [_p, ctypes.POINTER(OldCache), _i32, _p, _i64, _i64, _i64, _p, _p,
                                             ctypes.POINTER(ctypes.c_void_p)]),
    "grpo_old_cache_record_paired": (ctypes.c_int, [_p, ctypes.POINTER(OldCache), _i32, _p, _i64, _i64, _i64, _p, _p,
                                             ctypes.POINTER(ctypes.c_void_p)]),
    "grpo_old_cache_replay": (ctypes.c_int, [ctypes.POINTER(OldCache), _i64, ctypes.POINTER(ctypes.c_void_p)]),
    "grpo_probe_compare": (ctypes.c_int, [_p, _p, _p, _p, _i64, _f32, _p]),
    "grpo_probe_init": (ctypes.c_int, [ctypes.POINTER(Probe), ctypes.c_double, ctypes.c_double]),
    "grpo_probe_finish": (ctypes.c_int, [ctypes.POINTER(Probe), ctypes.POINTER(ProbeStats),
                                         ctypes.POINTER(ctypes.c_int32)]),
    "grpo_accum_size": (ctypes.c_size_t, []),
    "grpo_accum_init": (ctypes.c_int, [_p, _i64]),
    "grpo_accum_add": (ctypes.c_int, [_p, ctypes.POINTER(Stats)]),
    "grpo_accum_finalize": (ctypes.c_int, [_p, ctypes.POINTER(StepResult),
                                           ctypes.POINTER(ctypes.c_int32)]),
}

_lib = None


def lib():
    """The loaded libgrpo.so; raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m grpo_token_level_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            if HOST_ONLY and not hasattr(L, name):
                continue
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(code):
    """Raise GrpoError for a negative status."""
    if code != 0:
        msg = lib().grpo_last_error().decode(errors="replace")
        raise GrpoError(code, msg)
    return code


def ptr64(a):
    return a.ctypes.data_as(_P64)


def ptr32(a):
    return a.ctypes.data_as(_P32)


def ptru8(a):
    return a.ctypes.data_as(_PU8)


def ptrf32(a):
    return a.ctypes.data_as(_PF32)
