"""Measurement infrastructure beside the product, not part of it.

* ``stream_kernels.hip`` -> ``libyardstick.so``: a plain streaming copy, read
  and zero fill of one buffer.  The benchmark times them next to the loss
  kernels so that those can be read against what the memory system delivers
  for the same bytes, and the copy calibrates the HBM byte counters.
* ``prof_summary``: turns rocprofv3 CSV output into the short summaries kept
  under ``profiles/``.

Only ``bench.py`` and ``tests/test_gpu_stream.py`` use this package; the
library ``libgrpo`` neither links nor calls it.
"""

import ctypes
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libyardstick.so")
COPY, READ, FILL = 0, 1, 2

_lib = None


def build(verbose=False):
    """Compile libyardstick.so for gfx950 (same flags as libgrpo)."""
    hipcc = next(c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc"))
                 if c and os.path.exists(c))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-Wall", os.path.join(HERE, "stream_kernels.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"yardstick build failed:\n{r.stdout}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import yardstick; yardstick.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        L.ys_stream.restype = ctypes.c_int
        L.ys_stream.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        L.ys_last_error.restype = ctypes.c_char_p
        L.ys_last_error.argtypes = []
        _lib = L
    return _lib


def stream(mode, src=None, dst=None, nbytes=None):
    """A plain copy (COPY, src -> dst), read (READ, src; dst is 16 bytes of
    scratch) or zero fill (FILL, dst) of ``nbytes`` bytes (default: the whole
    src, or dst for a fill), on torch's current stream.  Returns dst."""
    import torch
    if mode not in (COPY, READ, FILL):
        raise ValueError(f"unknown stream mode {mode}")
    if mode == READ and dst is None:
        dst = torch.empty(16, dtype=torch.uint8, device=src.device)
    size = lambda t: t.numel() * t.element_size()  # noqa: E731
    if nbytes is None:
        nbytes = size(dst if mode == FILL else src)
    for t, name, need in ((src, "src", nbytes if mode != FILL else 0),
                          (dst, "dst", 16 if mode == READ else nbytes)):
        if need and (t is None or not t.is_cuda or not t.is_contiguous() or size(t) < need):
            raise ValueError(f"{name} must be a contiguous GPU tensor of at least {need} bytes")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib().ys_stream(st, mode, ctypes.c_void_p(src.data_ptr()) if src is not None else None,
                         ctypes.c_void_p(dst.data_ptr()), nbytes)
    if rc != 0:
        raise RuntimeError(f"ys_stream: {lib().ys_last_error().decode(errors='replace')}")
    return dst
