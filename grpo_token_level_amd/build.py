"""Builds libgrpo.so (host C++ + gfx950 HIP kernels) in-tree.

    python -m grpo_token_level_amd.build [-v] [--sanitize]

``--sanitize`` builds instead ``libgrpo_host_san.so``: the host half only
(plans, advantages, accumulator, pi_old cache bookkeeping, probe verdict,
trace dump) under AddressSanitizer and UndefinedBehaviorSanitizer, with the
one device call the host half makes stubbed out.  Load it with the ASan
runtime preloaded (``sanitizer_env``).

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so that it travels with the source tree.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgrpo.so")
SAN_LIB = os.path.join(PKG, "libgrpo_host_san.so")
SAN_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

ARCH = "gfx950"
# Packed-fp32 VALU forms are kept out of the generated code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libgrpo)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".cpp", ".hip")))


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        objs.append(obj)
        if src.endswith(".hip"):
            cmd = [hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        else:
            cmd = ["g++", *CXX_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        jobs.append(cmd)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(verbose=False):
    """The host-only library under ASan + UBSan (g++; no GPU code in it)."""
    srcs = [s for s in sources() if s.endswith(".cpp")] + [os.path.join(CSRC, "sanitize", "device_stub.cpp")]
    tmp = SAN_LIB + ".tmp"
    _run(["g++", *SAN_FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp], verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def sanitizer_env(base=None):
    """Environment for a process that loads libgrpo_host_san.so: the ASan
    runtime preloaded (ahead of anything already preloaded), leak checks off
    (the interpreter keeps objects alive at exit), every report fatal."""
    env = dict(os.environ if base is None else base)
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["GRPO_LIB"] = SAN_LIB
    return env


if __name__ == "__main__":
    args = sys.argv[1:]
    print(build_sanitized(verbose="-v" in args) if "--sanitize" in args else build(verbose="-v" in args))
