"""The host half of libgrpo under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libgrpo_host_san.so (host sources only, g++ -fsanitize=address,undefined,
every report fatal) and runs the host-ABI and trace tests against it in a
child process with the ASan runtime preloaded.  Those tests drive the plans,
the dynamic packer, the compaction plan, the epochs shuffle, the advantages,
the accumulator's poisoned-window countdown ([P1] "The poisoned-window
countdown"), the pi_old cache state machine and the trace dump with random
and edge-case inputs; any out-of-bounds access or undefined behaviour aborts
the child and fails this test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_half_is_clean_under_asan_and_ubsan():
    from grpo_token_level_amd import build
    try:
        build.build_sanitized()
    except RuntimeError as e:   # pragma: no cover - toolchain without the sanitizer runtimes
        pytest.skip(f"sanitizer build unavailable: {e}")
    env = build.sanitizer_env()
    probe = ("import ctypes; from grpo_token_level_amd import _capi as C; C.lib(); "
             "assert C.HOST_ONLY and hasattr(ctypes.CDLL(None), '__asan_report_load8'); print('asan on')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0 and "asan on" in r.stdout, r.stdout[-2000:]
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_host_abi.py"), os.path.join(ROOT, "tests", "test_plan_trace.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600)
    tail = "\n".join(r.stdout.splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error:" not in r.stdout, tail
    assert " passed" in tail, tail
