"""The host side of the C ABI (step preparation, prefill work plan, scheduler,
graph argument checks) built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, no GPU) and driven with valid and malformed inputs by
tests/asan/host_driver.cpp."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_28_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_host_abi_under_address_and_ub_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "host_driver")
    cmd = [_hipcc(), "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "asan", "host_driver.cpp"), os.path.join(CSRC, "api.cpp"),
           os.path.join(CSRC, "sched.cpp"), os.path.join(CSRC, "graph.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failed checks" in r.stdout
