"""Builds libpkv.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: ``python -m paged_kv_attention_28_amd.build`` or ``build()`` from
Python. Always recompiles. Sources are compiled in parallel to objects
under ``_build/`` and linked into ``paged_kv_attention_28_amd/libpkv.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")
SOURCES = ["api.cpp", "sched.cpp", "graph.cpp", "kv_store.hip", "rope_store.hip", "sampler.hip", "decode.hip", "prefill.hip"]
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv.so)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            # packed fp32 instructions are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]


def _compile(src: str, obj: str, extra) -> str:
    cmd = [_hipcc(), *_flags(), *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in (p.stderr or "").splitlines() if noise not in l).strip()
    return warn


def build(verbose: bool = True, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        futs = {}
        for s in SOURCES:
            obj = os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            futs[ex.submit(_compile, os.path.join(CSRC, s), obj, list(extra))] = s
        for f in cf.as_completed(futs):
            w = f.result()
            if w and verbose:
                print(f"[pkv build] {futs[f]}:\n{w}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"[pkv build] wrote {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
