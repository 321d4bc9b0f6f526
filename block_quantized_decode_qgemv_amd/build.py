"""Build libqgemv.so in-tree for gfx950.

    python -m block_quantized_decode_qgemv_amd.build

Device code: hipcc --offload-arch=gfx950 -O3, with packed fp32 instructions
disabled.  Host reference quantizer: g++ -O2 -ffp-contract=off (IEEE fp32 in
the order written, no contraction).  The library lands next to this file.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqgemv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_SOURCES = ["gemv.hip", "gemv_norm.hip", "gemv_norm_unit.hip", "moe.hip", "quant.hip", "probe.hip"]
HOST_SOURCES = ["host.cpp"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off", "-fno-fast-math",
              "-I", INCLUDE, "-I", CSRC, "-I", "/opt/rocm/include"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _includes(path, seen=None) -> set:
    """The library headers `path` includes, directly or through other headers."""
    seen = set() if seen is None else seen
    with open(path, encoding="utf-8") as fh:
        for line in fh:
            m = re.match(r'\s*#include\s+"([^"]+)"', line)
            if not m:
                continue
            for base in (CSRC, INCLUDE):
                dep = os.path.join(base, m.group(1))
                if os.path.exists(dep) and dep not in seen:
                    seen.add(dep)
                    _includes(dep, seen)
                    break
    return seen


def _stale(obj, src) -> bool:
    """Whether obj is older than src or a header it includes."""
    if not os.path.exists(obj):
        return True
    return os.path.getmtime(obj) < max(os.path.getmtime(p) for p in [src, *_includes(src)])


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compile every source (or, incremental, only those whose object is older
    than the source or a header) and link libqgemv.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []  # (command, object); the sources compile concurrently
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append(([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    todo = [(cmd, obj) for cmd, obj in jobs if not incremental or _stale(obj, cmd[-3])]
    with ThreadPoolExecutor(max_workers=max(1, min(len(todo), 8))) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd, _ in todo]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o in jobs], "-o", tmp, "-lpthread"],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv, incremental="--incremental" in sys.argv)
