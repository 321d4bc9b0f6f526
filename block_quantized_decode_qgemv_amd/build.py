"""Build libqgemv.so in-tree for gfx950.

    python -m block_quantized_decode_qgemv_amd.build [--incremental]
    python -m block_quantized_decode_qgemv_amd.build --sanitize

--sanitize builds a second library, _build/sanitize/libqgemv.so, whose host
code (the reference quantizer and packers, and the argument checks of every
entry point) carries AddressSanitizer and UndefinedBehaviorSanitizer; the
device code is unchanged.  All host code goes through ROCm's clang, so one
sanitizer runtime (clang's, SANITIZER_RUNTIME) serves the whole library; a
process that loads it must preload that runtime (the CPU test
tests/test_sanitize_cpu.py does).

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
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_DIR = os.path.join(BUILD_DIR, "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libqgemv.so")
SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
             "-g"]
ARCH = "gfx950"

DEVICE_SOURCES = ["gemv.hip", "gemv_splitk.hip", "gemv_norm.hip", "gemv_norm_unit.hip", "moe.hip", "quant.hip", "probe.hip"]
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


def sanitizer_runtime() -> str:
    """clang's AddressSanitizer runtime (it carries the UBSan handlers too)."""
    out = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True,
                         check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        libdir = subprocess.run([CLANGXX, "-print-resource-dir"], capture_output=True, text=True,
                                check=True).stdout.strip()
        out = os.path.join(libdir, "lib", "linux", "libclang_rt.asan-x86_64.so")
    return out


def build_sanitized(verbose: bool = True) -> str:
    """The library with sanitized host code (see the module docstring)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    host_san = [f for flag in SAN_FLAGS for f in ("-Xarch_host", flag)]
    jobs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(SAN_DIR, src + ".o")
        jobs.append(([HIPCC, *HIP_FLAGS, *host_san, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    host_flags = [f for f in HOST_FLAGS if f != "-O2"] + ["-O1", "-D__HIP_PLATFORM_AMD__"]
    for src in HOST_SOURCES:
        obj = os.path.join(SAN_DIR, src + ".o")
        jobs.append(([CLANGXX, *host_flags, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd, _ in jobs]:
            f.result()
    tmp = SAN_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *host_san, "-Xarch_host", "-shared-libsan",
          *[o for _, o in jobs], "-o", tmp, "-lpthread"], verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        build_sanitized(verbose="-q" not in sys.argv)
    else:
        build(verbose="-q" not in sys.argv, incremental="--incremental" in sys.argv)
