"""The host code of the library under AddressSanitizer and
UndefinedBehaviorSanitizer: the reference quantizer and packers
(test_quant_cpp.py) and the argument checks of every entry point
(test_abi_cpu.py) run against the sanitized build
(`python -m block_quantized_decode_qgemv_amd.build --sanitize`) in a child
process with clang's sanitizer runtime preloaded.  Any heap or stack
overflow, use after free or undefined behaviour aborts the child.  Skipped
when that build is absent or older than the sources (it takes minutes, so
the CPU suite does not make it)."""
import os
import subprocess
import sys

import pytest

from block_quantized_decode_qgemv_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sanitized_build_current() -> bool:
    if not os.path.exists(B.SAN_LIB):
        return False
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)] + [os.path.join(B.INCLUDE, "qgemv.h")]
    return os.path.getmtime(B.SAN_LIB) >= max(os.path.getmtime(p) for p in srcs)


@pytest.mark.skipif(not _sanitized_build_current(),
                    reason="sanitized build absent or older than the sources (build.py --sanitize)")
def test_host_code_under_asan_ubsan():
    if os.environ.get("QG_TEST_LIB"):
        pytest.skip("already running against another library build")
    env = dict(os.environ, QG_TEST_LIB=B.SAN_LIB, LD_PRELOAD=B.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_quant_cpp.py", "tests/test_abi_cpu.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
