import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# QG_TEST_LIB: run the tests against another build of the library (the
# sanitized host build of tests/test_sanitize_cpu.py); unset, the in-tree one.
if os.environ.get("QG_TEST_LIB"):
    import block_quantized_decode_qgemv_amd as _qg

    _qg.lib_path = lambda: os.environ["QG_TEST_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Rows of a golden fixture, comments (#) and blank lines dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture
def golden():
    return read_golden
