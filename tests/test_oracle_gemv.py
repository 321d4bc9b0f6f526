"""Oracle pins for the GEMV reference and the decode bound (CPU only)."""
import math

import numpy as np
import pytest

import workloads
from oracle import decode_bound as DB
from oracle import formats as F
from oracle import gemv as G


@pytest.mark.parametrize("fmt", F.FORMATS)
@pytest.mark.parametrize("n", [1, 2, 3, 5])
def test_bruteforce_tiny(fmt, n):
    """float64 reference == math.fsum brute force on tiny shapes."""
    k = F.SPECS[fmt].block * 2
    if fmt == "tern":
        blk = F.tern_from_codes(workloads.ternary_codes(n, k, 1), workloads.scale_bits_f16((n, k // 128), 1))
    elif fmt == "bin":
        blk = F.bin_from_codes(workloads.binary_codes(n, k, 1), workloads.scale_bits_f16((n, k // 128), 1))
    elif fmt == "bin8":
        blk = F.bin8_from_codes(workloads.binary_codes(n, k, 1), workloads.scale_bits_f16((n, k // 128), 1))
    elif fmt == "tern3":
        blk = F.tern3_from_codes(workloads.ternary_codes(n, k, 1), workloads.scale_bits_f16((n, k // 64), 1))
    else:
        blk = F.quantize(fmt, workloads.student_t_weights(n, k, 1))
    w = F.dequant(fmt, blk)
    x = workloads.normal((2, k), 1, 7)
    ref = G.gemv_ref(w, x)
    bf = G.gemv_fsum(w, x)
    np.testing.assert_allclose(ref, bf, rtol=1e-13, atol=1e-15)
    ok, ratio, _ = G.check(bf.astype(np.float32), w, x)
    assert ok and ratio < 0.1


def test_every_code_value_enumerated():
    """Q4_K rows whose codes run through all 16 values; brute force with fsum."""
    n, k = 16, 256
    codes = (np.arange(n * k) % 16).reshape(n, k).astype(np.uint8)
    blk = {"d": np.full((n, 1), 0x2000, np.uint16), "dmin": np.full((n, 1), 0x1C00, np.uint16),
           "s": np.tile(np.arange(1, 9, dtype=np.uint8), (n, 1, 1)),
           "t": np.tile(np.arange(0, 16, 2, dtype=np.uint8), (n, 1, 1)), "n": codes}
    w = F.dequant("q4_k", blk)
    x = workloads.normal((1, k), 3)
    np.testing.assert_allclose(G.gemv_ref(w, x), G.gemv_fsum(w, x), rtol=1e-13)


def test_integer_exact():
    """Power-of-two scales and small-integer activations make every product and
    partial sum exact in fp32, so any summation order gives the same value,
    which equals an integer matvec."""
    g = np.random.default_rng(0)
    n, k = 7, 512
    nib = g.integers(0, 16, size=(n, k)).astype(np.uint8)
    blk = {"d": np.full((n, k // 32), 0x3C00, np.uint16), "n": nib}  # d = 1.0
    w = F.dequant("q4_0", blk)
    x = g.integers(-3, 4, size=(1, k)).astype(np.float32)
    exact = (nib.astype(np.int64) - 8) @ x[0].astype(np.int64)
    np.testing.assert_array_equal(G.gemv_ref(w, x)[0], exact.astype(np.float64))
    # fp32 sequential accumulation gives the same integers
    acc = np.zeros(n, np.float32)
    for j in range(k):
        acc = acc + w[:, j] * x[0, j]
    np.testing.assert_array_equal(acc.astype(np.float64), exact)


def test_tolerance_rejects_gross_errors():
    w = F.dequant("q8_0", F.quantize("q8_0", workloads.student_t_weights(8, 64, 2)))
    x = workloads.normal((1, 64), 2)
    y = G.gemv_ref(w, x)
    assert G.check(y, w, x)[0]
    y_bad = y.copy()
    y_bad[0, 3] += 1e-3 * np.abs(y).max() + 1e-4
    assert not G.check(y_bad, w, x)[0]
    # an off-by-one column index is a plausible mistake the check must catch
    shifted = (np.roll(w, 1, axis=1).astype(np.float64) @ x[0].astype(np.float64))[None]
    assert not G.check(shifted, w, x)[0]


def test_decode_bound_table(golden):
    for bw, tok in golden("handbook_decode_bound.txt"):
        assert round(DB.tokens_per_s(float(bw), 4.5e9)) == int(tok)


def test_decode_bound_exercise(golden):
    vals = {k: float(v) for k, v in golden("handbook_exercise.txt")}
    assert DB.max_weight_bytes(60e9, 20) == pytest.approx(vals["max_bytes_at_20_tok_s"], rel=1e-12)
    assert DB.model_bytes(3e9, 4.5) == pytest.approx(vals["bytes_at_4.5_bits"], rel=0.01)
    # 8 bits in the page's answer is the 8.5-bit Q8_0 block format
    b8 = DB.model_bytes(3e9, F.SPECS["q8_0"].bpw)
    assert b8 == pytest.approx(vals["bytes_at_8_bits"], rel=0.01)
    assert round(DB.tokens_per_s(60e9, b8)) == int(vals["tok_s_at_8_bits"])
    assert DB.model_bytes(3e9, 4.5) <= DB.max_weight_bytes(60e9, 20)
    assert not math.isnan(DB.tokens_per_s(1, 1))
