"""The library's host reference quantizer (C++) against the oracle (numpy):
packed bytes must be identical.  Two independent implementations of the same
definitions; no GPU needed."""
import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
import workloads
from oracle import formats as OF

QUANT = ("q8_0", "q4_0", "q4_1", "q4_k", "q2_k")


@pytest.mark.parametrize("fmt", QUANT)
@pytest.mark.parametrize("shape", [(1, 256), (7, 512), (64, 4096), (3, 14336)])
def test_student_t_bytes_identical(fmt, shape):
    w = workloads.student_t_weights(*shape, seed=11, tensor_id=hash(fmt) % 1000)
    np.testing.assert_array_equal(qg.qquant(fmt, w, n_threads=4), OF.quantize_packed(fmt, w))


@pytest.mark.parametrize("fmt", QUANT)
def test_edge_blocks_identical(fmt):
    g = np.random.default_rng(5)
    w = (g.standard_normal((12, 512)) * 0.02).astype(np.float32)
    w[0] = 0.0                                   # all-zero row
    w[1, :256] = -0.0                            # signed zeros
    w[2, :] = 0.37                               # constant positive
    w[3, :] = -0.37                              # constant negative
    w[4, :32] = 1e-8                             # scales in the fp16 subnormal range
    w[5] = np.abs(w[5])                          # all positive
    w[6] = -np.abs(w[6])                         # all negative
    w[7, 5] = w[7, 9] = np.abs(w[7]).max() * 2   # tie on the max-|.| element
    w[8, 5], w[8, 9] = 0.5, -0.5                 # opposite-signed tie
    w[9, :] = np.float32(2.0 ** -24)             # tiny values
    w[10] = np.round(w[10] * 1000) / 1000        # many exact ties in rounding
    w[11] = g.standard_t(2, 512).astype(np.float32)  # heavy tails
    np.testing.assert_array_equal(qg.qquant(fmt, w, n_threads=3), OF.quantize_packed(fmt, w))


@pytest.mark.parametrize("fmt", QUANT)
def test_threads_do_not_change_bytes(fmt):
    w = workloads.student_t_weights(37, 1024, seed=3)
    a = qg.qquant(fmt, w, n_threads=1)
    b = qg.qquant(fmt, w, n_threads=8)
    np.testing.assert_array_equal(a, b)


def test_tern_bin_packers_identical():
    codes = workloads.ternary_codes(9, 384, seed=2)
    bits = workloads.binary_codes(9, 384, seed=2)
    sc = workloads.scale_bits_f16((9, 3), seed=2)
    np.testing.assert_array_equal(qg.qpack_tern(codes, sc), OF.pack("tern", OF.tern_from_codes(codes, sc)))
    np.testing.assert_array_equal(qg.qpack_bin(bits, sc), OF.pack("bin", OF.bin_from_codes(bits, sc)))


@pytest.mark.parametrize("n,k", [(9, 384), (17, 128), (40, 2048), (3, 128 * 300)])
def test_bin8_packer_identical(n, k):
    """The C++ bin8 packer (per-row affine re-coding of the fp16 scales)
    against the oracle's, byte for byte: ragged groups, meta rows with and
    without a short unit, a one-block row (step 0) and long rows."""
    bits = workloads.binary_codes(n, k, seed=k)
    sc = workloads.scale_bits_f16((n, k // 128), seed=k, tensor_id=1)
    sc[0] = sc[0, 0]  # a row of equal scales
    np.testing.assert_array_equal(qg.qpack_bin8(bits, sc), OF.pack("bin8", OF.bin8_from_codes(bits, sc)))


@pytest.mark.parametrize("n,k", [(9, 256), (17, 768), (40, 4096), (3, 256 * 70)])
def test_tern3_packer_identical(n, k):
    """The C++ tern3 packer (base-3 bytes, 2-bit tail fields, per-64 scales)
    against the oracle's, byte for byte: ragged groups, code and meta rows
    with and without a short unit, rows of all -1 and all +1."""
    codes = workloads.ternary_codes(n, k, seed=k, tensor_id=3)
    codes[0] = 1
    codes[-1] = -1
    sc = workloads.scale_bits_f16((n, k // 64), seed=k, tensor_id=4)
    np.testing.assert_array_equal(qg.qpack_tern3(codes, sc), OF.pack("tern3", OF.tern3_from_codes(codes, sc)))


def test_tern3_packer_errors():
    with pytest.raises(qg.QGError) as e:
        qg.qpack_tern3(np.full((1, 256), -2, np.int8), np.zeros((1, 4), np.uint16))
    assert e.value.code == -1 and "(0, 0)" in e.value.detail
    with pytest.raises(qg.QGError) as e:
        qg.qquant("tern3", np.zeros((1, 256), np.float32))
    assert e.value.code == -1
    with pytest.raises(ValueError):
        qg.qpack_tern3(np.zeros((1, 128), np.int8), np.zeros((1, 2), np.uint16))   # K not a multiple of 256
    with pytest.raises(ValueError):
        qg.qpack_tern3(np.zeros((1, 256), np.int8), np.zeros((1, 2), np.uint16))   # scales per 128, not 64


def test_quantizer_errors():
    w = np.ones((2, 256), np.float32)
    w[1, 3] = np.inf
    with pytest.raises(qg.QGError) as e:
        qg.qquant("q4_k", w)
    assert e.value.code == -1 and "row 1" in e.value.detail
    with pytest.raises(qg.QGError) as e:
        qg.qquant("q8_0", np.full((1, 32), 2e7, np.float32))
    assert e.value.code == -4
    with pytest.raises(qg.QGError) as e:
        qg.qquant("tern", np.zeros((1, 128), np.float32))
    assert e.value.code == -1
    with pytest.raises(qg.QGError) as e:
        qg.qquant("q4_0", np.zeros((1, 48), np.float32))
    assert e.value.code == -2
    with pytest.raises(qg.QGError) as e:
        qg.qpack_tern(np.full((1, 128), 2, np.int8), np.zeros((1, 1), np.uint16))
    assert e.value.code == -1
    with pytest.raises(qg.QGError) as e:
        qg.qpack_bin(np.full((1, 128), 3, np.uint8), np.zeros((1, 1), np.uint16))
    assert e.value.code == -1
    with pytest.raises(qg.QGError) as e:
        qg.qpack_bin8(np.zeros((1, 256), np.uint8), np.array([[0x3C00, 0x7E00]], np.uint16))  # NaN scale
    assert e.value.code == -1
    with pytest.raises(qg.QGError) as e:
        qg.qquant("bin8", np.zeros((1, 128), np.float32))
    assert e.value.code == -1
