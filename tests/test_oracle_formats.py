"""Oracle pins for the block formats (CPU only).

What pins what:
* the handbook listing's printed error table pins the quantizer semantics
  (signed Q4_0 scale, Q4_1 min, Q4_K min clamp and 6-bit code ranges);
* the listing's bits/weight closed forms pin the plane sizes;
* hand-built blocks that must survive dequant -> quantize unchanged pin the
  quantizer/dequantizer pair and the byte layout;
* hand-computed bytes pin the byte order (reading R4).
"""
import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import page_sample
from tests import oracle_pins as P

F32 = np.float32

PAGE_NAMES = P.PAGE_NAMES


@pytest.fixture(scope="module")
def page_w():
    return page_sample.page_weights()


@pytest.fixture(scope="module")
def printed():
    from tests.conftest import read_golden

    return {r[0]: float(r[2]) for r in read_golden("handbook_error_table.txt")}


def test_page_sample_matches_listing_shape(page_w):
    assert page_w.shape == (4096 * 256,) and page_w.dtype == np.float32


def test_error_table_page_literal(page_w, printed):
    """The quantizers in page-literal mode (fp32 scales, as the listing keeps
    them) reproduce the printed table to 4 decimals."""
    P.error_table_literal(F, page_w, printed)


def test_error_table_fp16_storage(page_w, printed):
    """Production quantizers (fp16-stored scales) stay within 0.002 of the
    printed errors and keep the printed ordering Q8_0 << Q4_1 ~ Q4_K < Q4_0."""
    P.error_table_fp16(F, page_w, printed)


def test_page_literal_blocks_do_not_pack():
    blk = F.quantize("q8_0", np.ones((1, 32), F32), literal=True)
    assert blk["d"].dtype == F32 and blk["d"][0, 0] == F32(1) / F32(127)
    with pytest.raises(TypeError):
        F.pack("q8_0", blk)


def test_bpw_closed_forms(golden):
    """Plane sizes equal the printed bits/weight (and N*K*bpw/8 bytes): code
    bits plus the block's meta bits spread over its weights -- one fp16 per 32
    (Q8_0, Q4_0), two per 32 (Q4_1), and per 256 eight 6+6-bit code pairs
    plus two fp16 (Q4_K)."""
    printed = {r[0]: float(r[1]) for r in golden("handbook_error_table.txt")}
    kquant_meta = (8 * 12 + 2 * 16) / 256
    closed = {"Q8_0": 8 + 16 / 32, "Q4_0": 4 + 16 / 32, "Q4_1": 4 + 2 * 16 / 32, "Q4_K": 4 + kquant_meta}
    for name, fmt in PAGE_NAMES.items():
        assert F.SPECS[fmt].bpw == closed[name] == printed[name]
    # low-bit formats: 2-bit codes + the K-quant meta; 2-bit fields / bits + fp16 per 128
    assert F.SPECS["q2_k"].bpw == 2 + kquant_meta == 2.5
    assert F.SPECS["tern"].bpw == 2 + 16 / 128 == 2.125
    assert F.SPECS["bin"].bpw == 1 + 16 / 128 == 1.125
    for fmt, spec in F.SPECS.items():
        for n, k in ((1, 256), (7, 512), (4096, 4096), (14336, 4096)):
            pad = -(n * k // spec.block * spec.meta_bytes) % 16 if fmt in F.ROW_BYTES else 0
            assert F.packed_size(fmt, n, k) * 8 == n * k * spec.bpw + 8 * (n * F.ROW_BYTES.get(fmt, 0) + pad)
            assert F.codes_plane_size(fmt, n, k) % 16 == 0


def test_expert_sizes(golden):
    for name, fmt, rows, cols, mats, printed in golden("expert_sizes.txt"):
        assert mats_size(fmt, int(rows), int(cols), int(mats)) == int(printed), name
    assert mats_size("q4_k", 1024, 4096, 3) / 2**20 == 6.75


def mats_size(fmt, rows, cols, mats):
    # gate/up [rows x cols] and down [cols x rows] have the same element count
    return mats * F.packed_size(fmt, rows, cols)


# ----------------------------------------------------------------------------
# hand-built blocks (tests/oracle_pins.py)


@pytest.mark.parametrize("fmt,qmax", [("q4_k", 15), ("q2_k", 3)])
def test_roundtrip_kquant(fmt, qmax):
    P.roundtrip_kquant(F, fmt, qmax)


def test_roundtrip_q8_0():
    P.roundtrip_q8_0(F)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_roundtrip_q4_0(sign):
    P.roundtrip_q4_0(F, sign)


def test_roundtrip_q4_1():
    P.roundtrip_q4_1(F)


def test_roundtrip_tern_bin():
    P.roundtrip_tern_bin(F)


def test_roundtrip_tern3():
    P.roundtrip_tern3(F)


def test_tern3_hand_worked_bytes():
    P.tern3_bytes(F)


def test_q2k_hand_worked_bytes_and_values():
    P.q2k_bytes_and_values(F)


def test_tern3_density_matches_page(golden):
    """tern3 (R10): 48 bytes of base-3 digits (five weights per byte) and 12
    meta bytes (four fp16 scales, 16 weights in 2-bit fields) per 256 weights
    give the density the page prints, with its scale group of 64."""
    printed = {r[0]: float(r[1]) for r in golden("lowbit_ternary_density.txt")}
    spec = F.SPECS["tern3"]
    assert spec.bpw == (240 * 8 / 5 + 16 * 2 + 4 * 16) / 256 == printed["bits_per_weight"]
    assert spec.block // 4 == printed["scale_group"]
    assert 5 * np.log2(3) <= 8 and 3 ** 5 <= 256  # five base-3 digits fit a byte
    assert F.packed_size("tern3", 3, 4096) * 8 == 3 * 4096 * 1.875


def test_tern3_rejects():
    with pytest.raises(ValueError):
        F.tern3_from_codes(np.zeros((1, 128), np.int8), np.zeros((1, 2), np.uint16))
    with pytest.raises(F.QuantInputError):
        F.tern3_from_codes(np.full((1, 256), 2, np.int8), np.zeros((1, 4), np.uint16))
    buf = F.pack("tern3", F.tern3_from_codes(np.zeros((1, 256), np.int8), np.zeros((1, 4), np.uint16)))
    bad = buf.copy()
    bad[5] = 243  # not a five-digit base-3 number
    with pytest.raises(ValueError):
        F.unpack("tern3", bad, 1, 256)
    bad = buf.copy()
    bad[57] = 0x03  # a tail field of 3
    with pytest.raises(ValueError):
        F.unpack("tern3", bad, 1, 256)


def test_codes_against_stored_scale():
    P.q8_0_codes_against_stored_scale(F)


def test_q4_0_tie_takes_first_index():
    P.q4_0_tie_takes_first_index(F)


def test_bin8_size_saving_matches_page(golden):
    """The block part of bin8 (1 bit + one byte per 128 weights) against bin's
    1 bit + fp16 per 128: the saving the page prints (5.6 %); the per-row
    (base, step) pair adds 64 / K bits per weight on top."""
    printed = float(golden("lowbit_q1_affine_saving.txt")[0][1])
    assert F.SPECS["bin8"].bpw == 1 + 8 / 128 == 1.0625
    assert round(100 * (1 - F.SPECS["bin8"].bpw / F.SPECS["bin"].bpw), 1) == printed
    assert F.packed_size("bin8", 3, 4096) == F.packed_size("bin", 3, 4096) - 3 * 32 + 3 * 8  # 96 B meta: no pad
    assert F.packed_size("bin8", 3, 384) == 3 * 48 + 16 + 3 * 8  # 9 B of meta padded to 16


def test_bin8_affine_representable_scales_are_exact():
    P.bin8_affine_exact(F)


def test_bin8_scale_code_rounding_bound_and_constant_rows():
    P.bin8_rounding_bound(F)


def test_roundtrip_bin8_and_plane_order():
    bits = workloads.binary_codes(19, 384, seed=5)
    sc = workloads.scale_bits_f16((19, 3), seed=5, tensor_id=1)
    blk = F.bin8_from_codes(bits, sc)
    buf = F.pack("bin8", blk)
    assert buf.size == F.packed_size("bin8", 19, 384)
    P._same(F.unpack("bin8", buf, 19, 384), blk)
    # 19 * 48 B of codes, 57 B of meta padded to 64, then row r's (base, step) at 8 r
    assert np.all(buf[19 * 48 + 57:19 * 48 + 64] == 0)
    tail = buf[19 * 48 + 64:].view("<f4").reshape(19, 2)
    np.testing.assert_array_equal(tail[:, 0], blk["base"])
    np.testing.assert_array_equal(tail[:, 1], blk["step"])


# ----------------------------------------------------------------------------
# byte order (R4), pinned by hand-computed bytes


def test_nibble_and_crumb_order():
    P.byte_order(F)


def test_row_interleave_positions():
    """Hand-computed positions of the 16-row interleave (reading R8)."""
    P.row_interleave(F)


def test_kquant_meta_bytes():
    P.kquant_meta_bytes(F)


# ----------------------------------------------------------------------------
# degenerate blocks and errors (reading R3, R5)


def test_zero_and_constant_blocks():
    w = np.zeros((2, 256), np.float32)
    w[1, :32] = -0.0
    for fmt in ("q8_0", "q4_0", "q4_1", "q4_k", "q2_k"):
        blk = F.quantize(fmt, w)
        np.testing.assert_array_equal(F.dequant(fmt, blk), 0.0)
        b1 = F.pack(fmt, blk)
        b2 = F.pack(fmt, F.quantize(fmt, np.abs(w)))
        np.testing.assert_array_equal(b1, b2)  # -0 canonicalised
    assert np.all(F.quantize("q4_0", w)["n"] == 8)
    c = np.full((1, 256), -0.75, np.float32)
    deq = F.dequant("q4_k", F.quantize("q4_k", c))
    assert np.all(np.abs(deq - c) <= 0.75 / 63)


def test_errors():
    bad = np.ones((1, 256), np.float32)
    bad[0, 7] = np.nan
    for fmt in ("q8_0", "q4_0", "q4_1", "q4_k", "q2_k"):
        with pytest.raises(F.QuantInputError):
            F.quantize(fmt, bad)
    huge = np.full((1, 32), 6e4 * 127 * 2, np.float32)
    with pytest.raises(F.QuantRangeError):
        F.quantize("q8_0", huge)
    with pytest.raises(ValueError):
        F.quantize("q4_k", np.ones((1, 100), np.float32))


# ----------------------------------------------------------------------------
# a scalar re-implementation on tiny inputs guards the vectorised indexing


def _scalar_q4k(b):
    f = np.float32
    lo = [min(min(b[j * 32:(j + 1) * 32]), f(0)) for j in range(8)]
    hi = [max(b[j * 32:(j + 1) * 32]) for j in range(8)]
    sc = [f(f(hi[j] - lo[j]) / f(15)) for j in range(8)]
    mn = [-lo[j] for j in range(8)]
    D = np.float16(f(max(sc) / f(63))).astype(f)
    M = np.float16(f(max(mn) / f(63))).astype(f)
    s = [1 if D == 0 else int(np.clip(np.rint(f(sc[j] / D)), 1, 63)) for j in range(8)]
    t = [0 if M == 0 else int(np.clip(np.rint(f(mn[j] / M)), 0, 63)) for j in range(8)]
    out = []
    for j in range(8):
        S = f(f(s[j]) * D)
        Mn = f(f(t[j]) * M)
        for i in range(32):
            v = b[32 * j + i]
            out.append(0 if S == 0 else int(np.clip(np.rint(f(f(v + Mn) / S)), 0, 15)))
    return s, t, out


def test_q4k_matches_scalar_loop():
    w = workloads.student_t_weights(3, 512, seed=5)
    blk = F.quantize("q4_k", w)
    with np.errstate(divide="ignore", invalid="ignore"):
        for r in range(3):
            for sb in range(2):
                s, t, n = _scalar_q4k(list(w[r, sb * 256:(sb + 1) * 256]))
                assert list(blk["s"][r, sb]) == s
                assert list(blk["t"][r, sb]) == t
                assert list(blk["n"][r, sb * 256:(sb + 1) * 256]) == n
