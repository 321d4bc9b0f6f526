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
from oracle import page_listing as PL

F32 = np.float32

PAGE_NAMES = {"Q8_0": "q8_0", "Q4_0": "q4_0", "Q4_1": "q4_1", "Q4_K": "q4_k"}


@pytest.fixture(scope="module")
def page_w():
    return PL.page_weights()


def test_page_sample_matches_listing_shape(page_w):
    assert page_w.shape == (4096 * 256,) and page_w.dtype == np.float32


def test_error_table_page_literal(page_w, golden):
    """The restated fp32 listing reproduces the printed table to 4 decimals."""
    rows = {r[0]: (float(r[1]), float(r[2])) for r in golden("handbook_error_table.txt")}
    fns = dict(PL.LISTING)
    for name, (bpw, err) in rows.items():
        deq, bits = fns[name](page_w)
        assert f"{bits:.2f}" == f"{bpw:.2f}"
        assert round(PL.relative_error(deq, page_w), 4) == pytest.approx(err, abs=1e-12), name


def test_error_table_fp16_storage(page_w, golden):
    """Production quantizers (fp16-stored scales) stay within 0.002 of the
    printed errors and keep the printed ordering Q8_0 << Q4_1 ~ Q4_K < Q4_0."""
    rows = {r[0]: float(r[2]) for r in golden("handbook_error_table.txt")}
    w = page_w.reshape(-1, 4096)
    errs = {}
    for name, fmt in PAGE_NAMES.items():
        deq = F.dequant(fmt, F.quantize(fmt, w))
        errs[name] = PL.relative_error(deq.reshape(-1), page_w)
        assert abs(errs[name] - rows[name]) < 0.002, (name, errs[name])
    assert errs["Q8_0"] < errs["Q4_1"] < errs["Q4_0"]
    assert errs["Q8_0"] < errs["Q4_K"] < errs["Q4_0"]


def test_bpw_closed_forms(golden):
    """Plane sizes equal the listing's closed forms (and N*K*bpw/8 bytes)."""
    printed = {r[0]: float(r[1]) for r in golden("handbook_error_table.txt")}
    listing = {"Q8_0": 8 + 16 / 32, "Q4_0": 4 + 16 / 32, "Q4_1": 4 + 32 / 32,
               "Q4_K": 4 + (6 + 6) * 8 / 256 + 2 * 16 / 256}
    for name, fmt in PAGE_NAMES.items():
        assert F.SPECS[fmt].bpw == listing[name] == printed[name]
    # low-bit formats: 2-bit codes + the K-quant meta; 2-bit fields / bits + fp16 per 128
    assert F.SPECS["q2_k"].bpw == 2 + (6 + 6) * 8 / 256 + 2 * 16 / 256 == 2.5
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
# hand-built blocks


def _f16(v):
    return F.to_f16_bits(np.float32(v))


def _handbuilt_kquant(qmax, n_rows=3, n_sb=2, seed=1):
    """Codes + dyadic d/dmin such that dequant -> quantize is the identity:
    every sub-block holds codes 0 and qmax, some scale code and some min code
    are 63, and all values are exact in fp32."""
    g = np.random.default_rng(seed)
    d16 = np.full((n_rows, n_sb), _f16(2.0 ** -10), dtype=np.uint16)
    dm16 = np.full((n_rows, n_sb), _f16(2.0 ** -9), dtype=np.uint16)
    s = g.integers(1, 64, size=(n_rows, n_sb, 8)).astype(np.uint8)
    t = g.integers(0, 64, size=(n_rows, n_sb, 8)).astype(np.uint8)
    s[:, :, 0] = 63
    t[:, :, 1] = 63
    t[:, :, 2] = 0
    n = g.integers(0, qmax + 1, size=(n_rows, n_sb, 8, 32)).astype(np.uint8)
    n[..., 0] = 0
    n[..., 31] = qmax
    # sub-block 2 has min code 0 and no weight code 0: all its weights are
    # positive, so it survives the round trip only if the sub-block minimum
    # is clamped to <= 0 before the scale is formed
    n[:, :, 2] = np.maximum(n[:, :, 2], 1)
    return {"d": d16, "dmin": dm16, "s": s, "t": t, "n": n.reshape(n_rows, n_sb * 256)}


def _same(a, b):
    assert a.keys() == b.keys()
    for key in a:
        np.testing.assert_array_equal(np.asarray(a[key]), np.asarray(b[key]), err_msg=key)


@pytest.mark.parametrize("fmt,qmax", [("q4_k", 15), ("q2_k", 3)])
def test_roundtrip_kquant(fmt, qmax):
    blk = _handbuilt_kquant(qmax)
    w = F.dequant(fmt, blk)
    _same(F.quantize(fmt, w), blk)
    buf = F.pack(fmt, blk)
    assert buf.size == F.packed_size(fmt, *w.shape)
    _same(F.unpack(fmt, buf, *w.shape), blk)
    np.testing.assert_array_equal(F.dequant_packed(fmt, buf, *w.shape), w)


def test_page_listing_q4k_identity_on_handbuilt():
    """The restated listing (fp32 scales) also maps a hand-built block to itself."""
    blk = _handbuilt_kquant(15)
    w = F.dequant("q4_k", blk)
    deq, _ = PL.q4_k(w.reshape(-1))
    np.testing.assert_array_equal(deq.reshape(w.shape), w)


def test_roundtrip_q8_0():
    g = np.random.default_rng(2)
    q = g.integers(-127, 128, size=(4, 96)).astype(np.int8)
    q[:, ::32] = 127
    q[1, 32] = -127
    d16 = np.array([[_f16(v) for v in (0.5, 2.0 ** -12, 3.0)]] * 4, dtype=np.uint16)
    blk = {"d": d16, "q": q}
    w = F.dequant("q8_0", blk)
    _same(F.quantize("q8_0", w), blk)
    _same(F.unpack("q8_0", F.pack("q8_0", blk), 4, 96), blk)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_roundtrip_q4_0(sign):
    g = np.random.default_rng(3)
    c = g.integers(-7, 8, size=(3, 64))
    c[:, 5] = -8   # the unique max-|.| element, on code -8
    c[:, 40] = -8
    c[:, 41] = 7
    d16 = np.full((3, 2), _f16(sign * 2.0 ** -7), dtype=np.uint16)
    blk = {"d": d16, "n": (c + 8).astype(np.uint8)}
    w = F.dequant("q4_0", blk)
    _same(F.quantize("q4_0", w), blk)
    _same(F.unpack("q4_0", F.pack("q4_0", blk), 3, 64), blk)


def test_roundtrip_q4_1():
    g = np.random.default_rng(4)
    n = g.integers(0, 16, size=(2, 64)).astype(np.uint8)
    n[:, 0] = 0
    n[:, 31] = 15
    n[:, 32] = 15
    n[:, 63] = 0
    d16 = np.array([[_f16(2.0 ** -8), _f16(2.0 ** -6)]] * 2, dtype=np.uint16)
    m16 = np.array([[_f16(-0.25), _f16(0.125)]] * 2, dtype=np.uint16)
    blk = {"d": d16, "m": m16, "n": n}
    w = F.dequant("q4_1", blk)
    _same(F.quantize("q4_1", w), blk)
    _same(F.unpack("q4_1", F.pack("q4_1", blk), 2, 64), blk)


def test_roundtrip_tern_bin():
    codes = workloads.ternary_codes(5, 256, seed=9)
    sc = workloads.scale_bits_f16((5, 2), seed=9, tensor_id=1)
    blk = F.tern_from_codes(codes, sc)
    _same(F.unpack("tern", F.pack("tern", blk), 5, 256), blk)
    w = F.dequant("tern", blk)
    np.testing.assert_array_equal(np.sign(w), codes)
    bits = workloads.binary_codes(5, 256, seed=9)
    blk = F.bin_from_codes(bits, sc)
    _same(F.unpack("bin", F.pack("bin", blk), 5, 256), blk)
    w = F.dequant("bin", blk)
    np.testing.assert_array_equal(w > 0, bits == 1)
    np.testing.assert_array_equal(np.abs(w), np.repeat(F.from_f16_bits(sc), 128, axis=1))


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
    """Block scales 0.5 + c/256 with c covering 0..255: base = 0.5 and
    step = 1/256 come out exactly, the codes are c, and the decode equals
    bin's decode of the same fp16 scales."""
    n, k = 3, 256 * 128
    c = np.stack([np.arange(256), np.arange(255, -1, -1), (np.arange(256) * 7) % 256]).astype(np.uint8)
    c[2, 0], c[2, 1] = 0, 255
    d16 = F.to_f16_bits((0.5 + c.astype(np.float64) / 256).astype(F32))
    bits = workloads.binary_codes(n, k, seed=3)
    blk = F.bin8_from_codes(bits, d16)
    assert np.all(blk["base"] == F32(0.5)) and np.all(blk["step"] == F32(1 / 256))
    np.testing.assert_array_equal(blk["c"], c)
    np.testing.assert_array_equal(F.dequant("bin8", blk), F.dequant("bin", F.bin_from_codes(bits, d16)))


def test_bin8_scale_code_rounding_bound_and_constant_rows():
    """Any fp16 scales: each decoded scale is within half a step (plus the two
    fp32 roundings) of the given one; a row of equal scales has step 0, codes
    0 and decodes exactly."""
    n, k = 6, 128 * 40
    sc = workloads.scale_bits_f16((n, k // 128), seed=4)
    sc[5] = sc[5, 0]
    blk = F.bin8_from_codes(workloads.binary_codes(n, k, seed=4), sc)
    d = F.from_f16_bits(sc).astype(np.float64)
    got = F.bin8_scales(blk).astype(np.float64)
    bound = blk["step"].astype(np.float64)[:, None] / 2 + 2 * np.abs(d) * 2.0 ** -24
    assert np.all(np.abs(got - d) <= bound)
    assert blk["step"][5] == 0 and np.all(blk["c"][5] == 0) and np.all(got[5] == d[5])
    # the extreme blocks of every row decode to their own scales up to rounding
    for r in range(n):
        assert got[r].min() == d[r].min()


def test_roundtrip_bin8_and_plane_order():
    bits = workloads.binary_codes(19, 384, seed=5)
    sc = workloads.scale_bits_f16((19, 3), seed=5, tensor_id=1)
    blk = F.bin8_from_codes(bits, sc)
    buf = F.pack("bin8", blk)
    assert buf.size == F.packed_size("bin8", 19, 384)
    _same(F.unpack("bin8", buf, 19, 384), blk)
    # 19 * 48 B of codes, 57 B of meta padded to 64, then row r's (base, step) at 8 r
    assert np.all(buf[19 * 48 + 57:19 * 48 + 64] == 0)
    tail = buf[19 * 48 + 64:].view("<f4").reshape(19, 2)
    np.testing.assert_array_equal(tail[:, 0], blk["base"])
    np.testing.assert_array_equal(tail[:, 1], blk["step"])


# ----------------------------------------------------------------------------
# byte order (R4), pinned by hand-computed bytes


def test_nibble_and_crumb_order():
    n = np.arange(32, dtype=np.uint8)[None] % 16
    buf = F.pack("q4_0", {"d": np.array([[0x3C00]], np.uint16), "n": n})
    assert list(buf[:4]) == [0x10, 0x32, 0x54, 0x76]
    assert list(buf[16:18]) == [0x00, 0x3C]  # fp16 1.0 little-endian
    f = np.array([[0, 1, 2, 0] * 32], dtype=np.uint8)
    buf = F.pack("tern", {"d": np.array([[0x3C00]], np.uint16), "f": f})
    assert buf[0] == 0b00_10_01_00
    b = np.zeros((1, 128), np.uint8)
    b[0, [0, 3, 9]] = 1
    buf = F.pack("bin", {"d": np.array([[0x3C00]], np.uint16), "b": b})
    assert list(buf[:2]) == [0b0000_1001, 0b0000_0010]


def test_row_interleave_positions():
    """Hand-computed positions of the 16-row interleave (reading R8)."""
    n, rb = 35, 40  # two full groups + 3 rows; 2 full units + an 8-byte short unit per row
    plane = (np.arange(n * rb) % 251).astype(np.uint8).reshape(n, rb)
    buf = F.interleave_rows(plane)
    assert buf.size == n * rb
    # group 0: unit 0 of rows 0..15, then unit 1 of rows 0..15, then short units
    np.testing.assert_array_equal(buf[0:16], plane[0, 0:16])
    np.testing.assert_array_equal(buf[16:32], plane[1, 0:16])
    np.testing.assert_array_equal(buf[16 * 16:16 * 17], plane[0, 16:32])
    np.testing.assert_array_equal(buf[32 * 16:32 * 16 + 8], plane[0, 32:40])
    np.testing.assert_array_equal(buf[32 * 16 + 8:32 * 16 + 16], plane[1, 32:40])
    # group 2 (rows 32..34): starts after 32 full rows
    g2 = 32 * rb
    np.testing.assert_array_equal(buf[g2:g2 + 16], plane[32, 0:16])
    np.testing.assert_array_equal(buf[g2 + 16:g2 + 32], plane[33, 0:16])
    np.testing.assert_array_equal(buf[g2 + 3 * 32:g2 + 3 * 32 + 8], plane[32, 32:40])
    np.testing.assert_array_equal(F.deinterleave_rows(buf, n, rb), plane)


def test_kquant_meta_bytes():
    blk = _handbuilt_kquant(15, n_rows=1, n_sb=1)
    blk["d"][:] = 0x1234
    blk["dmin"][:] = 0xABCD
    blk["s"][0, 0] = np.arange(1, 9, dtype=np.uint8)
    blk["t"][0, 0] = np.arange(50, 58, dtype=np.uint8)
    meta = F.pack("q4_k", blk)[128:]
    assert list(meta[12:16]) == [0x34, 0x12, 0xCD, 0xAB]
    field = int.from_bytes(bytes(meta[0:12]), "little")
    for j in range(8):
        pj = (field >> (12 * j)) & 0xFFF
        assert pj & 0x3F == j + 1 and pj >> 6 == 50 + j


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


# planted mistakes in copies of the bin8 re-coding (R9), each caught by a pin above

def _bin8_mutant(kind):
    def recode(bits, scale_bits):
        n, k = np.asarray(bits).shape
        d = F.from_f16_bits(np.asarray(scale_bits, np.uint16).reshape(n, k // 128))
        base = d.min(axis=1)
        div = F32(256) if kind == "divisor" else F32(255)
        step = ((d.max(axis=1) - base) / div).astype(F32)
        q = (d - base[:, None]) / np.where(step == 0, F32(1), step)[:, None]
        q = np.floor(q) if kind == "floor" else np.rint(q)
        c = np.where(step[:, None] == 0, 0, np.clip(q, 0, 255)).astype(np.uint8)
        if kind == "max_base":
            base = d.max(axis=1)
        return {"b": np.asarray(bits, np.uint8), "c": c, "base": base.astype(F32), "step": step}
    return recode


@pytest.mark.parametrize("kind", ["divisor", "floor", "max_base"])
def test_bin8_planted_mistakes_fail(kind):
    mutant = _bin8_mutant(kind)
    n, k = 3, 256 * 128
    c = np.stack([np.arange(256), np.arange(255, -1, -1), (np.arange(256) * 7) % 256]).astype(np.uint8)
    d16 = F.to_f16_bits((0.5 + c.astype(np.float64) / 256).astype(F32))
    bits = workloads.binary_codes(n, k, seed=3)
    blk = mutant(bits, d16)
    exact = np.array_equal(F.dequant("bin8", blk), F.dequant("bin", F.bin_from_codes(bits, d16)))
    # the rounding-bound pin on random scales
    sc = workloads.scale_bits_f16((6, 40), seed=4)
    b2 = mutant(workloads.binary_codes(6, 40 * 128, seed=4), sc)
    d = F.from_f16_bits(sc).astype(np.float64)
    bound = b2["step"].astype(np.float64)[:, None] / 2 + 2 * np.abs(d) * 2.0 ** -24
    within = bool(np.all(np.abs(F.bin8_scales(b2).astype(np.float64) - d) <= bound))
    assert not (exact and within), f"{kind} passes both pins"
