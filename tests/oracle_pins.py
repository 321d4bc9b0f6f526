"""Pins of the oracle, written as functions of the oracle module they check.

Each pin raises AssertionError when the module under test disagrees with
what the pages or the mathematics fix.  The same pin runs on the oracle
itself (tests/test_oracle_*.py, which must pass) and on mutants of the
oracle's own source with one planted mistake each
(tests/test_oracle_mutations.py, which the pins must reject).  Expected
values here never come from the module under test: they are the pages'
printed figures, hand-computed bytes and codes, or brute-force sums written
out with ``math.fsum`` over exact float64 products.
"""
from __future__ import annotations

import math

import numpy as np

import workloads

F32 = np.float32

PAGE_NAMES = {"Q8_0": "q8_0", "Q4_0": "q4_0", "Q4_1": "q4_1", "Q4_K": "q4_k"}


def _f16(v) -> np.uint16:
    """fp16 bit pattern of a value exactly representable in fp16 (numpy's own cast)."""
    h = np.float16(v)
    assert float(h) == float(v), v
    return h.view(np.uint16)


def _same(a, b):
    assert a.keys() == b.keys()
    for key in a:
        np.testing.assert_array_equal(np.asarray(a[key]), np.asarray(b[key]), err_msg=key)


# ----------------------------------------------------------------------------
# Handbook page "端侧推理：llama.cpp 与 GGUF、MLX、ExecuTorch", section
# "GGUF 的量化格式": the printed error table of the quantizer listing


def error_table_literal(F, page_w, printed) -> None:
    """Page-literal mode (fp32 scales, as the listing keeps them) reproduces the
    printed relative errors to their 4 decimals."""
    for name, fmt in PAGE_NAMES.items():
        blk = F.quantize(fmt, page_w.reshape(-1, 4096), literal=True)
        err = F.relative_error(F.dequant(fmt, blk).reshape(-1), page_w)
        assert round(err, 4) == printed[name], (name, err, printed[name])


def error_table_fp16(F, page_w, printed) -> None:
    """fp16-stored scales stay within 0.002 of the printed errors and keep the
    printed order Q8_0 << Q4_1 ~ Q4_K < Q4_0."""
    errs = {}
    for name, fmt in PAGE_NAMES.items():
        deq = F.dequant(fmt, F.quantize(fmt, page_w.reshape(-1, 4096)))
        errs[name] = F.relative_error(deq.reshape(-1), page_w)
        assert abs(errs[name] - printed[name]) < 0.002, (name, errs[name])
    assert errs["Q8_0"] < errs["Q4_1"] < errs["Q4_0"]
    assert errs["Q8_0"] < errs["Q4_K"] < errs["Q4_0"]


# ----------------------------------------------------------------------------
# hand-built blocks: dequant -> quantize is the identity


def handbuilt_kquant(qmax, n_rows=3, n_sb=2, seed=1):
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


def roundtrip_kquant(F, fmt, qmax) -> None:
    blk = handbuilt_kquant(qmax)
    w = F.dequant(fmt, blk)
    _same(F.quantize(fmt, w), blk)
    buf = F.pack(fmt, blk)
    assert buf.size == F.packed_size(fmt, *w.shape)
    _same(F.unpack(fmt, buf, *w.shape), blk)
    np.testing.assert_array_equal(F.dequant_packed(fmt, buf, *w.shape), w)
    # the page-literal mode maps the same weights to the same codes and values
    lit = F.quantize(fmt, w, literal=True)
    np.testing.assert_array_equal(lit["n"], blk["n"])
    np.testing.assert_array_equal(F.dequant(fmt, lit), w)


def roundtrip_q8_0(F) -> None:
    g = np.random.default_rng(2)
    q = g.integers(-127, 128, size=(4, 96)).astype(np.int8)
    q[:, ::32] = 127
    q[1, 32] = -127
    d16 = np.array([[_f16(v) for v in (0.5, 2.0 ** -12, 3.0)]] * 4, dtype=np.uint16)
    blk = {"d": d16, "q": q}
    w = F.dequant("q8_0", blk)
    np.testing.assert_array_equal(w, q.astype(np.float64) * np.repeat([[0.5, 2.0 ** -12, 3.0]], 32, axis=1))
    _same(F.quantize("q8_0", w), blk)
    _same(F.unpack("q8_0", F.pack("q8_0", blk), 4, 96), blk)


def roundtrip_q4_0(F, sign) -> None:
    g = np.random.default_rng(3)
    c = g.integers(-7, 8, size=(3, 64))
    c[:, 5] = -8   # the unique max-|.| element, on code -8
    c[:, 40] = -8
    c[:, 41] = 7
    d16 = np.full((3, 2), _f16(sign * 2.0 ** -7), dtype=np.uint16)
    blk = {"d": d16, "n": (c + 8).astype(np.uint8)}
    w = F.dequant("q4_0", blk)
    np.testing.assert_array_equal(w, c * sign * 2.0 ** -7)
    _same(F.quantize("q4_0", w), blk)
    _same(F.unpack("q4_0", F.pack("q4_0", blk), 3, 64), blk)


def roundtrip_q4_1(F) -> None:
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
    want = n * np.repeat([[2.0 ** -8, 2.0 ** -6]], 32, axis=1) + np.repeat([[-0.25, 0.125]], 32, axis=1)
    np.testing.assert_array_equal(w, want)
    _same(F.quantize("q4_1", w), blk)
    _same(F.unpack("q4_1", F.pack("q4_1", blk), 2, 64), blk)


def roundtrip_tern_bin(F) -> None:
    codes = workloads.ternary_codes(5, 256, seed=9)
    sc = workloads.scale_bits_f16((5, 2), seed=9, tensor_id=1)
    scale = np.repeat(sc.view(np.float16).astype(np.float64), 128, axis=1)
    blk = F.tern_from_codes(codes, sc)
    _same(F.unpack("tern", F.pack("tern", blk), 5, 256), blk)
    np.testing.assert_array_equal(F.dequant("tern", blk), codes * scale)
    bits = workloads.binary_codes(5, 256, seed=9)
    blk = F.bin_from_codes(bits, sc)
    _same(F.unpack("bin", F.pack("bin", blk), 5, 256), blk)
    np.testing.assert_array_equal(F.dequant("bin", blk), np.where(bits == 1, 1.0, -1.0) * scale)


def roundtrip_tern3(F) -> None:
    """tern3 is lossless: pack -> unpack returns the codes and scales, and the
    decode is t * d with one scale per 64 weights; every code byte stays
    within 0..242 and every tail field within 0..2."""
    n, k = 7, 768
    codes = workloads.ternary_codes(n, k, seed=10)
    codes[0] = 1   # all +1: every code byte 242, every tail field 2
    codes[1] = -1  # all -1: every byte 0
    sc = workloads.scale_bits_f16((n, k // 64), seed=10, tensor_id=1)
    blk = F.tern3_from_codes(codes, sc)
    buf = F.pack("tern3", blk)
    assert buf.size == n * k * 15 // 64
    _same(F.unpack("tern3", buf, n, k), blk)
    scale = np.repeat(sc.view(np.float16).astype(np.float64), 64, axis=1)
    np.testing.assert_array_equal(F.dequant("tern3", blk), codes * scale)
    cp = F.codes_plane_size("tern3", n, k)
    code_rows = F.deinterleave_rows(buf[:cp], n, 3 * 48)
    meta_rows = F.deinterleave_rows(buf[cp:], n, 3 * 12).reshape(n, 3, 12)
    assert code_rows.max() <= 242
    assert np.all(code_rows[0] == 242) and np.all(meta_rows[0, :, 8:] == 0xAA)
    assert np.all(code_rows[1] == 0) and np.all(meta_rows[1, :, 8:] == 0)


def tern3_bytes(F) -> None:
    """Hand-worked tern3 bytes (reading R10) for one row of 256 weights, all
    t = -1 (field 0) except:
      column 0   (group 0, byte 0, digit 0) t = 0  -> byte 0 gets 1
      column 4   (group 0, byte 0, digit 4) t = +1 -> byte 0 gets 2 * 81, so 163
      column 117 (group 1, column 53 = 5 * 10 + 3: byte 12 + 10 = 22,
                  digit 3) t = +1 -> byte 22 = 2 * 27 = 54
      column 63  (group 0, tail column 3: field byte 3, bits 0..1) t = +1
      column 189 (group 2, tail column 1: field byte 1, bits 4..5) t = 0
      column 255 (group 3, tail column 3: field byte 3, bits 6..7) t = +1
    so the field bytes are 00 10 00 82; scales 1.0, 2.0, -0.5 and the
    smallest fp16 subnormal, little-endian."""
    t = np.full((1, 256), -1, np.int8)
    t[0, [0, 189]] = 0
    t[0, [4, 117, 63, 255]] = 1
    d16 = np.array([[0x3C00, 0x4000, 0xB800, 0x0001]], np.uint16)
    buf = F.pack("tern3", F.tern3_from_codes(t, d16))
    assert buf.size == 60
    want = np.zeros(48, np.uint8)
    want[0], want[22] = 163, 54
    np.testing.assert_array_equal(buf[:48], want)
    assert list(buf[48:56]) == [0x00, 0x3C, 0x00, 0x40, 0x00, 0xB8, 0x01, 0x00]
    assert list(buf[56:60]) == [0x00, 0x10, 0x00, 0x82]
    w = F.dequant("tern3", F.unpack("tern3", buf, 1, 256))
    assert w[0, 4] == 1.0 and w[0, 117] == 2.0 and w[0, 189] == 0.0 and w[0, 255] == 2.0 ** -24
    assert w[0, 1] == -1.0 and w[0, 130] == 0.5


def q2k_bytes_and_values(F) -> None:
    """Hand-worked Q2_K block (readings R4, R6): d = 1.0, dmin = 0.5, scale
    codes s_j = j + 1 and min codes t_j = 2j for the eight 32-weight
    sub-blocks; every weight code 0 except column 1 (code 1), column 6
    (code 3) and column 255 (code 2).  Code bytes: field i in byte i >> 2 at
    bits 2 (i & 3), so byte 0 = 1 << 2, byte 1 = 3 << 4, byte 63 = 2 << 6.
    Values d s_j q - dmin t_j: column 1 -> 1, column 6 -> 3, column 255 ->
    8 * 2 - 0.5 * 14 = 9, column 32 (sub-block 1, code 0) -> -1."""
    n = np.zeros((1, 256), np.uint8)
    n[0, 1], n[0, 6], n[0, 255] = 1, 3, 2
    blk = {"d": np.array([[0x3C00]], np.uint16), "dmin": np.array([[0x3800]], np.uint16),
           "s": np.arange(1, 9, dtype=np.uint8).reshape(1, 1, 8),
           "t": (2 * np.arange(8)).astype(np.uint8).reshape(1, 1, 8), "n": n}
    buf = F.pack("q2_k", blk)
    cp = F.codes_plane_size("q2_k", 1, 256)
    assert cp == 64 and buf.size == 80
    want = np.zeros(64, np.uint8)
    want[0], want[1], want[63] = 0x04, 0x30, 0x80
    np.testing.assert_array_equal(buf[:64], want)
    assert list(buf[76:80]) == [0x00, 0x3C, 0x00, 0x38]
    field = int.from_bytes(bytes(buf[64:76]), "little")
    assert [(field >> (12 * j)) & 0x3F for j in range(8)] == list(range(1, 9))
    assert [(field >> (12 * j + 6)) & 0x3F for j in range(8)] == [2 * j for j in range(8)]
    w = F.dequant_packed("q2_k", buf, 1, 256)
    assert w[0, 1] == 1.0 and w[0, 6] == 3.0 and w[0, 255] == 9.0 and w[0, 32] == -1.0 and w[0, 0] == 0.0


# ----------------------------------------------------------------------------
# hand-worked single blocks for the readings R1 and point 3 (Q4_0 ties)


def q8_0_codes_against_stored_scale(F) -> None:
    """Reading R1 worked by hand: max|b| = 1 gives d = 1/127, stored as the
    fp16 1032 * 2^-17, slightly below 1/127.  For v = 0.39762598 (fp32),
    v / (1/127) = 50.4985 would give code 50, while v / (1032 * 2^-17) =
    50.5016 gives code 51: 51 only when the codes are computed against the
    stored scale, which is all a decoder sees."""
    d = 1032 * 2.0 ** -17
    v = float(F32(0.39762598))
    assert round(v * 127) == 50 and round(v / d) == 51
    b = np.zeros((1, 32), F32)
    b[0, 0] = 1.0
    b[0, 1] = v
    blk = F.quantize("q8_0", b)
    assert int(blk["d"][0, 0]) == int(_f16(d))
    assert int(blk["q"][0, 1]) == 51
    assert int(blk["q"][0, 0]) == 127


def q4_0_tie_takes_first_index(F) -> None:
    """Handbook listing, Q4_0: the scale follows the element of largest |b|;
    between +0.5 at index 3 and -0.5 at index 7 the first index wins (torch's
    argmax returns the first maximal index), so d = 0.5 / -8 = -1/16, index 3
    decodes to 0.5 exactly and index 7 to 7 * (-1/16) = -0.4375."""
    b = np.zeros((1, 32), F32)
    b[0, 3] = 0.5
    b[0, 7] = -0.5
    w = F.dequant("q4_0", F.quantize("q4_0", b))
    assert w[0, 3] == 0.5 and w[0, 7] == -0.4375


# ----------------------------------------------------------------------------
# byte order (R4) and the 16-row interleave (R8), hand-computed bytes


def byte_order(F) -> None:
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


def kquant_meta_bytes(F) -> None:
    blk = handbuilt_kquant(15, n_rows=1, n_sb=1)
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


def row_interleave(F) -> None:
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


# ----------------------------------------------------------------------------
# bin8 (reading R9): exact affine scales and the scale-code rounding bound


def bin8_affine_exact(F) -> None:
    """Block scales 0.5 + c/256 with c covering 0..255: base = 0.5 and
    step = 1/256 come out exactly, the codes are c, and the decode equals the
    given scales times the signs."""
    n, k = 3, 256 * 128
    c = np.stack([np.arange(256), np.arange(255, -1, -1), (np.arange(256) * 7) % 256]).astype(np.uint8)
    c[2, 0], c[2, 1] = 0, 255
    d = 0.5 + c.astype(np.float64) / 256
    d16 = d.astype(np.float16).view(np.uint16)
    bits = workloads.binary_codes(n, k, seed=3)
    blk = F.bin8_from_codes(bits, d16)
    assert np.all(blk["base"] == F32(0.5)) and np.all(blk["step"] == F32(1 / 256))
    np.testing.assert_array_equal(blk["c"], c)
    np.testing.assert_array_equal(F.dequant("bin8", blk), np.where(bits == 1, 1.0, -1.0) * np.repeat(d, 128, axis=1))


def bin8_rounding_bound(F) -> None:
    """Any fp16 scales: each decoded scale is within half a step (plus the two
    fp32 roundings) of the given one; a row of equal scales has step 0, codes
    0 and decodes exactly; each row's smallest block decodes exactly."""
    n, k = 6, 128 * 40
    sc = workloads.scale_bits_f16((n, k // 128), seed=4)
    sc[5] = sc[5, 0]
    blk = F.bin8_from_codes(workloads.binary_codes(n, k, seed=4), sc)
    d = sc.view(np.float16).astype(np.float64)
    got = F.bin8_scales(blk).astype(np.float64)
    bound = (d.max(axis=1) - d.min(axis=1))[:, None] / 255 / 2 * (1 + 2.0 ** -20) + 2 * np.abs(d) * 2.0 ** -24
    assert np.all(np.abs(got - d) <= bound)
    assert blk["step"][5] == 0 and np.all(blk["c"][5] == 0) and np.all(got[5] == d[5])
    for r in range(n):
        assert got[r].min() == d[r].min()


# ----------------------------------------------------------------------------
# MoE (Flash-MoE page, sections "模型架构", "Metal 计算着色器", "每层流水线"):
# brute force with math.fsum on tiny fp32 experts


def _rows64(a):
    return [[float(v) for v in row] for row in np.asarray(a, F32)]


def expert_fsum(wg, wu, wd, x_row):
    """One expert by brute force: g_j = sum_k wg[j][k] x[k] (exact float64
    products, one rounding by fsum), likewise u; h_j = g_j / (1 + e^-g_j) * u_j
    (fused SwiGLU: silu of the gate times the up projection);
    o_i = fsum_j wd[i][j] h_j.  wg, wu are [I][H], wd is [H][I]."""
    x = [float(v) for v in np.asarray(x_row, F32)]
    g = [math.fsum(a * b for a, b in zip(row, x)) for row in _rows64(wg)]
    u = [math.fsum(a * b for a, b in zip(row, x)) for row in _rows64(wu)]
    h = [gj / (1.0 + math.exp(-gj)) * uj for gj, uj in zip(g, u)]
    o = [math.fsum(a * b for a, b in zip(row, h)) for row in _rows64(wd)]
    return g, u, h, o


def _tiny_expert(h, i, seed):
    g = np.random.default_rng(seed)
    wg = (g.standard_t(5, (i, h)) * 0.02).astype(F32)
    wu = (g.standard_t(5, (i, h)) * 0.02).astype(F32)
    wd = (g.standard_t(5, (h, i)) * 0.02).astype(F32)
    x = g.standard_normal((2, h)).astype(F32) * 4
    return wg, wu, wd, x


def expert_forward_fsum(M) -> None:
    """expert_forward against the brute-force expert on H != I (so a down
    projection applied transposed cannot even run) and on a square expert
    (where it would run and give other numbers); the activations are scaled
    so silu(g) * u, g * silu(u) and silu(u) * g all differ."""
    for h_dim, i_dim, seed in ((96, 160, 11), (128, 128, 12)):
        wg, wu, wd, x = _tiny_expert(h_dim, i_dim, seed)
        g, u, hh, o = M.expert_forward(wg, wu, wd, x)
        for b in range(x.shape[0]):
            eg, eu, eh, eo = expert_fsum(wg, wu, wd, x[b])
            tol_g = 1e-13 * (np.abs(x[b]).astype(np.float64) @ np.abs(wg).astype(np.float64).T) + 1e-300
            np.testing.assert_allclose(g[b], eg, rtol=0, atol=tol_g.max())
            np.testing.assert_allclose(u[b], eu, rtol=1e-12, atol=1e-13 * np.max(np.abs(eu)))
            np.testing.assert_allclose(hh[b], eh, rtol=1e-11, atol=1e-13 * np.max(np.abs(eh)))
            scale = np.abs(wd).astype(np.float64) @ np.abs(np.asarray(eh))
            assert np.all(np.abs(o[b] - np.asarray(eo)) <= 1e-12 * scale), "down projection"


def route_fsum(logits_row, top_k, renorm=False):
    """Softmax by brute force (max-subtracted exponentials over their fsum),
    top-K by descending probability with ties to the lower index."""
    z = [float(v) for v in np.asarray(logits_row, F32)]
    z = [-math.inf if math.isnan(v) else v for v in z]
    m = max(z)
    e = [math.exp(v - m) for v in z]
    s = math.fsum(e)
    p = [v / s for v in e]
    ids = sorted(range(len(p)), key=lambda j: (-p[j], j))[:top_k]
    w = [p[j] for j in ids]
    if renorm:
        ws = math.fsum(w)
        w = [v / ws for v in w]
    return ids, w


def route_pin(M) -> None:
    """route() against the brute-force softmax and top-K: ids exactly, weights
    to 1e-15 relative; ties to the lower index; renormalisation only on request."""
    logits = workloads.normal((5, 24), 21)
    logits[4, [3, 9, 17]] = logits[4].max() + 1.0  # a three-way tie at the top
    for renorm in (False, True):
        ids, w, _ = M.route(logits, 4, renorm=renorm)
        for t in range(logits.shape[0]):
            eids, ew = route_fsum(logits[t], 4, renorm)
            assert list(ids[t]) == eids, (t, list(ids[t]), eids)
            np.testing.assert_allclose(w[t], ew, rtol=1e-15, atol=0)
    assert list(M.route(logits, 4)[0][4][:3]) == [3, 9, 17]


def moe_combine_fsum(M) -> None:
    """The whole layer by brute force on E = 4 tiny experts + 1 shared, top-2,
    T = 2: out_t = residual_t + sum_k w_k o_{e_k} + sigmoid(s_t) o_shared,
    each expert from expert_fsum and the route from route_fsum."""
    e, h_dim, i_dim, top_k = 4, 48, 80, 2
    experts = [_tiny_expert(h_dim, i_dim, 30 + j)[:3] for j in range(e + 1)]
    wg = [ex[0] for ex in experts]
    wu = [ex[1] for ex in experts]
    wd = [ex[2] for ex in experts]
    x = workloads.normal((2, h_dim), 31) * 3
    res = workloads.normal((2, h_dim), 31, 1)
    logits = workloads.normal((2, e), 31, 2) * 2
    s = np.array([0.7, -1.3], F32)
    ref = M.moe_ref(wg, wu, wd, x, res, logits, s, top_k)
    for t in range(2):
        ids, w = route_fsum(logits[t], top_k)
        sig = 1.0 / (1.0 + math.exp(-float(s[t])))
        outs = [expert_fsum(wg[j], wu[j], wd[j], x[t])[3] for j in ids] + [expert_fsum(wg[e], wu[e], wd[e], x[t])[3]]
        coef = w + [sig]
        for n in range(h_dim):
            terms = [float(res[t, n])] + [c * o[n] for c, o in zip(coef, outs)]
            want = math.fsum(terms)
            mag = math.fsum(abs(v) for v in terms)
            assert abs(ref["out"][t, n] - want) <= 1e-12 * mag, (t, n, ref["out"][t, n], want)
        assert list(ref["ids"][t]) == ids
