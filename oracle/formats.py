"""Block formats: quantize, dequantize, pack, unpack (oracle; test infrastructure only).

Sources (the reader has the pages):

* Handbook page "端侧推理：llama.cpp 与 GGUF、MLX、ExecuTorch", section
  "GGUF 的量化格式" (the format list and the simplified PyTorch quantizer
  listing) defines Q8_0, Q4_0, Q4_1 and the simplified Q4_K.
* The low-bit README page ("我正让 LLM 能在小型老旧设备上运行"), kernel
  before/after table: ternary weights held in 2-bit fields with one scale per
  128 weights, 1-bit sign weights with a block scale, and Q2_K experts.
* The Flash-MoE page: 2-bit experts.

Readings where the pages are silent (each also listed with its reason in the
design notes):

R1  Scales and mins are *stored* as fp16 (the text says fp16; the listing
    keeps fp32).  Each one is computed in fp32 exactly as the listing does,
    rounded to fp16 (round-to-nearest-even, subnormals kept), and the codes
    are computed against the stored value, because that is all a decoder sees.
R2  Rounding is round-half-to-even (torch ``round``); divisions are IEEE fp32
    divisions in the order written; clamps follow rounding.
R3  A zero divisor gives the "zero" code: Q8_0 0, Q4_0 nibble 8, Q4_1 nibble 0,
    K-quant scale code 1 / min code 0 / weight code 0.  Non-finite input is
    rejected; a scale that overflows fp16 is rejected.
R4  Byte order: nibble i of a block in byte i>>1 (low nibble when i is even);
    2-bit field i in byte i>>2, bits 2*(i&3); bit i in byte i>>3, bit i&7.
    K-quant meta (16 B per 256 weights): a 96-bit little-endian field holding
    eight 12-bit pairs p_j = s_j | t_j << 6 at bits [12j, 12j+12) (bytes
    0..11), then fp16 d (bytes 12..13) and fp16 dmin (bytes 14..15).
R5  Signed zeros in the input are canonicalised to +0 before quantization
    (w + 0.0), so the sign of a zero scale is a function of the values only.
R6  Q2_K (layout on no page) is the handbook's Q4_K construction with 2-bit
    codes: 15 -> 3 and weight codes clamped to [0, 3]; 80 B per 256 weights.
R7  tern: field f = t + 1 for t in {-1, 0, +1} (3 never emitted); bin: bit 1
    means +1.  One fp16 scale per 128 weights for both.  The pages give no
    ternarizer or binarizer (those models are trained so), so these two
    "quantizers" pack given codes and scales exactly.
R8  The pages fix block contents, not where blocks sit in memory; rows are
    interleaved in groups of 16 (see the plane layout below).
R9  bin8 is the low-bit page's 1-bit format whose block scales are 8-bit
    codes of an affine map held per row (kernel table, the Q1_0 bit-plane
    row, which prints the size saving): the 1-bit codes of ``bin`` and, per
    128-weight block, one byte c_j, with the block scale
    d_j = fp32(base + fp32(step * c_j)) from a per-row fp32 pair
    (base, step).  From given fp16 block scales d (as ``bin`` takes them):
    base = min_j d_j, step = (max_j d_j - base) / 255 in fp32, and
    c_j = clamp(round_half_even((d_j - base) / step), 0, 255) (all 0 when
    step = 0).  The (base, step) pairs form a third plane after the meta
    plane, which is zero-padded to a multiple of 16 bytes: N rows of two
    little-endian fp32, row-major, not interleaved.
R10 tern3 is the low-bit page's lossless 1.875-bit form of ternary weights
    that keep one scale per 64 weights (kernel table, the ternary Q2_0 row):
    values t*d with t in {-1, 0, +1} (field f = t + 1, as in tern) and an
    fp16 d per 64 weights.  The page gives the density, not the bytes.
    Packing block: 256 weights = four 64-weight scale groups, 48 code bytes
    and 12 meta bytes (1.875 bits per weight).  Codes: for group s of the
    block, byte 12s + m (m < 12) holds the base-3 number
    sum_{l<5} f(64s + 5m + l) * 3^l (at most 242): five consecutive weights
    per byte, the first in the least significant digit.  The last four weights of each group (columns 60..63) sit in a
    32-bit field at the end of the meta entry: its byte l holds, at bits
    2s..2s+1, f(64s + 60 + l).  Meta entry: the four fp16 scales in group
    order (little-endian), then that field.  So a 64-weight group takes 12
    bytes of base-3 digits plus one byte of 2-bit fields -- the 13 bytes that
    1.875 bits per weight leave beside the 2-byte scale.  Like tern, these
    blocks pack given codes and scales exactly (no ternarizer on any page).

Plane layout of one packed [N][K] matrix (reading R8): the codes plane
followed by the meta plane.  Each plane starts from the row-major byte image
of its rows (row n = its K/bs blocks' code bytes, resp. meta bytes, in block
order) and interleaves it by groups of 16 rows: the rows of a group
(n_g = min(16, N - 16g) of them) are cut into 16-byte units, and unit u of
every row of the group is stored contiguously (row order), unit after unit;
a row whose byte count is not a multiple of 16 keeps its short last unit
(length L), and those short units follow, row after row.  So byte i of unit u
of row r in group g sits at  group_base + u*n_g*16 + r*len(u) + i,  with
len(u) = 16 except the short last unit.  Total = N*K*bpw/8 bytes.  This is the
low-bit README page's repacking of rows for the dot-product lanes (kernel
table, Q2_K row interleave), set to 16 rows: one 16-lane quarter of a gfx950
wave reads one unit of 16 rows as 256 contiguous bytes.

Page-literal mode.  The listing keeps every scale and min in fp32; the
quantizers take ``literal=True`` to do the same (no fp16 storage: the block
dict then holds fp32 scale values instead of fp16 bit patterns, which
``dequant`` accepts and ``pack`` refuses).  It exists only so the page's
printed error table can pin the quantizer arithmetic this module shares with
the listing; everything else uses fp16 storage (R1).

Parity: bin8 is pinned by the page's printed size saving (5.6 %), by exact
round trips of affine-representable scales and by the rounding bound of the
scale codes.  Q8_0, Q4_0, Q4_1, Q4_K are pinned by the page's printed error
table (page-literal mode), by the bits/weight closed forms in the listing and
by round trips of hand-built blocks.  Q2_K, tern and bin are pinned by round
trips, closed forms and brute force only (their layouts are readings).
tern3 is pinned by the page's printed density (1.875 bits per weight), by
hand-worked bytes of single weights in each position class and by exact
round trips (its byte arrangement is a reading).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32 = np.float32

FORMATS = ("q8_0", "q4_0", "q4_1", "q4_k", "q2_k", "tern", "bin", "bin8", "tern3")


class QuantInputError(ValueError):
    """Non-finite weight given to a quantizer (reading R3)."""


class QuantRangeError(ValueError):
    """A computed scale or min does not fit in fp16 (reading R3)."""


@dataclass(frozen=True)
class Spec:
    block: int        # weights per block (scale group of the meta plane)
    code_bytes: int   # bytes of codes per block
    meta_bytes: int   # bytes of meta per block

    @property
    def bpw(self) -> float:
        return (self.code_bytes + self.meta_bytes) * 8.0 / self.block


SPECS = {
    "q8_0": Spec(32, 32, 2),
    "q4_0": Spec(32, 16, 2),
    "q4_1": Spec(32, 16, 4),
    "q4_k": Spec(256, 128, 16),
    "q2_k": Spec(256, 64, 16),
    "tern": Spec(128, 32, 2),
    "bin": Spec(128, 16, 2),
    "bin8": Spec(128, 16, 1),
    "tern3": Spec(256, 48, 12),  # four 64-weight scale groups per block (R10)
}

# bytes per row of the per-row plane after the meta plane (R9)
ROW_BYTES = {"bin8": 8}


def packed_size(fmt: str, n: int, k: int) -> int:
    s = SPECS[fmt]
    if k % s.block:
        raise ValueError(f"K={k} is not a multiple of the {fmt} block ({s.block})")
    return n * (k // s.block) * s.code_bytes + _meta_span(fmt, n, k) + n * ROW_BYTES.get(fmt, 0)


def _meta_span(fmt: str, n: int, k: int) -> int:
    """Bytes of the meta plane, padded to 16 when a per-row plane follows (R9)."""
    s = SPECS[fmt]
    mp = n * (k // s.block) * s.meta_bytes
    return -(-mp // 16) * 16 if fmt in ROW_BYTES else mp


def codes_plane_size(fmt: str, n: int, k: int) -> int:
    s = SPECS[fmt]
    return n * (k // s.block) * s.code_bytes


# ----------------------------------------------------------------------------
# fp16 storage (R1)

def to_f16_bits(v) -> np.ndarray:
    """fp32 -> fp16 bit pattern, round-to-nearest-even, subnormals kept.

    Raises QuantRangeError when the value overflows fp16.
    """
    v = np.asarray(v, dtype=F32)
    with np.errstate(over="ignore", invalid="ignore"):
        h = v.astype(np.float16)
    if not np.all(np.isfinite(h)):
        raise QuantRangeError("scale or min overflows fp16")
    return h.view(np.uint16)


def from_f16_bits(bits) -> np.ndarray:
    """fp16 bit pattern -> fp32 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(F32)


def _store(v, literal: bool) -> np.ndarray:
    """A computed scale or min as stored: its fp16 bit pattern (R1), or in the
    page-literal mode the fp32 value itself."""
    return np.asarray(v, dtype=F32).copy() if literal else to_f16_bits(v)


def scale_values(stored) -> np.ndarray:
    """fp32 values of stored scales or mins: fp16 bit patterns widened exactly,
    page-literal fp32 values as they are."""
    stored = np.asarray(stored)
    if stored.dtype == np.uint16:
        return from_f16_bits(stored)
    if stored.dtype != F32:
        raise TypeError(f"stored scales must be fp16 bit patterns or fp32 values, got {stored.dtype}")
    return stored


def _canonical(w: np.ndarray, block: int) -> np.ndarray:
    w = np.asarray(w, dtype=F32)
    if w.ndim != 2:
        raise ValueError("weights must be a 2-D [N, K] array")
    if w.shape[1] % block:
        raise ValueError(f"K={w.shape[1]} is not a multiple of {block}")
    if not np.all(np.isfinite(w)):
        raise QuantInputError("non-finite weight")
    return w + F32(0.0)  # R5: -0 -> +0


def _div(a, b):
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.divide(a, b, dtype=F32)


# ----------------------------------------------------------------------------
# Quantizers (one per format).  Each returns a dict of plain arrays: the
# block representation that ``pack`` lays out and ``dequant`` decodes.

def quantize_q8_0(w, literal: bool = False) -> dict:
    """32 weights per block; d = max|b| / 127 (fp16); q = rint(b / d) in [-127, 127]."""
    w = _canonical(w, 32)
    n, k = w.shape
    b = w.reshape(n, k // 32, 32)
    a = np.abs(b).max(axis=2)
    d_st = _store(_div(a, F32(127)), literal)
    d = scale_values(d_st)[..., None]
    q = np.where(d == 0, F32(0), np.clip(np.rint(_div(b, d)), -127, 127))
    return {"d": d_st, "q": q.astype(np.int8).reshape(n, k)}


def quantize_q4_0(w, literal: bool = False) -> dict:
    """32 weights per block; signed d = (the max-|b| element, first on ties) / -8,
    so that element lands on code -8; codes rint(b / d) in [-8, 7], stored + 8."""
    w = _canonical(w, 32)
    n, k = w.shape
    b = w.reshape(n, k // 32, 32)
    j = np.argmax(np.abs(b), axis=2)  # first index of the maximum
    bj = np.take_along_axis(b, j[..., None], axis=2)[..., 0]
    d_st = _store(_div(bj, F32(-8)), literal)
    d = scale_values(d_st)[..., None]
    c = np.where(d == 0, F32(0), np.clip(np.rint(_div(b, d)), -8, 7))
    return {"d": d_st, "n": (c.astype(np.int16) + 8).astype(np.uint8).reshape(n, k)}


def quantize_q4_1(w, literal: bool = False) -> dict:
    """32 weights per block; d = (max - min) / 15 and m = min (both fp16);
    codes rint((b - m) / d) in [0, 15]."""
    w = _canonical(w, 32)
    n, k = w.shape
    b = w.reshape(n, k // 32, 32)
    lo = b.min(axis=2)
    hi = b.max(axis=2)
    d_st = _store(_div(hi - lo, F32(15)), literal)
    m_st = _store(lo, literal)
    d = scale_values(d_st)[..., None]
    m = scale_values(m_st)[..., None]
    q = np.where(d == 0, F32(0), np.clip(np.rint(_div(b - m, d)), 0, 15))
    return {"d": d_st, "m": m_st, "n": q.astype(np.uint8).reshape(n, k)}


def _quantize_kquant(w, qmax: int, literal: bool = False) -> dict:
    """Handbook's simplified K-quant with weight codes in [0, qmax].

    Per 32-weight sub-block j: lo = min(min b, 0), hi = max b,
    sc = (hi - lo) / qmax, mn = -lo.  Per 256-weight super-block: fp16
    d = max_j sc / 63 and dmin = max_j mn / 63; 6-bit codes s_j = rint(sc / d)
    in [1, 63] and t_j = rint(mn / dmin) in [0, 63]; restored S = s*d and
    Mn = t*dmin (exact in fp32); weight codes rint((b + Mn) / S) in [0, qmax];
    the weight decodes as code*S - Mn.
    """
    w = _canonical(w, 256)
    n, k = w.shape
    b = w.reshape(n, k // 256, 8, 32)
    lo = np.minimum(b.min(axis=3), F32(0))
    hi = b.max(axis=3)
    sc = _div(hi - lo, F32(qmax))
    mn = -lo
    d_st = _store(_div(sc.max(axis=2), F32(63)), literal)
    dmin_st = _store(_div(mn.max(axis=2), F32(63)), literal)
    dd = scale_values(d_st)[..., None]
    dm = scale_values(dmin_st)[..., None]
    s = np.where(dd == 0, F32(1), np.clip(np.rint(_div(sc, dd)), 1, 63))
    t = np.where(dm == 0, F32(0), np.clip(np.rint(_div(mn, dm)), 0, 63))
    S = (s * dd)[..., None]
    Mn = (t * dm)[..., None]
    q = np.where(S == 0, F32(0), np.clip(np.rint(_div(b + Mn, S)), 0, qmax))
    return {
        "d": d_st,
        "dmin": dmin_st,
        "s": s.astype(np.uint8),
        "t": t.astype(np.uint8),
        "n": q.astype(np.uint8).reshape(n, k),
    }


def quantize_q4_k(w, literal: bool = False) -> dict:
    return _quantize_kquant(w, 15, literal)


def quantize_q2_k(w, literal: bool = False) -> dict:
    return _quantize_kquant(w, 3, literal)


def tern_from_codes(codes, scale_bits) -> dict:
    """Ternary codes t in {-1, 0, +1} [N, K] plus fp16 scale bits [N, K/128]."""
    codes = np.asarray(codes)
    n, k = codes.shape
    if k % 128:
        raise ValueError("K must be a multiple of 128")
    if not np.all((codes >= -1) & (codes <= 1)):
        raise QuantInputError("ternary codes must be -1, 0 or +1")
    sb = np.asarray(scale_bits, dtype=np.uint16).reshape(n, k // 128)
    return {"d": sb.copy(), "f": (codes.astype(np.int16) + 1).astype(np.uint8)}


def tern3_from_codes(codes, scale_bits) -> dict:
    """Ternary codes t in {-1, 0, +1} [N, K] plus fp16 scale bits [N, K/64] (R10)."""
    codes = np.asarray(codes)
    n, k = codes.shape
    if k % 256:
        raise ValueError("K must be a multiple of 256")
    if not np.all((codes >= -1) & (codes <= 1)):
        raise QuantInputError("ternary codes must be -1, 0 or +1")
    sb = np.asarray(scale_bits, dtype=np.uint16).reshape(n, k // 64)
    return {"d": sb.copy(), "f": (codes.astype(np.int16) + 1).astype(np.uint8)}


def bin_from_codes(bits, scale_bits) -> dict:
    """1-bit codes in {0, 1} [N, K] (1 means +1) plus fp16 scale bits [N, K/128]."""
    bits = np.asarray(bits)
    n, k = bits.shape
    if k % 128:
        raise ValueError("K must be a multiple of 128")
    if not np.all((bits == 0) | (bits == 1)):
        raise QuantInputError("1-bit codes must be 0 or 1")
    sb = np.asarray(scale_bits, dtype=np.uint16).reshape(n, k // 128)
    return {"d": sb.copy(), "b": bits.astype(np.uint8)}


def bin8_from_codes(bits, scale_bits) -> dict:
    """1-bit codes [N, K] plus fp16 block scales [N, K/128] -> bin8 (R9): the
    scales re-coded as 8-bit codes of a per-row affine map."""
    bits = np.asarray(bits)
    n, k = bits.shape
    if k % 128:
        raise ValueError("K must be a multiple of 128")
    if not np.all((bits == 0) | (bits == 1)):
        raise QuantInputError("1-bit codes must be 0 or 1")
    d = from_f16_bits(np.asarray(scale_bits, dtype=np.uint16).reshape(n, k // 128))
    if not np.all(np.isfinite(d)):
        raise QuantInputError("block scales must be finite")
    base = d.min(axis=1)
    step = ((d.max(axis=1) - base) / F32(255)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.where(step[:, None] == 0, F32(0), np.clip(np.rint((d - base[:, None]) / step[:, None]), 0, 255))
    return {"b": bits.astype(np.uint8), "c": c.astype(np.uint8), "base": base.astype(F32), "step": step}


def bin8_scales(blk) -> np.ndarray:
    """fp32 [N, K/128] block scales of a bin8 block set: base + step * c."""
    prod = (blk["step"][:, None] * blk["c"].astype(F32)).astype(F32)
    return (blk["base"][:, None] + prod).astype(F32)


QUANTIZERS = {
    "q8_0": quantize_q8_0,
    "q4_0": quantize_q4_0,
    "q4_1": quantize_q4_1,
    "q4_k": quantize_q4_k,
    "q2_k": quantize_q2_k,
}


def quantize(fmt: str, w, literal: bool = False) -> dict:
    """fp32 [N, K] -> block representation; literal=True keeps the scales in
    fp32 as the page's listing does (see the module docstring)."""
    return QUANTIZERS[fmt](w, literal)


def relative_error(deq, w) -> float:
    """The page's accuracy figure ||deq - w|| / ||w||, evaluated in float64."""
    w64 = np.asarray(w, np.float64)
    return float(np.linalg.norm(np.asarray(deq, np.float64) - w64) / np.linalg.norm(w64))


# ----------------------------------------------------------------------------
# Dequantization: every product below is exact in fp32 (codes of <= 8 bits
# times fp16 significands); the only rounding is the final add/subtract of
# Q4_1's m and the K-quants' Mn.

def _per_block(v, block: int, k: int):
    """Broadcast a per-block [N, K/block] array over [N, K]."""
    return np.repeat(v, block, axis=-1).reshape(v.shape[0], k)


def dequant(fmt: str, blk: dict) -> np.ndarray:
    if fmt == "q8_0":
        q = blk["q"]
        return q.astype(F32) * _per_block(scale_values(blk["d"]), 32, q.shape[1])
    if fmt == "q4_0":
        nn = blk["n"]
        c = (nn.astype(np.int16) - 8).astype(F32)
        return c * _per_block(scale_values(blk["d"]), 32, nn.shape[1])
    if fmt == "q4_1":
        nn = blk["n"]
        k = nn.shape[1]
        d = _per_block(scale_values(blk["d"]), 32, k)
        m = _per_block(scale_values(blk["m"]), 32, k)
        return nn.astype(F32) * d + m
    if fmt in ("q4_k", "q2_k"):
        nn = blk["n"]
        n, k = nn.shape
        dd = scale_values(blk["d"])[..., None]
        dm = scale_values(blk["dmin"])[..., None]
        S = (blk["s"].astype(F32) * dd).reshape(n, k // 32)
        Mn = (blk["t"].astype(F32) * dm).reshape(n, k // 32)
        return nn.astype(F32) * _per_block(S, 32, k) - _per_block(Mn, 32, k)
    if fmt == "tern":
        f = blk["f"]
        return (f.astype(np.int16) - 1).astype(F32) * _per_block(scale_values(blk["d"]), 128, f.shape[1])
    if fmt == "tern3":
        f = blk["f"]
        return (f.astype(F32) - F32(1)) * _per_block(scale_values(blk["d"]), 64, f.shape[1])
    if fmt == "bin":
        bb = blk["b"]
        return (2 * bb.astype(np.int16) - 1).astype(F32) * _per_block(scale_values(blk["d"]), 128, bb.shape[1])
    if fmt == "bin8":
        bb = blk["b"]
        return (2 * bb.astype(np.int16) - 1).astype(F32) * _per_block(bin8_scales(blk), 128, bb.shape[1])
    raise KeyError(fmt)


# ----------------------------------------------------------------------------
# Byte layout (R4)

def _nibbles_to_bytes(v):
    v = v.astype(np.uint8)
    return (v[:, 0::2] | (v[:, 1::2] << 4)).astype(np.uint8)


def _bytes_to_nibbles(by, k):
    out = np.empty((by.shape[0], k), dtype=np.uint8)
    out[:, 0::2] = by & 0x0F
    out[:, 1::2] = by >> 4
    return out


def _crumbs_to_bytes(v):
    v = v.astype(np.uint8)
    return (v[:, 0::4] | (v[:, 1::4] << 2) | (v[:, 2::4] << 4) | (v[:, 3::4] << 6)).astype(np.uint8)


def _bytes_to_crumbs(by, k):
    out = np.empty((by.shape[0], k), dtype=np.uint8)
    for i in range(4):
        out[:, i::4] = (by >> (2 * i)) & 3
    return out


def _tern3_bytes(f, d16):
    """tern3 (R10): fields f [N, K] and scale bits [N, K/64] -> code bytes
    [N, K/256, 48] and meta bytes [N, K/256, 12]."""
    n, k = f.shape
    nb = k // 256
    g = f.astype(np.uint32).reshape(n, nb, 4, 64)        # [row, block, group s, column]
    main = g[..., :60].reshape(n, nb, 4, 12, 5)         # [.., s, m, l]: column 5m + l
    digits = sum(main[..., l] * 3 ** l for l in range(5))  # [.., s, m]
    codes = digits.reshape(n, nb, 48).astype(np.uint8)  # byte 12s + m
    tail = g[..., 60:]                                  # [.., s, l]: column 60 + l
    field = sum(tail[:, :, s, :] << (2 * s) for s in range(4))  # [.., l]: byte l, bits 2s
    scales = _u16_le(d16.reshape(n, nb, 4)).reshape(n, nb, 8)
    meta = np.concatenate([scales, field.astype(np.uint8)], axis=-1)
    return codes, meta


def _tern3_unbytes(codes, meta, k):
    """Inverse of ``_tern3_bytes`` for [N, K/256, 48] and [N, K/256, 12] bytes."""
    n, nb = codes.shape[:2]
    by = codes.reshape(n, nb, 4, 12).astype(np.uint32)  # [.., s, m]
    main = np.empty((n, nb, 4, 12, 5), dtype=np.uint8)
    for l in range(5):
        main[..., l] = by % 3
        by = by // 3
    if np.any(by):
        raise ValueError("tern3 code byte above 242")
    tail = np.empty((n, nb, 4, 4), dtype=np.uint8)      # [.., s, l]
    for s in range(4):
        tail[:, :, s, :] = (meta[..., 8:12] >> (2 * s)) & 3
    if np.any(tail == 3):
        raise ValueError("tern3 tail field 3")
    f = np.concatenate([main.reshape(n, nb, 4, 60), tail], axis=-1).reshape(n, k)
    return f, _le_u16(meta[..., :8].reshape(n, nb, 4, 2)).reshape(n, nb * 4)


def _kquant_meta_bytes(blk) -> np.ndarray:
    """[N, SB, 16] bytes: pairs p_j = s_j | t_j<<6 at bits [12j, 12j+12) of a
    96-bit little-endian field (bytes 0..11), then d and dmin as little-endian
    fp16 (bytes 12..13 and 14..15)."""
    d16, dm16 = blk["d"], blk["dmin"]
    n, sb = d16.shape
    p = blk["s"].astype(np.uint32) | (blk["t"].astype(np.uint32) << 6)  # [N, SB, 8], 12 bits each
    out = np.empty((n, sb, 16), dtype=np.uint8)
    for m in range(4):  # pairs (2m, 2m+1) fill bits [24m, 24m+24) = bytes 3m .. 3m+2
        v = p[..., 2 * m] | (p[..., 2 * m + 1] << 12)
        out[..., 3 * m] = v & 0xFF
        out[..., 3 * m + 1] = (v >> 8) & 0xFF
        out[..., 3 * m + 2] = (v >> 16) & 0xFF
    out[..., 12] = d16 & 0xFF
    out[..., 13] = d16 >> 8
    out[..., 14] = dm16 & 0xFF
    out[..., 15] = dm16 >> 8
    return out


def _kquant_meta_unpack(mb):
    """Inverse of ``_kquant_meta_bytes`` for an [N, SB, 16] uint8 array."""
    mb = mb.astype(np.uint32)
    d16 = (mb[..., 12] | (mb[..., 13] << 8)).astype(np.uint16)
    dm16 = (mb[..., 14] | (mb[..., 15] << 8)).astype(np.uint16)
    n, sb = d16.shape
    s = np.empty((n, sb, 8), dtype=np.uint8)
    t = np.empty((n, sb, 8), dtype=np.uint8)
    for m in range(4):
        v = mb[..., 3 * m] | (mb[..., 3 * m + 1] << 8) | (mb[..., 3 * m + 2] << 16)
        for h in range(2):
            pj = (v >> (12 * h)) & 0xFFF
            s[..., 2 * m + h] = pj & 0x3F
            t[..., 2 * m + h] = pj >> 6
    return d16, dm16, s, t


def _u16_le(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.uint16)
    return np.stack([(v & 0xFF).astype(np.uint8), (v >> 8).astype(np.uint8)], axis=-1)


def _le_u16(by) -> np.ndarray:
    by = by.astype(np.uint16)
    return (by[..., 0] | (by[..., 1] << 8)).astype(np.uint16)


ROW_GROUP = 16
UNIT = 16


def interleave_rows(plane) -> np.ndarray:
    """Row-major [N, row_bytes] plane -> the 16-row interleaved byte order."""
    plane = np.asarray(plane, dtype=np.uint8)
    n, rb = plane.shape
    units, rem = divmod(rb, UNIT)
    out = []
    for g0 in range(0, n, ROW_GROUP):
        rows = plane[g0:g0 + ROW_GROUP]
        ng = rows.shape[0]
        out.append(rows[:, :units * UNIT].reshape(ng, units, UNIT).transpose(1, 0, 2).reshape(-1))
        out.append(rows[:, units * UNIT:].reshape(-1))
    return np.concatenate(out) if out else np.zeros(0, np.uint8)


def deinterleave_rows(buf, n: int, rb: int) -> np.ndarray:
    """Inverse of ``interleave_rows``: bytes -> row-major [n, rb]."""
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    units, rem = divmod(rb, UNIT)
    plane = np.empty((n, rb), dtype=np.uint8)
    pos = 0
    for g0 in range(0, n, ROW_GROUP):
        ng = min(ROW_GROUP, n - g0)
        full = ng * units * UNIT
        plane[g0:g0 + ng, :units * UNIT] = buf[pos:pos + full].reshape(units, ng, UNIT).transpose(1, 0, 2).reshape(ng, -1)
        pos += full
        plane[g0:g0 + ng, units * UNIT:] = buf[pos:pos + ng * rem].reshape(ng, rem)
        pos += ng * rem
    return plane


def pack(fmt: str, blk: dict) -> np.ndarray:
    """Block representation -> packed bytes (codes plane then meta plane).
    Page-literal blocks (fp32 scales) have no byte layout and are refused."""
    for key in ("d", "m", "dmin"):
        if key in blk and fmt != "bin8" and np.asarray(blk[key]).dtype != np.uint16:
            raise TypeError(f"{fmt}: '{key}' must be fp16 bit patterns to be packed (page-literal blocks do not pack)")
    if fmt == "q8_0":
        codes = blk["q"].view(np.uint8)
        meta = _u16_le(blk["d"])
    elif fmt in ("q4_0",):
        codes = _nibbles_to_bytes(blk["n"])
        meta = _u16_le(blk["d"])
    elif fmt == "q4_1":
        codes = _nibbles_to_bytes(blk["n"])
        meta = np.stack([_u16_le(blk["d"]), _u16_le(blk["m"])], axis=-2)
    elif fmt == "q4_k":
        codes = _nibbles_to_bytes(blk["n"])
        meta = _kquant_meta_bytes(blk)
    elif fmt == "q2_k":
        codes = _crumbs_to_bytes(blk["n"])
        meta = _kquant_meta_bytes(blk)
    elif fmt == "tern":
        codes = _crumbs_to_bytes(blk["f"])
        meta = _u16_le(blk["d"])
    elif fmt == "tern3":
        codes, meta = _tern3_bytes(blk["f"], blk["d"])
    elif fmt == "bin":
        codes = np.packbits(blk["b"].astype(np.uint8), axis=1, bitorder="little")
        meta = _u16_le(blk["d"])
    elif fmt == "bin8":
        codes = np.packbits(blk["b"].astype(np.uint8), axis=1, bitorder="little")
        meta = blk["c"].astype(np.uint8)
    else:
        raise KeyError(fmt)
    n = codes.shape[0]
    codes = np.ascontiguousarray(codes).reshape(n, -1)
    meta = np.ascontiguousarray(meta).reshape(n, -1)
    parts = [interleave_rows(codes), interleave_rows(meta)]
    if fmt == "bin8":  # zero pad to 16, then the per-row (base, step) plane, little-endian fp32
        parts.append(np.zeros(-parts[1].size % 16, np.uint8))
        pairs = np.stack([blk["base"], blk["step"]], axis=1).astype("<f4")
        parts.append(pairs.view(np.uint8).reshape(-1))
    return np.concatenate(parts).astype(np.uint8)


def unpack(fmt: str, buf, n: int, k: int) -> dict:
    """Packed bytes -> block representation (inverse of ``pack``)."""
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    spec = SPECS[fmt]
    if buf.size != packed_size(fmt, n, k):
        raise ValueError("buffer size does not match the format and shape")
    nb = k // spec.block
    cp = codes_plane_size(fmt, n, k)
    codes = deinterleave_rows(buf[:cp], n, nb * spec.code_bytes)
    mp = n * nb * spec.meta_bytes
    meta = deinterleave_rows(buf[cp:cp + mp], n, nb * spec.meta_bytes).reshape(n, nb, spec.meta_bytes)
    if fmt == "q8_0":
        return {"d": _le_u16(meta), "q": codes.view(np.int8).copy()}
    if fmt == "q4_0":
        return {"d": _le_u16(meta), "n": _bytes_to_nibbles(codes, k)}
    if fmt == "q4_1":
        return {"d": _le_u16(meta[..., 0:2]), "m": _le_u16(meta[..., 2:4]), "n": _bytes_to_nibbles(codes, k)}
    if fmt in ("q4_k", "q2_k"):
        d16, dm16, s, t = _kquant_meta_unpack(meta)
        nn = _bytes_to_nibbles(codes, k) if fmt == "q4_k" else _bytes_to_crumbs(codes, k)
        return {"d": d16, "dmin": dm16, "s": s, "t": t, "n": nn}
    if fmt == "tern":
        return {"d": _le_u16(meta), "f": _bytes_to_crumbs(codes, k)}
    if fmt == "tern3":
        f, d16 = _tern3_unbytes(codes.reshape(n, nb, 48), meta, k)
        return {"d": d16, "f": f}
    if fmt == "bin":
        return {"d": _le_u16(meta), "b": np.unpackbits(codes, axis=1, bitorder="little")[:, :k]}
    if fmt == "bin8":
        pairs = buf[cp + _meta_span(fmt, n, k):].copy().view("<f4").reshape(n, 2).astype(F32)
        return {"b": np.unpackbits(codes, axis=1, bitorder="little")[:, :k], "c": meta[..., 0].copy(),
                "base": pairs[:, 0].copy(), "step": pairs[:, 1].copy()}
    raise KeyError(fmt)


def quantize_packed(fmt: str, w) -> np.ndarray:
    """fp32 [N, K] -> packed bytes (the quantizable formats)."""
    return pack(fmt, quantize(fmt, w))


def dequant_packed(fmt: str, buf, n: int, k: int) -> np.ndarray:
    return dequant(fmt, unpack(fmt, buf, n, k))
