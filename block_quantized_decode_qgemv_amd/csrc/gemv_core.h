// Row-group GEMV core shared by the dense GEMV (gemv.hip) and the MoE expert
// kernels (moe.hip): format traits, code decoders, interleaved addressing and
// the GemvDpp<F, B, W, KCS> device routine that computes one 16-row group.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>
#include <utility>

#include "internal.h"

namespace qg {
namespace core {

constexpr int kRowGroup = 16;          // rows per interleave group (layout constant)

// ------------------------------------------------------------------ traits
//
// CPC: weights per 16-byte code unit; MBU: meta bytes per code unit; GS:
// weights per column sum (0 = none); BLOCK, CB, MB: the format's block.
template <int F> struct Fmt;
template <> struct Fmt<QG_Q8_0> { static constexpr int CPC = 16,  MBU = 1, GS = 0,   BLOCK = 32,  CB = 32,  MB = 2; };
template <> struct Fmt<QG_Q4_0> { static constexpr int CPC = 32,  MBU = 2, GS = 32,  BLOCK = 32,  CB = 16,  MB = 2; };
template <> struct Fmt<QG_Q4_1> { static constexpr int CPC = 32,  MBU = 4, GS = 32,  BLOCK = 32,  CB = 16,  MB = 4; };
template <> struct Fmt<QG_Q4_K> { static constexpr int CPC = 32,  MBU = 2, GS = 32,  BLOCK = 256, CB = 128, MB = 16; };
template <> struct Fmt<QG_Q2_K> { static constexpr int CPC = 64,  MBU = 4, GS = 32,  BLOCK = 256, CB = 64,  MB = 16; };
template <> struct Fmt<QG_TERN> { static constexpr int CPC = 64,  MBU = 1, GS = 64,  BLOCK = 128, CB = 32,  MB = 2; };
template <> struct Fmt<QG_BIN>  { static constexpr int CPC = 128, MBU = 2, GS = 128, BLOCK = 128, CB = 16,  MB = 2; };
template <> struct Fmt<QG_BIN8> { static constexpr int CPC = 128, MBU = 1, GS = 128, BLOCK = 128, CB = 16,  MB = 1; };
// tern3: a "unit" is one 64-weight scale group (12 code bytes, its scale and
// its four tail fields); the code bytes of a 256-weight block fill three
// 16-byte units, which a lane part reads whole (4 groups) or by halves (2)
template <> struct Fmt<QG_TERN3> { static constexpr int CPC = 64, MBU = 3, GS = 64,  BLOCK = 256, CB = 48,  MB = 12; };

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Keep a masked code dword opaque to the optimizer so each byte pair converts
// with one v_cvt_pk_f32_fp8 (the mask would otherwise be re-folded into
// per-byte bit-field extracts).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Bytes 0..3 of v (each 0..15) as floats n * 2^-9 (OCP e4m3 encodes a byte n
// in 0..15 exactly as n * 2^-9, subnormals included).
__device__ __forceinline__ void fp8x4(uint32_t v, float& b0, float& b1, float& b2, float& b3) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, true);
    b0 = lo[0]; b1 = lo[1]; b2 = hi[0]; b3 = hi[1];
}

// ------------------------------------------------------------ DPP reduction

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over aligned groups of LPR lanes (LPR in 4..64); the full sum is valid in
// the last lane of each group.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<0xB1>(v);                                 // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);                                 // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) v += dpp<0x141>(v);        // row_half_mirror
    if constexpr (LPR >= 16) v += dpp<0x140>(v);       // row_mirror
    if constexpr (LPR >= 32) v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
    if constexpr (LPR >= 64) v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
    return v;
}

// -------------------------------------------------- per-format unit decode
//
// Unit<F>::decode(v, w) turns one code dword into the CPC/4 code values of
// its columns, in column order, scaled by 2^-9 (the value of the e4m3 byte
// 0x01) for the formats decoded through e4m3 (all but Q8_0).

template <int F> struct Unit;

template <> struct Unit<QG_Q8_0> {
    static constexpr int CPD = 4;
    __device__ static void decode(uint32_t v, float* w) {
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = (float)(int)(int8_t)(v >> (8 * k));
    }
};

// nibble i of a block in byte i>>1, low nibble first: byte k of a dword holds
// columns 2k (low) and 2k+1 (high)
template <> struct Unit<QG_Q4_0> {
    static constexpr int CPD = 8;
    __device__ static void decode(uint32_t v, float* w) {
        const uint32_t lo = opaque(v & 0x0F0F0F0Fu), hi = opaque((v >> 4) & 0x0F0F0F0Fu);
        fp8x4(lo, w[0], w[2], w[4], w[6]);
        fp8x4(hi, w[1], w[3], w[5], w[7]);
    }
};
template <> struct Unit<QG_Q4_1> : Unit<QG_Q4_0> {};
template <> struct Unit<QG_Q4_K> : Unit<QG_Q4_0> {};

// 2-bit field i in byte i>>2 at bits 2*(i&3): byte k of a dword holds columns
// 4k..4k+3
template <> struct Unit<QG_Q2_K> {
    static constexpr int CPD = 16;
    __device__ static void decode(uint32_t v, float* w) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t f = opaque((v >> (2 * s)) & 0x03030303u);
            fp8x4(f, w[s], w[4 + s], w[8 + s], w[12 + s]);
        }
    }
};
template <> struct Unit<QG_TERN> : Unit<QG_Q2_K> {};

// bit i in byte i>>3 at bit i&7: byte k of a dword holds columns 8k..8k+7
template <> struct Unit<QG_BIN> {
    static constexpr int CPD = 32;
    __device__ static void decode(uint32_t v, float* w) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint32_t f = opaque((v >> s) & 0x01010101u);
            fp8x4(f, w[s], w[8 + s], w[16 + s], w[24 + s]);
        }
    }
};

template <> struct Unit<QG_BIN8> : Unit<QG_BIN> {};

// tern3: the five base-3 digits of each byte of a code dword, digit l of byte
// j to w[5j + l] (the group's column 20e + 5j + l for code dword e), as
// e4m3 values n * 2^-9.  Bytes 0, 2 and 1, 3 ride in the two 16-bit halves
// of a register each (packed 16-bit integer arithmetic), and
// floor(b / 3) = (171 b) >> 9 exactly for b <= 255.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void tern3_digits(uint32_t v, float* w) {
    u16x2_t lo = __builtin_bit_cast(u16x2_t, v & 0x00FF00FFu);
    u16x2_t hi = __builtin_bit_cast(u16x2_t, (v >> 8) & 0x00FF00FFu);
#pragma unroll
    for (int l = 0; l < 4; ++l) {
        const u16x2_t ql = (lo * (unsigned short)171) >> (unsigned short)9;
        const u16x2_t qh = (hi * (unsigned short)171) >> (unsigned short)9;
        const uint32_t d = __builtin_bit_cast(uint32_t, (u16x2_t)(lo - ql * (unsigned short)3)) |
                           (__builtin_bit_cast(uint32_t, (u16x2_t)(hi - qh * (unsigned short)3)) << 8);
        fp8x4(opaque(d), w[l], w[5 + l], w[10 + l], w[15 + l]);
        lo = ql;
        hi = qh;
    }
    const uint32_t d = __builtin_bit_cast(uint32_t, lo) | (__builtin_bit_cast(uint32_t, hi) << 8);
    fp8x4(opaque(d), w[4], w[9], w[14], w[19]);
}

// tern3 with a decode table (the GEMV's default): entry b holds the five
// base-3 digits of b as e4m3 bytes (digits 0..3 in .x, digit 4 in byte 0 of
// .y), so a code byte costs one LDS read and three conversions instead of
// the arithmetic above (about 1 against 2 VALU operations per weight; batch
// 1 measured 14-18 % faster at 12288-14336 x 4096 and 4096 x 12288).  Every
// byte value has an entry (243..255 never occur in packed data), so no read
// leaves the table.  QG_TERN3_LUT=0 builds the arithmetic decode instead.
#ifndef QG_TERN3_LUT
#define QG_TERN3_LUT 1
#endif
constexpr int kTern3Lut = 256;
__device__ __forceinline__ void tern3_lut_build(uint2* lut, int tid, int nt) {
    for (int b = tid; b < kTern3Lut; b += nt) {
        uint32_t x = (uint32_t)b, lo = 0;
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            lo |= (x % 3u) << (8 * l);
            x /= 3u;
        }
        lut[b] = make_uint2(lo, x);
    }
}
__device__ __forceinline__ void tern3_digits_lut(uint32_t v, const uint2* lut, float* w) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint2 e = lut[(v >> (8 * j)) & 0xFFu];
        fp8x4(e.x, w[5 * j], w[5 * j + 1], w[5 * j + 2], w[5 * j + 3]);
        w[5 * j + 4] = __builtin_amdgcn_cvt_f32_fp8((int)e.y, 0);
    }
}

// tern3: the four tail columns (60..63) of group i from its block's field,
// shifted so that group i sits at bits 2i of each byte
__device__ __forceinline__ void tern3_tail(uint32_t field, int i, float* w) {
    fp8x4(opaque((field >> (2 * i)) & 0x03030303u), w[0], w[1], w[2], w[3]);
}

// Weight bytes are read exactly once per call: stream them past the caches.
#ifndef QG_WEIGHT_NT
#define QG_WEIGHT_NT 1
#endif
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <typename V> struct NtLoad;
template <> struct NtLoad<uint4> {
    __device__ static uint4 ld(const uint8_t* p) {
#if QG_WEIGHT_NT
        const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
        return make_uint4(v.x, v.y, v.z, v.w);
#else
        return *(const uint4*)p;
#endif
    }
};
template <> struct NtLoad<uint2> {
    __device__ static uint2 ld(const uint8_t* p) {
#if QG_WEIGHT_NT
        const u32x2_t v = __builtin_nontemporal_load((const u32x2_t*)p);
        return make_uint2(v.x, v.y);
#else
        return *(const uint2*)p;
#endif
    }
};
template <> struct NtLoad<uint32_t> {
    __device__ static uint32_t ld(const uint8_t* p) {
#if QG_WEIGHT_NT
        return __builtin_nontemporal_load((const uint32_t*)p);
#else
        return *(const uint32_t*)p;
#endif
    }
};
template <typename V>
__device__ __forceinline__ V ld_weights(const uint8_t* p) { return NtLoad<V>::ld(p); }

// --------------------------------------------------- interleaved addressing
//
// A row group g holds n_g = min(16, N - 16g) rows.  Its codes start at
// 16*g*row_codes in the codes plane and its meta at 16*g*row_meta in the meta
// plane.  Unit u of row r: base + (u*n_g + r)*16; a row's short last meta
// unit (row_meta % 16 bytes) sits after the group's full units at
// base + full_units*n_g*16 + r*rem.

// Meta bytes [o0, o0 + NB) of row r (NB = 4, 8, 16 or 32; o0 a multiple of
// min(NB, 16)).  Full units are read with one vector load each; a part that
// reaches into the short last unit is read two bytes at a time and only up to
// the row's last meta byte (bytes past it belong to no code unit in range).
template <int NB>
__device__ __forceinline__ void load_meta(const uint8_t* gm, int n_g, int r, int o0, int row_meta,
                                          uint32_t (&wd)[(NB + 3) / 4]) {
    const int full = row_meta >> 4, rem = row_meta & 15;
    constexpr int W = NB >= 16 ? 4 : (NB + 3) / 4;  // dwords per part
#pragma unroll
    for (int h = 0; h < (NB + 15) / 16; ++h) {
        const int o = o0 + 16 * h;
        const int u = o >> 4, i0 = o & 15;
        if (u < full) {
            const uint8_t* p = gm + ((size_t)u * n_g + r) * 16 + i0;
            if constexpr (W == 4) {
                const uint4 v = *(const uint4*)p;
                wd[4 * h] = v.x; wd[4 * h + 1] = v.y; wd[4 * h + 2] = v.z; wd[4 * h + 3] = v.w;
            } else if constexpr (W == 2) {
                const uint2 v = *(const uint2*)p;
                wd[0] = v.x; wd[1] = v.y;
            } else if constexpr (NB == 4) {
                wd[0] = *(const uint32_t*)p;
            } else if constexpr (NB == 2) {
                wd[0] = *(const uint16_t*)p;
            } else {
                wd[0] = *p;  // NB == 1
            }
        } else {
            const uint8_t* p = gm + (size_t)full * n_g * 16 + (size_t)r * rem;
#pragma unroll
            for (int k = 0; k < W; ++k) {
                uint32_t lo = 0, hi = 0;
                if constexpr (NB == 1) {
                    if (u == full && i0 < rem) lo = p[i0];
                } else if (u == full && i0 + 4 * k < rem) lo = *(const uint16_t*)(p + i0 + 4 * k);
                if (NB > 2 && u == full && i0 + 4 * k + 2 < rem) hi = *(const uint16_t*)(p + i0 + 4 * k + 2);
                wd[W * h + k] = lo | (hi << 16);
            }
        }
    }
}

// ----------------------------------------------------------- scale applies
//
// Apply<F>::unit(wd, i, s, P, X, st, acc, ok) folds the partial sum P (sum of
// decoded code * x over sub-group s of the lane's unit i) and the column sum X
// of that sub-group into the row sum acc, using the lane's meta words wd.
// i and s are compile-time after unrolling, so every meta field extraction
// has constant positions.  K-quants keep two running sums per batch row in st
// and apply d, dmin once per super-block.  Units with ok false lie past the
// end of K and contribute nothing.

struct KqState { float sp = 0.0f, tx = 0.0f; };

// fp16 half-word h of the meta words
__device__ __forceinline__ float meta_h(const uint32_t* wd, int h) {
    return h2f((wd[h >> 1] >> (16 * (h & 1))) & 0xFFFFu);
}

template <int F> struct Apply;

template <> struct Apply<QG_Q8_0> {
    static constexpr int SUBS = 1;
    // unit i belongs to block i/2; w = q d
    __device__ static void unit(const uint32_t* wd, int i, int, float P, float, KqState&, float& acc, bool ok) {
        const float v = fmaf(meta_h(wd, i >> 1), P, acc);
        acc = ok ? v : acc;
    }
};

template <> struct Apply<QG_Q4_0> {
    static constexpr int SUBS = 1;
    // w = (n - 8) d:  d * (512 P - 8 X)
    __device__ static void unit(const uint32_t* wd, int i, int, float P, float X, KqState&, float& acc, bool ok) {
        const float v = fmaf(meta_h(wd, i), fmaf(512.0f, P, -8.0f * X), acc);
        acc = ok ? v : acc;
    }
};

template <> struct Apply<QG_Q4_1> {
    static constexpr int SUBS = 1;
    // w = n d + m:  (512 d) P + m X
    __device__ static void unit(const uint32_t* wd, int i, int, float P, float X, KqState&, float& acc, bool ok) {
        const float v = fmaf(512.0f * meta_h(wd, 2 * i), P, fmaf(meta_h(wd, 2 * i + 1), X, acc));
        acc = ok ? v : acc;
    }
};

// K-quant meta entry: pairs p_j = s_j | t_j << 6 at bits [12j, 12j+12) of words
// 0..2, fp16 d and dmin in word 3.
__device__ __forceinline__ uint32_t kq_pair(const uint32_t* e, int j) {
    const int bit = 12 * j, w = bit >> 5, sh = bit & 31;
    return sh <= 20 ? (e[w] >> sh) : __builtin_amdgcn_alignbit(e[w + 1], e[w], sh);
}

// w = n s d - t dmin:  per super-block (512 d) * sum_j s_j P_j - dmin * sum_j t_j X_j
template <int UPS>  // code units per super-block (8 for Q4_K, 4 for Q2_K)
struct ApplyKq {
    static constexpr int SUBS = 8 / UPS;
    __device__ static void unit(const uint32_t* wd, int i, int s, float P, float X, KqState& st, float& acc, bool ok) {
        const uint32_t* e = wd + 4 * (i / UPS);
        const int j = (i % UPS) * SUBS + s;
        const uint32_t p = kq_pair(e, j);
        st.sp = fmaf((float)(p & 63u), P, st.sp);
        st.tx = fmaf((float)((p >> 6) & 63u), X, st.tx);
        if (j == 7) {
            const float v = fmaf(512.0f * h2f(e[3] & 0xFFFFu), st.sp, fmaf(-h2f(e[3] >> 16), st.tx, acc));
            acc = ok ? v : acc;
            st.sp = 0.0f;
            st.tx = 0.0f;
        }
    }
};
template <> struct Apply<QG_Q4_K> : ApplyKq<8> {};
template <> struct Apply<QG_Q2_K> : ApplyKq<4> {};

template <> struct Apply<QG_TERN> {
    static constexpr int SUBS = 1;
    // f = t + 1:  w = (f - 1) d  ->  d * (512 P - X); unit i is half of block i/2
    __device__ static void unit(const uint32_t* wd, int i, int, float P, float X, KqState&, float& acc, bool ok) {
        const float v = fmaf(meta_h(wd, i >> 1), fmaf(512.0f, P, -X), acc);
        acc = ok ? v : acc;
    }
};

template <> struct Apply<QG_TERN3> {
    static constexpr int SUBS = 1;
    // as tern, with one fp16 scale per 64-weight group: the part's scales are
    // the consecutive halves of wd
    __device__ static void unit(const uint32_t* wd, int i, int, float P, float X, KqState&, float& acc, bool ok) {
        const float v = fmaf(meta_h(wd, i), fmaf(512.0f, P, -X), acc);
        acc = ok ? v : acc;
    }
};

template <> struct Apply<QG_BIN> {
    static constexpr int SUBS = 1;
    // w = (2 beta - 1) d  ->  d * (1024 P - X)
    __device__ static void unit(const uint32_t* wd, int i, int, float P, float X, KqState&, float& acc, bool ok) {
        const float v = fmaf(meta_h(wd, i), fmaf(1024.0f, P, -X), acc);
        acc = ok ? v : acc;
    }
};

// bin8 block scale fp32(base + fp32(step * c)): two roundings, never fused
__device__ __forceinline__ float bin8_scale(float base, float step, uint32_t c) {
#pragma clang fp contract(off)
    const float prod = step * (float)c;
    return base + prod;
}

// bin8: the block scale is base + step * c for the unit's meta byte c; the
// lane's row (base, step) ride in wd[1], wd[2]
template <> struct Apply<QG_BIN8> {
    static constexpr int SUBS = 1;
    __device__ static void unit(const uint32_t* wd, int i, int, float P, float X, KqState&, float& acc, bool ok) {
        const float d = bin8_scale(__uint_as_float(wd[1]), __uint_as_float(wd[2]), (wd[0] >> (8 * i)) & 0xFFu);
        const float v = fmaf(d, fmaf(1024.0f, P, -X), acc);
        acc = ok ? v : acc;
    }
};

// --------------------------------------------------- register-x GEMV (DPP)
//
// Template: format F, batch B, waves W, code units per lane part KCS.  Grid:
// one workgroup per 16-row group; the epilogue functor receives the group's
// 16*B sums (row-major by row, then batch).  The 16 lanes of a DPP row are
// the 16 rows of the group working on one part of KCS code units (NXC =
// KCS*CPC columns from column k0); lane r keeps x columns k0 + 64m + 4r .. +3
// (m < NXC/64) of every batch row in registers, and each multiply-add reads
// its x operand from the lane holding it (row_newbcast).  x is thus read once
// per wave from the cache and never staged; column sums are DPP sums over the
// lanes of a sum group.  Part sums are combined with lane swaps inside a wave
// and through a small LDS array across waves, in a fixed order.

template <int... Is, class Fn>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, Fn&& fn) {
    (fn(std::integral_constant<int, Is>{}), ...);
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
    static_for_impl(std::make_integer_sequence<int, N>{}, fn);
}

// a[k % 4] += w[k] * (component k of lane L's xa), k = 0..3.
//
// Hazard rule: a DPP instruction reads all its VGPR operands (the broadcast x,
// the weight and the accumulator) early, so none of them may have been
// written by a VALU instruction in the two instructions before it.  The
// compiler cannot see into inline asm, so (1) every block starts with
// s_nop 1, covering whatever the compiler placed just before it, and (2)
// consecutive multiply-adds rotate over four accumulators, so an accumulator
// is read three instructions after its last write.  The x operands are only
// read, and the blocks' results are never DPP sources elsewhere.
template <int L>
__device__ __forceinline__ void fma4_bcast(float (&a)[4], const float4& xa, const float* w) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:%c12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %9 row_newbcast:%c12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:%c12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %11 row_newbcast:%c12 row_mask:0xf bank_mask:0xf"
        : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
        : "v"(xa.x), "v"(xa.y), "v"(xa.z), "v"(xa.w), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "n"(L));
}
// a[k] = w[k] * (component k of lane L's xa): the first block of a sum, so
// the accumulators need no zeroing (outputs written before the inputs are
// all read, hence early-clobber)
template <int L>
__device__ __forceinline__ void mul4_bcast(float (&a)[4], const float4& xa, const float* w) {
    asm("s_nop 1\n\t"
        "v_mul_f32_dpp %0, %4, %8 row_newbcast:%c12 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %5, %9 row_newbcast:%c12 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %6, %10 row_newbcast:%c12 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %7, %11 row_newbcast:%c12 row_mask:0xf bank_mask:0xf"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
        : "v"(xa.x), "v"(xa.y), "v"(xa.z), "v"(xa.w), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "n"(L));
}
template <int L>
__device__ __forceinline__ void mul8_bcast(float (&a)[4], const float4& xa, const float* w) {
    asm("s_nop 1\n\t"
        "v_mul_f32_dpp %0, %4, %8 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %5, %9 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %6, %10 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %7, %11 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %12 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %13 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %14 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %15 row_newbcast:%c17 row_mask:0xf bank_mask:0xf"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
        : "v"(xa.x), "v"(xa.y), "v"(xa.z), "v"(xa.w), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]),
          "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]), "n"(L), "n"(L + 1));
}

// the same for w[0..3] against lane L and w[4..7] against lane L + 1
template <int L>
__device__ __forceinline__ void fma8_bcast(float (&a)[4], const float4& xa, const float* w) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %9 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %11 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %12 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %13 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %14 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %15 row_newbcast:%c17 row_mask:0xf bank_mask:0xf"
        : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
        : "v"(xa.x), "v"(xa.y), "v"(xa.z), "v"(xa.w), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]),
          "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]), "n"(L), "n"(L + 1));
}

// lane L's value of v in every lane of its DPP row
template <int L>
__device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + L, 0xF, 0xF, true));
}

// a[t % 4] += w[t] * x[column CB + t] over the CPD columns from part column CB
// (FIRST: the accumulators start with these products)
template <int CB, int CPD, int NX4, bool FIRST>
__device__ __forceinline__ void fma_cols(float (&a)[4], const float4 (&xv)[NX4], const float* w) {
    if constexpr (CPD == 4) {
        if constexpr (FIRST) mul4_bcast<(CB % 64) / 4>(a, xv[CB / 64], w);
        else fma4_bcast<(CB % 64) / 4>(a, xv[CB / 64], w);
    } else {
        static_for<CPD / 8>([&](auto G) {
            constexpr int c = CB + 8 * decltype(G)::value;
            if constexpr (FIRST && decltype(G)::value == 0) mul8_bcast<(c % 64) / 4>(a, xv[c / 64], w);
            else fma8_bcast<(c % 64) / 4>(a, xv[c / 64], w + 8 * decltype(G)::value);
        });
    }
}

// Component C of v.
template <int C>
__device__ __forceinline__ float comp(const float4& v) {
    if constexpr (C == 0) return v.x;
    else if constexpr (C == 1) return v.y;
    else if constexpr (C == 2) return v.z;
    else return v.w;
}

// a[j] += w * (lane L's xj), j < NB (NB <= 4): one weight column against NB
// batch rows (FIRST: a[j] = the product).  Interleaving batch rows spaces the
// writes of one accumulator NB instructions apart, so with three or more
// batch rows a single accumulator per row meets the DPP rule (see fma4_bcast)
// without rotation; the block starts with s_nop 1 for whatever precedes it.
template <int L, int NB, bool FIRST>
__device__ __forceinline__ void fma_batch_bcast(float* a, float x0, float x1, float x2, float x3, float w) {
    if constexpr (FIRST) {
        if constexpr (NB == 1) {
            asm("s_nop 1\n\tv_mul_f32_dpp %0, %1, %2 row_newbcast:%c3 row_mask:0xf bank_mask:0xf"
                : "=&v"(a[0]) : "v"(x0), "v"(w), "n"(L));
        } else if constexpr (NB == 2) {
            asm("s_nop 1\n\t"
                "v_mul_f32_dpp %0, %2, %4 row_newbcast:%c5 row_mask:0xf bank_mask:0xf\n\t"
                "v_mul_f32_dpp %1, %3, %4 row_newbcast:%c5 row_mask:0xf bank_mask:0xf"
                : "=&v"(a[0]), "=&v"(a[1]) : "v"(x0), "v"(x1), "v"(w), "n"(L));
        } else if constexpr (NB == 3) {
            asm("s_nop 1\n\t"
                "v_mul_f32_dpp %0, %3, %6 row_newbcast:%c7 row_mask:0xf bank_mask:0xf\n\t"
                "v_mul_f32_dpp %1, %4, %6 row_newbcast:%c7 row_mask:0xf bank_mask:0xf\n\t"
                "v_mul_f32_dpp %2, %5, %6 row_newbcast:%c7 row_mask:0xf bank_mask:0xf"
                : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]) : "v"(x0), "v"(x1), "v"(x2), "v"(w), "n"(L));
        } else {
            asm("s_nop 1\n\t"
                "v_mul_f32_dpp %0, %4, %8 row_newbcast:%c9 row_mask:0xf bank_mask:0xf\n\t"
                "v_mul_f32_dpp %1, %5, %8 row_newbcast:%c9 row_mask:0xf bank_mask:0xf\n\t"
                "v_mul_f32_dpp %2, %6, %8 row_newbcast:%c9 row_mask:0xf bank_mask:0xf\n\t"
                "v_mul_f32_dpp %3, %7, %8 row_newbcast:%c9 row_mask:0xf bank_mask:0xf"
                : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
                : "v"(x0), "v"(x1), "v"(x2), "v"(x3), "v"(w), "n"(L));
        }
    } else {
        if constexpr (NB == 1) {
            asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%c3 row_mask:0xf bank_mask:0xf"
                : "+v"(a[0]) : "v"(x0), "v"(w), "n"(L));
        } else if constexpr (NB == 2) {
            asm("s_nop 1\n\t"
                "v_fmac_f32_dpp %0, %2, %4 row_newbcast:%c5 row_mask:0xf bank_mask:0xf\n\t"
                "v_fmac_f32_dpp %1, %3, %4 row_newbcast:%c5 row_mask:0xf bank_mask:0xf"
                : "+v"(a[0]), "+v"(a[1]) : "v"(x0), "v"(x1), "v"(w), "n"(L));
        } else if constexpr (NB == 3) {
            asm("s_nop 1\n\t"
                "v_fmac_f32_dpp %0, %3, %6 row_newbcast:%c7 row_mask:0xf bank_mask:0xf\n\t"
                "v_fmac_f32_dpp %1, %4, %6 row_newbcast:%c7 row_mask:0xf bank_mask:0xf\n\t"
                "v_fmac_f32_dpp %2, %5, %6 row_newbcast:%c7 row_mask:0xf bank_mask:0xf"
                : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]) : "v"(x0), "v"(x1), "v"(x2), "v"(w), "n"(L));
        } else {
            asm("s_nop 1\n\t"
                "v_fmac_f32_dpp %0, %4, %8 row_newbcast:%c9 row_mask:0xf bank_mask:0xf\n\t"
                "v_fmac_f32_dpp %1, %5, %8 row_newbcast:%c9 row_mask:0xf bank_mask:0xf\n\t"
                "v_fmac_f32_dpp %2, %6, %8 row_newbcast:%c9 row_mask:0xf bank_mask:0xf\n\t"
                "v_fmac_f32_dpp %3, %7, %8 row_newbcast:%c9 row_mask:0xf bank_mask:0xf"
                : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
                : "v"(x0), "v"(x1), "v"(x2), "v"(x3), "v"(w), "n"(L));
        }
    }
}

// The same for 5 to 8 batch rows in one block: one s_nop per column instead
// of one per four rows (the accumulator writes are then NB apart).
#define QG_DPPI(op, d, x) op " %" #d ", %" #x ", %[w] row_newbcast:%c[l] row_mask:0xf bank_mask:0xf\n\t"
template <int L, int NB, bool FIRST>
__device__ __forceinline__ void fma_batch_bcast_wide(float* a, const float* x, float w) {
    static_assert(NB >= 5 && NB <= 8, "wide blocks hold 5 to 8 batch rows");
    if constexpr (FIRST) {
        if constexpr (NB == 5)
            asm("s_nop 1\n\t" QG_DPPI("v_mul_f32_dpp", 0, 5) QG_DPPI("v_mul_f32_dpp", 1, 6) QG_DPPI("v_mul_f32_dpp", 2, 7)
                QG_DPPI("v_mul_f32_dpp", 3, 8) QG_DPPI("v_mul_f32_dpp", 4, 9)
                : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4])
                : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), [w] "v"(w), [l] "n"(L));
        else if constexpr (NB == 6)
            asm("s_nop 1\n\t" QG_DPPI("v_mul_f32_dpp", 0, 6) QG_DPPI("v_mul_f32_dpp", 1, 7) QG_DPPI("v_mul_f32_dpp", 2, 8)
                QG_DPPI("v_mul_f32_dpp", 3, 9) QG_DPPI("v_mul_f32_dpp", 4, 10) QG_DPPI("v_mul_f32_dpp", 5, 11)
                : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5])
                : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), [w] "v"(w), [l] "n"(L));
        else if constexpr (NB == 7)
            asm("s_nop 1\n\t" QG_DPPI("v_mul_f32_dpp", 0, 7) QG_DPPI("v_mul_f32_dpp", 1, 8) QG_DPPI("v_mul_f32_dpp", 2, 9)
                QG_DPPI("v_mul_f32_dpp", 3, 10) QG_DPPI("v_mul_f32_dpp", 4, 11) QG_DPPI("v_mul_f32_dpp", 5, 12)
                QG_DPPI("v_mul_f32_dpp", 6, 13)
                : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6])
                : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), [w] "v"(w), [l] "n"(L));
        else
            asm("s_nop 1\n\t" QG_DPPI("v_mul_f32_dpp", 0, 8) QG_DPPI("v_mul_f32_dpp", 1, 9) QG_DPPI("v_mul_f32_dpp", 2, 10)
                QG_DPPI("v_mul_f32_dpp", 3, 11) QG_DPPI("v_mul_f32_dpp", 4, 12) QG_DPPI("v_mul_f32_dpp", 5, 13)
                QG_DPPI("v_mul_f32_dpp", 6, 14) QG_DPPI("v_mul_f32_dpp", 7, 15)
                : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
                : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), [w] "v"(w),
                  [l] "n"(L));
    } else {
        if constexpr (NB == 5)
            asm("s_nop 1\n\t" QG_DPPI("v_fmac_f32_dpp", 0, 5) QG_DPPI("v_fmac_f32_dpp", 1, 6) QG_DPPI("v_fmac_f32_dpp", 2, 7)
                QG_DPPI("v_fmac_f32_dpp", 3, 8) QG_DPPI("v_fmac_f32_dpp", 4, 9)
                : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4])
                : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), [w] "v"(w), [l] "n"(L));
        else if constexpr (NB == 6)
            asm("s_nop 1\n\t" QG_DPPI("v_fmac_f32_dpp", 0, 6) QG_DPPI("v_fmac_f32_dpp", 1, 7) QG_DPPI("v_fmac_f32_dpp", 2, 8)
                QG_DPPI("v_fmac_f32_dpp", 3, 9) QG_DPPI("v_fmac_f32_dpp", 4, 10) QG_DPPI("v_fmac_f32_dpp", 5, 11)
                : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5])
                : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), [w] "v"(w), [l] "n"(L));
        else if constexpr (NB == 7)
            asm("s_nop 1\n\t" QG_DPPI("v_fmac_f32_dpp", 0, 7) QG_DPPI("v_fmac_f32_dpp", 1, 8) QG_DPPI("v_fmac_f32_dpp", 2, 9)
                QG_DPPI("v_fmac_f32_dpp", 3, 10) QG_DPPI("v_fmac_f32_dpp", 4, 11) QG_DPPI("v_fmac_f32_dpp", 5, 12)
                QG_DPPI("v_fmac_f32_dpp", 6, 13)
                : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6])
                : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), [w] "v"(w), [l] "n"(L));
        else
            asm("s_nop 1\n\t" QG_DPPI("v_fmac_f32_dpp", 0, 8) QG_DPPI("v_fmac_f32_dpp", 1, 9) QG_DPPI("v_fmac_f32_dpp", 2, 10)
                QG_DPPI("v_fmac_f32_dpp", 3, 11) QG_DPPI("v_fmac_f32_dpp", 4, 12) QG_DPPI("v_fmac_f32_dpp", 5, 13)
                QG_DPPI("v_fmac_f32_dpp", 6, 14) QG_DPPI("v_fmac_f32_dpp", 7, 15)
                : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
                : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), [w] "v"(w),
                  [l] "n"(L));
    }
}
#undef QG_DPPI

// ps[b] (+)= sum over the CPD columns from part column CB of w[t] * x_b, for
// all B >= 3 batch rows: column by column, batch rows interleaved in blocks
// of four, or (WIDE, 5 to 8 rows) all rows in one block.
template <int CB, int CPD, int NX4, int B, bool FIRST, bool WIDE>
__device__ __forceinline__ void fma_cols_batched(float (&ps)[B], const float4 (&xv)[B][NX4], const float* w) {
    static_assert(B >= 3, "hazard spacing needs three or more batch rows");
    static_assert(!WIDE || B >= 5, "wide blocks hold 5 to 8 batch rows");
    static_for<CPD>([&](auto T) {
        constexpr int t = decltype(T)::value, c = CB + t;
        constexpr int L = (c % 64) / 4, C = c % 4, M = c / 64;
        constexpr bool first = FIRST && t == 0;
        if constexpr (WIDE) {
            float x[B];
#pragma unroll
            for (int b = 0; b < B; ++b) x[b] = comp<C>(xv[b][M]);
            fma_batch_bcast_wide<L, B, first>(ps, x, w[t]);
            return;
        }
        static_for<(B + 3) / 4>([&](auto Q) {
            constexpr int b0 = 4 * decltype(Q)::value, nb = B - b0 < 4 ? B - b0 : 4;
            const float x0 = comp<C>(xv[b0][M]);
            const float x1 = nb > 1 ? comp<C>(xv[b0 + (nb > 1)][M]) : 0.0f;
            const float x2 = nb > 2 ? comp<C>(xv[b0 + 2 * (nb > 2)][M]) : 0.0f;
            const float x3 = nb > 3 ? comp<C>(xv[b0 + 3 * (nb > 3)][M]) : 0.0f;
            fma_batch_bcast<L, nb, first>(&ps[b0], x0, x1, x2, x3, w[t]);
        });
    });
}

template <int F> constexpr bool is_kquant() { return F == QG_Q4_K || F == QG_Q2_K; }

// Code units per lane part in the register-x kernel at batch B: the largest
// of 4 (2 for bin), 2, 1 whose part (KCS*CPC columns) covers whole 64-column
// spans and whole blocks (inside one super-block for K-quants) and keeps the
// x registers per lane (B * KCS * CPC / 16) within 32; else the smallest such
// part.  Fewer x registers leave room for more waves per SIMD at the larger
// batches.
template <int F> constexpr bool dpp_units_ok(int kcs) {
    using T = Fmt<F>;
    if (F == QG_TERN3) return kcs == 4 || kcs == 2;  // a whole block, or one half of it
    return (kcs * T::CPC) % 64 == 0 &&
           (is_kquant<F>() ? (T::BLOCK / T::CPC) % kcs == 0      // inside one super-block
                           : (kcs * T::CPC) % T::BLOCK == 0) &&  // whole blocks (aligned meta)
           (kcs * T::MBU >= 2 || T::MB == 1) &&                  // at least one fp16 of meta, or whole 1-byte entries
           (is_kquant<F>() || kcs * T::MBU <= 16);               // the part's meta in one 16-byte load
}
template <int F, int B> constexpr int dpp_lane_units() {
    int best = 0;
    // 1-bit parts of 4 units (512 weights per lane) decode into too many
    // registers even at batch 1
    for (int kcs = (F == QG_BIN || F == QG_BIN8) ? 2 : 4; kcs >= 1; kcs /= 2) {
        if (!dpp_units_ok<F>(kcs)) continue;
        if (B * kcs * Fmt<F>::CPC / 16 <= 32) return kcs;
        best = kcs;
    }
    return best;
}
// Largest batch for the register-x kernel: x registers per lane <= 64 with the
// narrowest part.
template <int F> constexpr int dpp_max_batch() {
    constexpr int nx = dpp_lane_units<F, 64>() * Fmt<F>::CPC / 16;  // x floats per batch row
    return 64 / nx < 8 ? 64 / nx : 8;
}

template <int F, int B, int W, int KCS>
struct GemvDpp {
    using T = Fmt<F>;
    using U = Unit<F>;
    using A = Apply<F>;
    static constexpr int NT = W * 64, P = 4 * W;
    static constexpr int CPC = T::CPC, CPD = U::CPD, GS = T::GS, SUBS = A::SUBS;
    static constexpr int SU = P * KCS;            // code units per slice
    // one DPP block per column at batches 5..8 (measured 1-4 % faster, except
    // Q2_K at batch 8, 4 % slower)
    static constexpr bool WIDE = B >= 5 && F != QG_Q2_K;
    static constexpr int NXC = KCS * CPC;         // x columns per part
    static constexpr int NX4 = NXC / 64;          // x float4 per lane per batch row
    static constexpr int MB = KCS * T::MBU;       // meta bytes per lane part
    static constexpr int DPS = 4 / SUBS;          // code dwords per sub-group
    static constexpr int UPS = is_kquant<F>() ? T::BLOCK / CPC : 1;  // units per super-block
    static_assert(NXC % 64 == 0, "a part covers whole 64-column spans");
    static_assert(dpp_units_ok<F>(KCS), "lane part width");
    static_assert(!is_kquant<F>() || UPS % KCS == 0, "a K-quant part stays in one super-block");
    static_assert(B * NX4 * 4 <= 64, "x registers per lane");

    // column sum of the GS columns from part column CS of one batch row;
    // gs[m] holds the DPP sums of span m
    template <int CS>
    __device__ static float col_sum(const float (&gs)[NX4]) {
        if constexpr (GS == 32) return row_bcast<(CS % 64) / 4>(gs[CS / 64]);
        else if constexpr (GS == 64) return gs[CS / 64];
        else return gs[CS / 64] + gs[CS / 64 + 1];  // GS == 128
    }

    template <class XRow, class Epi>
    __device__ static void run(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
                               int N, int K, int g, XRow xrow, int nb, Epi epi) {
        __shared__ float red[W * kRowGroup * B];
        run_group(codes, meta, N, K, g, xrow, nb, epi, 0, red);
    }

    // The same with the activation rows RMS-normalised on the way in:
    // x_k -> x_k * gamma_k / sqrt(mean_k x_k^2 + eps), per batch row.  The
    // waves that load x also sum its squares (every column once), gamma is
    // applied to x in registers, and the 1/rms of each batch row scales the
    // finished row sums, so the normalised x is never stored.  GAMMA false:
    // unit gain (gamma folded into W by the caller), no gamma loads.
    template <bool GAMMA = true, class XRow, class Epi>
    __device__ static void run_rmsnorm(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
                                       int N, int K, int g, XRow xrow, int nb, const float* __restrict__ gamma,
                                       float eps, Epi epi) {
        __shared__ float red[W * kRowGroup * B];
        __shared__ float red_ss[W * B];
        run_group<true, GAMMA>(codes, meta, N, K, g, xrow, nb, epi, 0, red, gamma, eps, red_ss);
    }

    // The same on waves [wave0, wave0 + W) of a larger workgroup, with the
    // cross-wave partials in red (W * 16 * B floats of LDS).  Every wave of the
    // workgroup must call it (it synchronizes the whole workgroup once; tern3
    // twice, the first time after the workgroup has built its decode table).
    // NORM, GAMMA: see run_rmsnorm; red_ss holds W * B floats.  [cb, ce):
    // the code units of each row to sum over (ce < 0: to the row's end), for
    // a split of K; cb * CPC must be a multiple of 256 columns (whole
    // super-blocks and 64-column spans).  A split sums only its own columns,
    // so NORM (which needs every column's square) takes the whole row.
    template <bool NORM = false, bool GAMMA = true, class XRow, class Epi>
    __device__ static void run_group(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
                                     int N, int K, int g, XRow xrow, int nb, Epi epi, int wave0, float* red,
                                     const float* __restrict__ gamma = nullptr, float eps = 0.0f,
                                     float* red_ss = nullptr, int cb = 0, int ce = -1) {
        const int tid = threadIdx.x - 64 * wave0, lane = tid & 63, wave = tid >> 6;
        const int r = lane & 15, p = wave * 4 + (lane >> 4);
        const int n_g = min(kRowGroup, N - g * kRowGroup);
        const int rr = min(r, n_g - 1);
        const int nb_blocks = K / T::BLOCK;
        const int row_codes = nb_blocks * T::CB, row_meta = nb_blocks * T::MB;
        const int nch = K / CPC;              // code units of a row (tern3: 64-weight groups)
        const int c_end = ce < 0 ? nch : ce;  // this call's units: [cb, c_end)
        const int k_end = c_end * CPC;        // and columns: [cb * CPC, k_end)
        const bool meta_whole = (row_meta & 15) == 0;
        const int ustride = n_g * 16;
        // uniform group bases plus unsigned 32-bit lane offsets (scalar-base loads)
        const uint8_t* gc = codes + (size_t)g * kRowGroup * row_codes;
        const uint8_t* gm = meta + (size_t)g * kRowGroup * row_meta;
        const uint32_t ro = (uint32_t)rr * 16;

        // bin8: the meta byte of the part plus the row's (base, step), from
        // the per-row plane after the 16-byte-padded meta plane
        uint32_t wx[3] = {0u, 0u, 0u};
        if constexpr (F == QG_BIN8) {
            const size_t span = ((size_t)N * row_meta + 15) / 16 * 16;
            const float2 ab = *(const float2*)(meta + span + ((size_t)g * kRowGroup + rr) * 8);
            wx[1] = __float_as_uint(ab.x);
            wx[2] = __float_as_uint(ab.y);
        }
        // tern3 decode table (one per workgroup, built before the first slice)
        [[maybe_unused]] uint2* t3lut = nullptr;
        if constexpr (F == QG_TERN3 && QG_TERN3_LUT) {
            __shared__ uint2 lut[kTern3Lut];
            tern3_lut_build(lut, threadIdx.x, blockDim.x);
            __syncthreads();
            t3lut = lut;
        }
        float acc[B], ss[B];  // row sums; sums of x^2 (NORM)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = ss[b] = 0.0f;

        // FULL: a whole 16-row group and whole slices, so no address needs a
        // clamp and every part is valid (constant strides).  Batch 1 keeps the
        // clamped loop alone: with this second copy it measured 2-6 % slower
        // on Q4_K; from batch 2 up the copy is as fast or faster (Q4_K batch 2:
        // up to 10 %).
        auto slices = [&](auto full_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            const uint32_t ust = FULL ? kRowGroup * 16 : (uint32_t)ustride;
            const uint32_t rof = FULL ? (uint32_t)r * 16 : ro;
            for (int c_slice = cb; c_slice < c_end; c_slice += SU) {
                const int c0 = c_slice + p * KCS;  // first code unit of this lane's part
                const int k0 = c0 * CPC;           // its first column
                const int nvalid = FULL ? KCS : c_end - c0;

                // (1) x of the part, four columns per lane per span
                float4 xv[B][NX4];
                float4 gv[NORM && GAMMA ? NX4 : 1];  // gamma of the same columns
                if constexpr (NORM && GAMMA) {
#pragma unroll
                    for (int m = 0; m < NX4; ++m) {
                        const uint32_t c = (uint32_t)(FULL ? k0 + 64 * m + 4 * r : min(k0 + 64 * m + 4 * r, k_end - 4));
                        gv[m] = *(const float4*)((const uint8_t*)gamma + c * 4u);
                    }
                }
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    if (b < nb) {
                        const float* xb = xrow(b);
#pragma unroll
                        for (int m = 0; m < NX4; ++m) {
                            // columns past K read the row's last float4 instead: they
                            // only meet code units whose contributions are dropped
                            const uint32_t c = (uint32_t)(FULL ? k0 + 64 * m + 4 * r : min(k0 + 64 * m + 4 * r, k_end - 4));
                            xv[b][m] = *(const float4*)((const uint8_t*)xb + c * 4u);
                        }
                    }
                }
                if constexpr (NORM) {
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        if (b >= nb) continue;
#pragma unroll
                        for (int m = 0; m < NX4; ++m) {
                            const float4 v = xv[b][m];
                            // each column once: the lanes of a part tile it, parts are
                            // disjoint, and clamped columns past K are not added
                            const float sq = fmaf(v.w, v.w, fmaf(v.z, v.z, fmaf(v.y, v.y, fmaf(v.x, v.x, ss[b]))));
                            if (FULL || k0 + 64 * m + 4 * r < k_end) ss[b] = sq;
                            if constexpr (GAMMA) {
                                const float4 g4 = gv[m];
                                xv[b][m] = make_float4(v.x * g4.x, v.y * g4.y, v.z * g4.z, v.w * g4.w);
                            }
                        }
                    }
                }
                // (2) meta, then the code units (clamped into the row; units past
                // its end are dropped by the scale step)
                uint32_t wd[is_kquant<F>() ? 4 : (MB + 3) / 4];
                uint4 q[F == QG_TERN3 ? 1 : KCS];
                uint32_t t3[F == QG_TERN3 ? 3 * KCS : 1];  // tern3: the part's code dwords, 3 per group
                uint32_t t3f = 0;                            // tern3: tail field, group i at bits 2i
                if constexpr (F == QG_TERN3) {
                    // a part is a whole block (KCS 4) or one half of it (KCS 2), wholly
                    // inside the row or wholly past it (then clamped to the last part)
                    const int ce0 = FULL ? c0 : min(c0, c_end - KCS);
                    const uint32_t blk = (uint32_t)ce0 >> 2, h = ((uint32_t)ce0 >> 1) & 1u;
                    const int mo = 12 * (int)blk;  // the block's meta entry in the row's meta bytes
                    auto meta_dw = [&](int o) -> uint32_t {
                        if (meta_whole || (o >> 4) < (row_meta >> 4))
                            return ld_weights<uint32_t>(gm + ((uint32_t)(o >> 4) * ust + rof + (uint32_t)(o & 15)));
                        uint32_t m1[1];
                        load_meta<4>(gm, n_g, rr, o, row_meta, m1);
                        return m1[0];
                    };
                    if constexpr (KCS == 4) {
#pragma unroll
                        for (int u = 0; u < 3; ++u) {
                            const uint4 v = ld_weights<uint4>(gc + ((3 * blk + u) * ust + rof));
                            t3[4 * u] = v.x; t3[4 * u + 1] = v.y; t3[4 * u + 2] = v.z; t3[4 * u + 3] = v.w;
                        }
                        wd[0] = meta_dw(mo);
                        wd[1] = meta_dw(mo + 4);
                        t3f = meta_dw(mo + 8);
                    } else {
                        // half h: code dwords 6h .. 6h+5 of the block, i.e. unit 2h whole
                        // and the half h of unit 1
                        const uint4 a = ld_weights<uint4>(gc + ((3 * blk + 2 * h) * ust + rof));
                        const uint2 b = ld_weights<uint2>(gc + ((3 * blk + 1) * ust + rof + 8 * h));
                        t3[0] = h ? b.x : a.x; t3[1] = h ? b.y : a.y; t3[2] = h ? a.x : a.z;
                        t3[3] = h ? a.y : a.w; t3[4] = h ? a.z : b.x; t3[5] = h ? a.w : b.y;
                        wd[0] = meta_dw(mo + 4 * (int)h);
                        t3f = meta_dw(mo + 8) >> (4 * h);
                    }
                } else if constexpr (is_kquant<F>()) {
                    const int sbi = c0 / UPS, uo = c0 % UPS;
                    const uint32_t u = (uint32_t)(FULL ? sbi : min(sbi, (c_end - 1) / UPS));
                    const uint4 v = ld_weights<uint4>(gm + (u * ust + rof));
                    // pairs of the part's first unit moved to the bottom of the field
                    const unsigned __int128 f =
                        ((unsigned __int128)v.z << 64 | (unsigned __int128)v.y << 32 | v.x) >> (12 * SUBS * uo);
                    wd[0] = (uint32_t)f; wd[1] = (uint32_t)(f >> 32); wd[2] = (uint32_t)(f >> 64); wd[3] = v.w;
                } else {
                    const int m0 = (FULL ? c0 : min(c0, (c_end - 1) / KCS * KCS)) * T::MBU;
                    if (meta_whole) {
                        const uint8_t* pm = gm + ((uint32_t)(m0 >> 4) * ust + rof + (m0 & 15));
                        if constexpr (MB >= 16) {
                            const uint4 v = ld_weights<uint4>(pm);
                            wd[0] = v.x; wd[1] = v.y; wd[2] = v.z; wd[3] = v.w;
                        } else if constexpr (MB == 8) {
                            const uint2 v = ld_weights<uint2>(pm);
                            wd[0] = v.x; wd[1] = v.y;
                        } else if constexpr (MB == 4) {
                            wd[0] = ld_weights<uint32_t>(pm);
                        } else if constexpr (MB == 2) {
                            wd[0] = *(const uint16_t*)pm;
                        } else {
                            wd[0] = *pm;  // MB == 1
                        }
                    } else {
                        load_meta<MB>(gm, n_g, rr, m0, row_meta, wd);
                    }
                    if constexpr (F == QG_BIN8) wx[0] = wd[0];
                }
                if constexpr (F != QG_TERN3) {
#pragma unroll
                    for (int i = 0; i < KCS; ++i) {
                        const uint32_t u = (uint32_t)(FULL ? c0 + i : min(c0 + i, c_end - 1));
                        q[i] = ld_weights<uint4>(gc + (u * ust + rof));
                    }
                }

                // (3) column-sum spans of every batch row
                float gs[B][NX4];
                if constexpr (GS > 0) {
#pragma unroll
                    for (int b = 0; b < B; ++b)
#pragma unroll
                        for (int m = 0; m < NX4; ++m) {
                            const float s = (xv[b][m].x + xv[b][m].y) + (xv[b][m].z + xv[b][m].w);
                            gs[b][m] = GS == 32 ? group_sum<8>(s) : group_sum<16>(s);
                        }
                }

                // (4) decode each unit once, multiply-add it for every batch row
                KqState st[B];
                static_for<KCS>([&](auto I) {
                    constexpr int i = decltype(I)::value;
                    const bool ok = i < nvalid;
                    if constexpr (F == QG_TERN3) {
                        // group i: three code dwords of 20 columns, then the four tail columns
                        float ps[B];
                        if constexpr (B >= 3) {
                            static_for<3>([&](auto E) {
                                constexpr int e = decltype(E)::value;
                                float w[20];
                                if constexpr (QG_TERN3_LUT) tern3_digits_lut(t3[3 * i + e], t3lut, w);
                                else tern3_digits(t3[3 * i + e], w);
                                fma_cols_batched<i * CPC + 20 * e, 20, NX4, B, e == 0, WIDE>(ps, xv, w);
                            });
                            float w[4];
                            tern3_tail(t3f, i, w);
                            fma_cols_batched<i * CPC + 60, 4, NX4, B, false, WIDE>(ps, xv, w);
                        } else {
                            float pa[B][4];  // started by the first column block's multiplies
                            static_for<3>([&](auto E) {
                                constexpr int e = decltype(E)::value;
                                float w[20];
                                if constexpr (QG_TERN3_LUT) tern3_digits_lut(t3[3 * i + e], t3lut, w);
                                else tern3_digits(t3[3 * i + e], w);
                                static_for<5>([&](auto G) {
                                    constexpr int c = 20 * e + 4 * decltype(G)::value;
#pragma unroll
                                    for (int b = 0; b < B; ++b)
                                        fma_cols<i * CPC + c, 4, NX4, c == 0>(pa[b], xv[b], w + (c - 20 * e));
                                });
                            });
                            float w[4];
                            tern3_tail(t3f, i, w);
#pragma unroll
                            for (int b = 0; b < B; ++b) fma_cols<i * CPC + 60, 4, NX4, false>(pa[b], xv[b], w);
#pragma unroll
                            for (int b = 0; b < B; ++b) ps[b] = (pa[b][0] + pa[b][1]) + (pa[b][2] + pa[b][3]);
                        }
#pragma unroll
                        for (int b = 0; b < B; ++b) A::unit(wd, i, 0, ps[b], col_sum<i * CPC>(gs[b]), st[b], acc[b], ok);
                    } else {
                    const uint32_t dw[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
                    static_for<SUBS>([&](auto S) {
                        constexpr int s = decltype(S)::value;
                        float ps[B];
                        if constexpr (B >= 3) {
                            // one accumulator per batch row, batch rows interleaved
                            static_for<DPS>([&](auto D) {
                                constexpr int d = s * DPS + decltype(D)::value;
                                float w[CPD];
                                U::decode(dw[d], w);
                                fma_cols_batched<i * CPC + d * CPD, CPD, NX4, B, decltype(D)::value == 0, WIDE>(ps, xv, w);
                            });
                        } else {
                            float pa[B][4];  // started by the first dword's multiplies
                            static_for<DPS>([&](auto D) {
                                constexpr int d = s * DPS + decltype(D)::value;
                                float w[CPD];
                                U::decode(dw[d], w);
#pragma unroll
                                for (int b = 0; b < B; ++b)
                                    fma_cols<i * CPC + d * CPD, CPD, NX4, decltype(D)::value == 0>(pa[b], xv[b], w);
                            });
#pragma unroll
                            for (int b = 0; b < B; ++b) ps[b] = (pa[b][0] + pa[b][1]) + (pa[b][2] + pa[b][3]);
                        }
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            float X = 0.0f;
                            if constexpr (GS > 0) X = col_sum<i * CPC + s * (CPC / SUBS)>(gs[b]);
                            if constexpr (is_kquant<F>()) {
                                const uint32_t pr = kq_pair(wd, i * SUBS + s);
                                st[b].sp = fmaf((float)(pr & 63u), ps[b], st[b].sp);
                                st[b].tx = fmaf((float)((pr >> 6) & 63u), X, st[b].tx);
                            } else {
                                if constexpr (F == QG_BIN8) A::unit(wx, i, s, ps[b], X, st[b], acc[b], ok);
                                else A::unit(wd, i, s, ps[b], X, st[b], acc[b], ok);
                            }
                        }
                    });
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
                if constexpr (is_kquant<F>()) {
                    // a K-quant part lies in one super-block: valid as a whole or not at all
                    const float d = 512.0f * h2f(wd[3] & 0xFFFFu), dmin = h2f(wd[3] >> 16);
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float v = fmaf(d, st[b].sp, fmaf(-dmin, st[b].tx, acc[b]));
                        acc[b] = nvalid > 0 ? v : acc[b];
                    }
                }
            }
        };
        if constexpr (B > 1) {
            if (n_g == kRowGroup && (c_end - cb) % SU == 0) slices(std::true_type{});
            else slices(std::false_type{});
        } else {
            slices(std::false_type{});
        }

        // (5) combine the parts: lanes r, r+16, r+32, r+48 of a wave, then waves
#pragma unroll
        for (int b = 0; b < B; ++b) {
            // (lanes l and l ^ 32, then l and l ^ 16: VALU lane swaps, no LDS)
            const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[b]), __float_as_uint(acc[b]),
                                                            false, false);
            const float v2 = __uint_as_float(h[0]) + __uint_as_float(h[1]);
            const auto q2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v2), false, false);
            const float v = __uint_as_float(q2[0]) + __uint_as_float(q2[1]);
            if (lane < 16) red[(wave * kRowGroup + r) * B + b] = v;
        }
        if constexpr (NORM) {
            // the wave's sum of squares per batch row: the four rows of lanes,
            // then the 16 lanes of a row (valid in its last lane)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss[b]), __float_as_uint(ss[b]),
                                                                false, false);
                const float v2 = __uint_as_float(h[0]) + __uint_as_float(h[1]);
                const auto q2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v2), false,
                                                                 false);
                const float v = group_sum<16>(__uint_as_float(q2[0]) + __uint_as_float(q2[1]));
                if (lane == 15) red_ss[wave * B + b] = v;
            }
        }
        __syncthreads();
        epi(
            [&](int t) {
                float v = 0.0f;
#pragma unroll
                for (int w = 0; w < W; ++w) v += red[w * kRowGroup * B + t];
                if constexpr (NORM) {
                    const int b = t % B;
                    float q = 0.0f;
#pragma unroll
                    for (int w = 0; w < W; ++w) q += red_ss[w * B + b];
                    // hardware reciprocal and reciprocal square root (about
                    // 1 ulp each), well inside the bound's fp32 allowance
                    v *= __builtin_amdgcn_rsqf(fmaf(q, __builtin_amdgcn_rcpf((float)K), eps));
                }
                return v;
            },
            n_g, tid);
    }
};

// Most waves per workgroup of the register-x kernel at batch B: 16, or 8 when
// more than 40 x registers per lane would leave too few VGPRs under the
// 128-per-wave limit of a 1024-thread workgroup.
template <int F, int B>
constexpr int dpp_max_waves() {
    return B * (dpp_lane_units<F, B>() * Fmt<F>::CPC / 16) > 40 ? 8 : 16;
}

// Waves per workgroup of the register-x kernel: the fewest (powers of two up
// to max_w) whose 4W parts cover the row in one slice, else max_w and several
// slices.
template <int F, int KCS>
int pick_waves_dpp(int K, int max_w = 16) {
    const int nch = K / Fmt<F>::CPC;
    int w = 1;
    while (w < max_w && 4 * w * KCS < nch) w *= 2;
    return w;
}

}  // namespace core
}  // namespace qg
