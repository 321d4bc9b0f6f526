// Block-quantized decode GEMV and dequant kernels for gfx950 (CDNA4).
//
// The operation is the handbook page's decode step ("端侧推理：llama.cpp 与
// GGUF、MLX、ExecuTorch", section "速度上限：带宽 ÷ 权重字节数"): every weight
// row is read once and dotted with the activation vector, y = W x, batch B
// stacking activation rows.  Block formats: section "GGUF 的量化格式" of the
// same page, plus Q2_K, ternary-in-2-bit and 1-bit from the low-bit README
// page's kernel table.
//
// Kernel shape (batch 1 is HBM-bound, so nothing here is a matrix-core
// contraction):
//   * a workgroup is 4 waves; it stages the activation slice x[B][k0:k0+KS]
//     in LDS once, plus per-group column sums X (the offset terms of Q4_0,
//     Q4_1, the K-quants and the low-bit formats are applied once per group
//     as scale * X instead of once per weight);
//   * each wave owns 64/LPR lane groups of R rows; lane sl of a group walks
//     the 16-byte code chunks sl, sl+LPR, ... of its rows, so one wave load
//     instruction reads LPR*16 contiguous bytes of every row (128-bit
//     coalesced streaming), and every x value read from LDS feeds R rows;
//   * codes are decoded in registers (mask/shift, byte -> float convert) and
//     multiplied in fp32; scales are decoded once per chunk and applied to
//     the chunk's partial sum -- the Flash-MoE page's fma(nibble, scale*x,
//     bias*x) rearrangement ("FMA 优化的反量化内核") with the bias term
//     hoisted over the shared x as bias * sum(x);
//   * lane partials are reduced with DPP (quad_perm, row mirrors,
//     row_bcast15/31) in a fixed order, so results are deterministic.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace qg {
namespace {

constexpr int kThreads = 256;            // 4 waves per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kLdsBudget = 64 * 1024;    // bytes of x + sums staged per workgroup

// ------------------------------------------------------------------ traits

template <int F> struct Fmt;
// CPC: columns (weights) per 16-byte code chunk; GS: columns per staged
// x-sum (0 = the format needs none); BLOCK / MB: weights and meta bytes per
// meta entry.
template <> struct Fmt<QG_Q8_0> { static constexpr int CPC = 16, GS = 0, BLOCK = 32, MB = 2, CB = 32; };
template <> struct Fmt<QG_Q4_0> { static constexpr int CPC = 32, GS = 32, BLOCK = 32, MB = 2, CB = 16; };
template <> struct Fmt<QG_Q4_1> { static constexpr int CPC = 32, GS = 32, BLOCK = 32, MB = 4, CB = 16; };
template <> struct Fmt<QG_Q4_K> { static constexpr int CPC = 32, GS = 32, BLOCK = 256, MB = 16, CB = 128; };
template <> struct Fmt<QG_Q2_K> { static constexpr int CPC = 64, GS = 32, BLOCK = 256, MB = 16, CB = 64; };
template <> struct Fmt<QG_TERN> { static constexpr int CPC = 64, GS = 64, BLOCK = 128, MB = 2, CB = 32; };
template <> struct Fmt<QG_BIN>  { static constexpr int CPC = 128, GS = 128, BLOCK = 128, MB = 2, CB = 16; };

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ float ubyte(uint32_t v, int k) { return (float)((v >> (8 * k)) & 0xFFu); }

// Hide a masked code dword from the optimizer so that each byte converts
// with one v_cvt_f32_ubyte{0..3} instead of a bit-field extract plus a
// convert (the mask would otherwise be folded into per-byte extracts).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// ------------------------------------------------------------ DPP reduction

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over aligned groups of LPR lanes (LPR in 4..64).  The full sum is valid
// in the last lane of each group.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<0xB1>(v);                          // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);                          // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) v += dpp<0x141>(v);  // row_half_mirror
    if constexpr (LPR >= 16) v += dpp<0x140>(v); // row_mirror
    if constexpr (LPR >= 32) v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
    if constexpr (LPR >= 64) v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
    return v;
}

// --------------------------------------------------- per-format chunk decode
//
// Chunk<F>::Meta holds what a lane needs from the meta plane for one (row,
// chunk); load() fetches it; codes(v, w) turns code dword v into the raw code
// values of its CPC/4 columns (column order); apply() folds the per-group
// partial sums P (sum of code * x) and the column sums X into the row sum.

template <int F> struct Chunk;

template <> struct Chunk<QG_Q8_0> {
    static constexpr int CPD = 4, SUBS = 1;
    struct Meta { uint32_t d; };
    __device__ static Meta load(const uint8_t* meta_row, int cg) {
        return {*(const uint16_t*)(meta_row + 2 * (cg >> 1))};
    }
    __device__ static void codes(uint32_t v, float* w) {
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = (float)(int)(int8_t)(v >> (8 * k));
    }
    __device__ static float apply(const Meta& m, const float* P, const float*) { return h2f(m.d) * P[0]; }
};

template <> struct Chunk<QG_Q4_0> {
    static constexpr int CPD = 8, SUBS = 1;
    struct Meta { uint32_t d; };
    __device__ static Meta load(const uint8_t* meta_row, int cg) { return {*(const uint16_t*)(meta_row + 2 * cg)}; }
    __device__ static void codes(uint32_t v, float* w) {
        const uint32_t lo = opaque(v & 0x0F0F0F0Fu), hi = opaque((v >> 4) & 0x0F0F0F0Fu);
#pragma unroll
        for (int k = 0; k < 4; ++k) { w[2 * k] = ubyte(lo, k); w[2 * k + 1] = ubyte(hi, k); }
    }
    // w = (n - 8) d  ->  d * (sum n x - 8 X)
    __device__ static float apply(const Meta& m, const float* P, const float* X) {
        return h2f(m.d) * fmaf(-8.0f, X[0], P[0]);
    }
};

template <> struct Chunk<QG_Q4_1> {
    static constexpr int CPD = 8, SUBS = 1;
    struct Meta { uint32_t dm; };
    __device__ static Meta load(const uint8_t* meta_row, int cg) { return {*(const uint32_t*)(meta_row + 4 * cg)}; }
    __device__ static void codes(uint32_t v, float* w) { Chunk<QG_Q4_0>::codes(v, w); }
    // w = n d + m  ->  d * sum n x + m X
    __device__ static float apply(const Meta& m, const float* P, const float* X) {
        return fmaf(h2f(m.dm & 0xFFFFu), P[0], h2f(m.dm >> 16) * X[0]);
    }
};

// K-quant meta entry (16 B per 256 weights): bytes 0..11 hold pairs
// p_j = s_j | t_j << 6 at bits [12j, 12j+12); bytes 12..15 hold fp16 d, dmin.
// A lane fetches the two dwords around its pair at a lane-specific offset and
// extracts the pair with one funnel shift; it never reads past the entry.
template <> struct Chunk<QG_Q4_K> {
    static constexpr int CPD = 8, SUBS = 1;
    struct Meta { uint32_t lo, hi, dd; int sh; };
    __device__ static Meta load(const uint8_t* meta_row, int cg) {
        const uint8_t* e = meta_row + 16 * (cg >> 3);
        const int j = cg & 7;
        const int w = (12 * j) >> 5;  // 0,0,0,1,1,1,2,2
        Meta m;
        m.lo = *(const uint32_t*)(e + 4 * w);
        m.hi = *(const uint32_t*)(e + 4 * w + 4);
        m.dd = *(const uint32_t*)(e + 12);
        m.sh = 12 * j - 32 * w;
        return m;
    }
    __device__ static void codes(uint32_t v, float* w) { Chunk<QG_Q4_0>::codes(v, w); }
    // w = n s d - t dmin  ->  d * (s * sum n x) - dmin * (t * X)
    __device__ static float apply(const Meta& m, const float* P, const float* X) {
        const uint32_t p = __builtin_amdgcn_alignbit(m.hi, m.lo, m.sh);
        const float s = (float)(p & 63u), t = (float)((p >> 6) & 63u);
        return fmaf(h2f(m.dd & 0xFFFFu), s * P[0], -h2f(m.dd >> 16) * (t * X[0]));
    }
};

// Q2_K: a 16-byte chunk is 64 weights = sub-blocks 2q and 2q+1 of its
// super-block (q = chunk & 3); their two pairs are 24 contiguous bits.
template <> struct Chunk<QG_Q2_K> {
    static constexpr int CPD = 16, SUBS = 2;
    struct Meta { uint32_t lo, hi, dd; int sh; };
    __device__ static Meta load(const uint8_t* meta_row, int cg) {
        const uint8_t* e = meta_row + 16 * (cg >> 2);
        const int q = cg & 3;
        const int w = (24 * q) >> 5;  // 0,0,1,2
        Meta m;
        m.lo = *(const uint32_t*)(e + 4 * w);
        m.hi = *(const uint32_t*)(e + 4 * w + 4);
        m.dd = *(const uint32_t*)(e + 12);
        m.sh = 24 * q - 32 * w;
        return m;
    }
    __device__ static void codes(uint32_t v, float* w) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t f = opaque((v >> (2 * s)) & 0x03030303u);
#pragma unroll
            for (int k = 0; k < 4; ++k) w[4 * k + s] = ubyte(f, k);
        }
    }
    __device__ static float apply(const Meta& m, const float* P, const float* X) {
        const uint32_t p = __builtin_amdgcn_alignbit(m.hi, m.lo, m.sh);
        const float s0 = (float)(p & 63u), t0 = (float)((p >> 6) & 63u);
        const float s1 = (float)((p >> 12) & 63u), t1 = (float)((p >> 18) & 63u);
        const float sp = fmaf(s0, P[0], s1 * P[1]);
        const float tx = fmaf(t0, X[0], t1 * X[1]);
        return fmaf(h2f(m.dd & 0xFFFFu), sp, -h2f(m.dd >> 16) * tx);
    }
};

// ternary: f = t + 1 in {0,1,2}; w = (f - 1) d -> d * (sum f x - X)
template <> struct Chunk<QG_TERN> {
    static constexpr int CPD = 16, SUBS = 1;
    struct Meta { uint32_t d; };
    __device__ static Meta load(const uint8_t* meta_row, int cg) { return {*(const uint16_t*)(meta_row + 2 * (cg >> 1))}; }
    __device__ static void codes(uint32_t v, float* w) { Chunk<QG_Q2_K>::codes(v, w); }
    __device__ static float apply(const Meta& m, const float* P, const float* X) { return h2f(m.d) * (P[0] - X[0]); }
};

// 1-bit: w = (2 beta - 1) d -> d * (2 sum_{beta=1} x - X)
template <> struct Chunk<QG_BIN> {
    static constexpr int CPD = 32, SUBS = 1;
    struct Meta { uint32_t d; };
    __device__ static Meta load(const uint8_t* meta_row, int cg) { return {*(const uint16_t*)(meta_row + 2 * cg)}; }
    __device__ static void codes(uint32_t v, float* w) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint32_t f = opaque((v >> s) & 0x01010101u);
#pragma unroll
            for (int k = 0; k < 4; ++k) w[8 * k + s] = ubyte(f, k);
        }
    }
    __device__ static float apply(const Meta& m, const float* P, const float* X) {
        return h2f(m.d) * fmaf(2.0f, P[0], -X[0]);
    }
};

// ------------------------------------------------------------ GEMV kernel

template <int F, int B, int R, int LPR>
__global__ void __launch_bounds__(kThreads)
gemv_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
            const float* __restrict__ x, float* __restrict__ y, int N, int K, int KS) {
    using T = Fmt<F>;
    using C = Chunk<F>;
    constexpr int CPC = T::CPC, CPD = C::CPD, GS = T::GS;
    constexpr int GPW = 64 / LPR;                 // lane groups per wave
    constexpr int XS_PER_CHUNK = GS ? CPC / GS : 1;  // column sums per chunk
    extern __shared__ float lds[];
    float* xs = lds;                    // [B][KS]
    float* xsum = lds + B * KS;         // [B][KS / GS]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = lane / LPR, sl = lane % LPR;
    const int row0 = ((blockIdx.x * kWaves + wave) * GPW + grp) * R;

    const size_t code_row = (size_t)(K / T::BLOCK) * T::CB;
    const size_t meta_row = (size_t)(K / T::BLOCK) * T::MB;
    const uint8_t* crow[R];
    const uint8_t* mrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);
        crow[r] = codes + (size_t)row * code_row;
        mrow[r] = meta + (size_t)row * meta_row;
    }

    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += KS) {
        const int ks = min(KS, K - k0);
        if (k0) __syncthreads();  // the previous slice is fully consumed
        for (int i = 4 * tid; i < B * ks; i += 4 * kThreads) {
            const int b = i / ks, c = i - b * ks;
            *(float4*)(xs + b * KS + c) = *(const float4*)(x + (size_t)b * K + k0 + c);
        }
        __syncthreads();
        if constexpr (GS > 0) {
            for (int g = tid; g < B * (ks / GS); g += kThreads) {
                const int b = g / (ks / GS), c = g - b * (ks / GS);
                const float* p = xs + b * KS + c * GS;
                float s = 0.0f;
                for (int i = 0; i < GS; i += 4) {
                    const float4 v = *(const float4*)(p + i);
                    s += (v.x + v.y) + (v.z + v.w);
                }
                xsum[b * (KS / GS) + c] = s;
            }
            __syncthreads();
        }

        const int nch = ks / CPC;
        const int c0 = k0 / CPC;
        for (int c = sl; c < nch; c += LPR) {
            const int cg = c0 + c;
            uint4 q[R];
            typename C::Meta m[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                q[r] = *(const uint4*)(crow[r] + 16 * (size_t)cg);
                m[r] = C::load(mrow[r], cg);
            }
            float P[R][B][C::SUBS];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b)
#pragma unroll
                    for (int s = 0; s < C::SUBS; ++s) P[r][b][s] = 0.0f;

#pragma unroll
            for (int d = 0; d < 4; ++d) {
                float xv[B][CPD];
#pragma unroll
                for (int b = 0; b < B; ++b)
#pragma unroll
                    for (int i = 0; i < CPD; i += 4) {
                        const float4 v = *(const float4*)(xs + b * KS + c * CPC + d * CPD + i);
                        xv[b][i] = v.x; xv[b][i + 1] = v.y; xv[b][i + 2] = v.z; xv[b][i + 3] = v.w;
                    }
                constexpr int DPS = 4 / C::SUBS;  // code dwords per scale group
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t v = d == 0 ? q[r].x : d == 1 ? q[r].y : d == 2 ? q[r].z : q[r].w;
                    float w[CPD];
                    C::codes(v, w);
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        float p = P[r][b][d / DPS];
#pragma unroll
                        for (int i = 0; i < CPD; ++i) p = fmaf(w[i], xv[b][i], p);
                        P[r][b][d / DPS] = p;
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float X[XS_PER_CHUNK > 0 ? XS_PER_CHUNK : 1];
                if constexpr (GS > 0) {
#pragma unroll
                    for (int s = 0; s < XS_PER_CHUNK; ++s) X[s] = xsum[b * (KS / GS) + c * XS_PER_CHUNK + s];
                } else {
                    X[0] = 0.0f;
                }
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r][b] += C::apply(m[r], P[r][b], X);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float v = group_sum<LPR>(acc[r][b]);
            if (sl == LPR - 1 && row0 + r < N) y[(size_t)b * N + row0 + r] = v;
        }
}

// ---------------------------------------------------------- dequant kernel
// One thread per 16-byte code chunk: decode CPC weights exactly.

template <int F>
__global__ void __launch_bounds__(kThreads)
dequant_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
               float* __restrict__ out, int N, int K) {
    using T = Fmt<F>;
    using C = Chunk<F>;
    constexpr int CPC = T::CPC, CPD = C::CPD;
    const int nch = K / CPC;
    const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (id >= (int64_t)N * nch) return;
    const int row = (int)(id / nch), cg = (int)(id - (int64_t)row * nch);
    const uint8_t* crow = codes + (size_t)row * (K / T::BLOCK) * T::CB;
    const uint8_t* mrow = meta + (size_t)row * (K / T::BLOCK) * T::MB;
    const uint4 q = *(const uint4*)(crow + 16 * (size_t)cg);
    float* o = out + (size_t)row * K + (size_t)cg * CPC;
    const uint32_t dw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        float w[CPD];
        C::codes(dw[d], w);
        float sc, off;  // weight = code * sc + off, exactly as the formats define it
        if constexpr (F == QG_Q8_0 || F == QG_Q4_0 || F == QG_TERN || F == QG_BIN) {
            const float dd = h2f(C::load(mrow, cg).d);
            sc = dd;
            off = 0.0f;
            if constexpr (F == QG_Q4_0) {
#pragma unroll
                for (int i = 0; i < CPD; ++i) w[i] -= 8.0f;
            } else if constexpr (F == QG_TERN) {
#pragma unroll
                for (int i = 0; i < CPD; ++i) w[i] -= 1.0f;
            } else if constexpr (F == QG_BIN) {
#pragma unroll
                for (int i = 0; i < CPD; ++i) w[i] = 2.0f * w[i] - 1.0f;
            }
        } else if constexpr (F == QG_Q4_1) {
            const uint32_t dm = C::load(mrow, cg).dm;
            sc = h2f(dm & 0xFFFFu);
            off = h2f(dm >> 16);
        } else {  // K-quants
            const auto m = C::load(mrow, cg);
            const uint32_t p = __builtin_amdgcn_alignbit(m.hi, m.lo, m.sh);
            const int sub = F == QG_Q2_K ? (d >> 1) : 0;
            const uint32_t pj = p >> (12 * sub);
            sc = (float)(pj & 63u) * h2f(m.dd & 0xFFFFu);
            off = -((float)((pj >> 6) & 63u) * h2f(m.dd >> 16));
        }
        constexpr bool has_offset = F == QG_Q4_1 || F == QG_Q4_K || F == QG_Q2_K;
#pragma unroll
        for (int i = 0; i < CPD; ++i) {
            // the product is exact in fp32, so fma and mul-then-add round
            // identically; formats without an offset take the bare product
            // (adding +0 would turn a -0 product into +0)
            o[d * CPD + i] = has_offset ? fmaf(w[i], sc, off) : w[i] * sc;
        }
    }
}

// ---------------------------------------------------------------- launchers

int pick_lpr(int nch) {
    if (nch >= 64) return 64;
    if (nch >= 32) return 32;
    if (nch >= 16) return 16;
    return 8;
}

template <int F, int B, int R, int LPR>
hipError_t launch_gemv_lpr(const uint8_t* codes, const uint8_t* meta, const float* x, float* y,
                           int N, int K, int KS, hipStream_t st) {
    constexpr int rows_per_wg = kWaves * (64 / LPR) * R;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    constexpr int GS = Fmt<F>::GS;
    const size_t lds = (size_t)B * KS * 4 + (GS ? (size_t)B * (KS / GS) * 4 : 0);
    hipLaunchKernelGGL((gemv_kernel<F, B, R, LPR>), dim3(grid), dim3(kThreads), lds, st,
                       codes, meta, x, y, N, K, KS);
    return hipGetLastError();
}

template <int F, int B>
hipError_t launch_gemv_b(const uint8_t* codes, const uint8_t* meta, const float* x, float* y,
                         int N, int K, hipStream_t st) {
    // K slice staged per pass: the whole K when x and its sums fit the LDS
    // budget, else the largest multiple of 256 columns that does
    constexpr int GS = Fmt<F>::GS;
    auto bytes = [](int ks) { return (size_t)B * ks * 4 + (GS ? (size_t)B * (ks / GS) * 4 : 0); };
    int KS = K;
    if (bytes(KS) > (size_t)kLdsBudget) {
        KS = 256;
        while (bytes(KS + 256) <= (size_t)kLdsBudget) KS += 256;
    }
    constexpr int R = B == 1 ? 4 : (B <= 4 ? 2 : 1);
    const int lpr = pick_lpr(KS / Fmt<F>::CPC);
    switch (lpr) {
        case 64: return launch_gemv_lpr<F, B, R, 64>(codes, meta, x, y, N, K, KS, st);
        case 32: return launch_gemv_lpr<F, B, R, 32>(codes, meta, x, y, N, K, KS, st);
        case 16: return launch_gemv_lpr<F, B, R, 16>(codes, meta, x, y, N, K, KS, st);
        default: return launch_gemv_lpr<F, B, R, 8>(codes, meta, x, y, N, K, KS, st);
    }
}

template <int F>
hipError_t launch_gemv_f(const uint8_t* codes, const uint8_t* meta, const float* x, float* y,
                         int N, int K, int B, hipStream_t st) {
    switch (B) {
        case 1: return launch_gemv_b<F, 1>(codes, meta, x, y, N, K, st);
        case 2: return launch_gemv_b<F, 2>(codes, meta, x, y, N, K, st);
        case 3: return launch_gemv_b<F, 3>(codes, meta, x, y, N, K, st);
        case 4: return launch_gemv_b<F, 4>(codes, meta, x, y, N, K, st);
        case 5: return launch_gemv_b<F, 5>(codes, meta, x, y, N, K, st);
        case 6: return launch_gemv_b<F, 6>(codes, meta, x, y, N, K, st);
        case 7: return launch_gemv_b<F, 7>(codes, meta, x, y, N, K, st);
        default: return launch_gemv_b<F, 8>(codes, meta, x, y, N, K, st);
    }
}

hipError_t launch_gemv(int fmt, const uint8_t* codes, const uint8_t* meta, const float* x, float* y,
                       int N, int K, int B, hipStream_t st) {
    switch (fmt) {
        case QG_Q8_0: return launch_gemv_f<QG_Q8_0>(codes, meta, x, y, N, K, B, st);
        case QG_Q4_0: return launch_gemv_f<QG_Q4_0>(codes, meta, x, y, N, K, B, st);
        case QG_Q4_1: return launch_gemv_f<QG_Q4_1>(codes, meta, x, y, N, K, B, st);
        case QG_Q4_K: return launch_gemv_f<QG_Q4_K>(codes, meta, x, y, N, K, B, st);
        case QG_Q2_K: return launch_gemv_f<QG_Q2_K>(codes, meta, x, y, N, K, B, st);
        case QG_TERN: return launch_gemv_f<QG_TERN>(codes, meta, x, y, N, K, B, st);
        default: return launch_gemv_f<QG_BIN>(codes, meta, x, y, N, K, B, st);
    }
}

template <int F>
hipError_t launch_dequant_f(const uint8_t* codes, const uint8_t* meta, float* out, int N, int K, hipStream_t st) {
    const int64_t n = (int64_t)N * (K / Fmt<F>::CPC);
    const int64_t grid = (n + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((dequant_kernel<F>), dim3((unsigned)grid), dim3(kThreads), 0, st, codes, meta, out, N, K);
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, const uint8_t* codes, const uint8_t* meta, float* out, int N, int K, hipStream_t st) {
    switch (fmt) {
        case QG_Q8_0: return launch_dequant_f<QG_Q8_0>(codes, meta, out, N, K, st);
        case QG_Q4_0: return launch_dequant_f<QG_Q4_0>(codes, meta, out, N, K, st);
        case QG_Q4_1: return launch_dequant_f<QG_Q4_1>(codes, meta, out, N, K, st);
        case QG_Q4_K: return launch_dequant_f<QG_Q4_K>(codes, meta, out, N, K, st);
        case QG_Q2_K: return launch_dequant_f<QG_Q2_K>(codes, meta, out, N, K, st);
        case QG_TERN: return launch_dequant_f<QG_TERN>(codes, meta, out, N, K, st);
        default: return launch_dequant_f<QG_BIN>(codes, meta, out, N, K, st);
    }
}

int check_gemv_args(int fmt, const void* w, const float* x, const float* y, int64_t N, int64_t K, int B,
                    void* ws, size_t ws_bytes) {
    int rc = check_matrix(fmt, N, K);
    if (rc) return rc;
    if (!w || !x || !y) return fail(QG_EINVAL, "null w, x or y");
    if (B < 1 || B > QG_MAX_BATCH) return fail(QG_ERANGE, "B=%d must be in [1, %d]", B, QG_MAX_BATCH);
    if (!aligned(w, 16)) return fail(QG_EALIGN, "w must be 16-byte aligned");
    if (!aligned(x, 16)) return fail(QG_EALIGN, "x must be 16-byte aligned");
    if (!aligned(y, 4)) return fail(QG_EALIGN, "y must be 4-byte aligned");
    (void)ws;
    (void)ws_bytes;
    return QG_OK;
}

}  // namespace
}  // namespace qg

using namespace qg;

extern "C" {

size_t qgemv_workspace_size(int fmt, int64_t N, int64_t K, int B) {
    (void)fmt; (void)N; (void)K; (void)B;
    return 0;
}

int qgemv(int fmt, const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
          void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    int rc = check_gemv_args(fmt, w, x, y, N, K, B, ws, ws_bytes);
    if (rc) return rc;
    const uint8_t* codes = static_cast<const uint8_t*>(w);
    const uint8_t* meta = codes + qg_codes_plane_size(fmt, N, K);
    hipError_t e = launch_gemv(fmt, codes, meta, x, y, (int)N, (int)K, B, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QG_EHIP, "GEMV launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

#define QG_GEMV_ALIAS(name, F)                                                                      \
    int name(const void* w, const float* x, float* y, int64_t N, int64_t K, int B, void* ws,        \
             size_t ws_bytes, void* stream) {                                                       \
        return qgemv(F, w, x, y, N, K, B, ws, ws_bytes, stream);                                    \
    }
QG_GEMV_ALIAS(qgemv_q8_0, QG_Q8_0)
QG_GEMV_ALIAS(qgemv_q4_0, QG_Q4_0)
QG_GEMV_ALIAS(qgemv_q4_1, QG_Q4_1)
QG_GEMV_ALIAS(qgemv_q4k, QG_Q4_K)
QG_GEMV_ALIAS(qgemv_q2k, QG_Q2_K)
QG_GEMV_ALIAS(qgemv_tern, QG_TERN)
QG_GEMV_ALIAS(qgemv_bin, QG_BIN)
#undef QG_GEMV_ALIAS

int qg_dequant(int fmt, const void* w, float* out, int64_t N, int64_t K, void* stream) {
    clear_error();
    int rc = check_matrix(fmt, N, K);
    if (rc) return rc;
    if (!w || !out) return fail(QG_EINVAL, "null w or out");
    if (!aligned(w, 16)) return fail(QG_EALIGN, "w must be 16-byte aligned");
    if (!aligned(out, 4)) return fail(QG_EALIGN, "out must be 4-byte aligned");
    const uint8_t* codes = static_cast<const uint8_t*>(w);
    const uint8_t* meta = codes + qg_codes_plane_size(fmt, N, K);
    hipError_t e = launch_dequant(fmt, codes, meta, out, (int)N, (int)K, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QG_EHIP, "dequant launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // extern "C"
