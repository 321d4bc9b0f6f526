// Block-quantized decode GEMV and dequant kernels for gfx950 (CDNA4).
//
// The operation is the handbook page's decode step ("端侧推理：llama.cpp 与
// GGUF、MLX、ExecuTorch", section "速度上限：带宽 ÷ 权重字节数"): every weight
// row is read once and dotted with the activation vector, y = W x, batch B
// stacking activation rows.  Block formats: section "GGUF 的量化格式" of the
// same page, plus Q2_K, ternary-in-2-bit and 1-bit from the low-bit README
// page's kernel table.
//
// Memory layout (see qgemv.h): rows are interleaved in groups of 16; in each
// group, 16-byte unit u of every row is contiguous.  This is the low-bit
// README page's row repack for dot-product lanes, sized to a gfx950 DPP row:
// 16 lanes own the 16 rows of a group, so one quarter-wave load reads 256
// contiguous bytes and the 16 lanes that share x columns can exchange x.
//
// Kernel (batch <= 8 is not a matrix-core contraction; everything is fp32
// VALU work): gemv_dpp_kernel (GemvDpp, gemv_core.h), one workgroup per
// 16-row group, W waves of four 16-lane parts of KCS code units each.  Each
// part's x columns live in the lanes' registers and every multiply-add reads
// its x operand from the owning lane with a DPP broadcast, so x never goes
// through LDS.  Fewer units per part at the larger batches keep x within 32
// registers per lane; the waves per workgroup follow the row length and how
// many workgroups a compute unit holds at that register count.
//   * codes are decoded in registers (masks put one code per byte and
//     v_cvt_pk_f32_fp8 turns two bytes into exact floats n * 2^-9, the 2^9
//     folded into the scale) and accumulate in fp32: the Flash-MoE page's
//     fma(nibble, scale*x, bias*x) rearrangement ("FMA 优化的反量化内核") with
//     the bias term hoisted over the shared x as bias * sum(x); K-quant scales
//     are applied once per super-block;
//   * the parts of a row are combined in a fixed order, so results repeat
//     bit for bit.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "gemv_core.h"
#include "gemv_dispatch.h"
#include "gemv_splitk.h"
#include "internal.h"

namespace qg {
namespace {

using namespace core;

template <int F, int B, int W, int KCS>
__global__ void __launch_bounds__(W * 64)
gemv_dpp_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
                const float* __restrict__ x, float* __restrict__ y, int N, int K) {
    const int g = blockIdx.x;
    GemvDpp<F, B, W, KCS>::run(
        codes, meta, N, K, g, [&](int b) { return x + (size_t)b * K; }, B,
        [&](auto sums, int n_g, int tid) {
            for (int t = tid; t < kRowGroup * B; t += W * 64)
                if (t / B < n_g) y[(size_t)(t % B) * N + g * kRowGroup + t / B] = sums(t);
        });
}

// ---------------------------------------------------------- dequant kernel
// One thread per (row, code unit): decode CPC weights exactly.

__device__ __forceinline__ uint32_t meta_u16(const uint8_t* gm, int n_g, int r, int o, int row_meta) {
    const int full = row_meta >> 4, rem = row_meta & 15;
    const int u = o >> 4, i = o & 15;
    const uint8_t* p = u < full ? gm + ((size_t)u * n_g + r) * 16 + i
                                : gm + (size_t)full * n_g * 16 + (size_t)r * rem + i;
    return *(const uint16_t*)p;
}

template <int F>
__global__ void __launch_bounds__(256)
dequant_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
               float* __restrict__ out, int N, int K) {
    using T = Fmt<F>;
    constexpr int CPC = T::CPC, CPD = CPC / 4;
    const int nb = K / T::BLOCK;
    const int row_codes = nb * T::CB, row_meta = nb * T::MB;
    const int nch = row_codes >> 4;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= (int64_t)N * nch) return;
    const int row = (int)(id / nch), c = (int)(id - (int64_t)row * nch);
    const int g = row / kRowGroup, r = row - g * kRowGroup;
    const int n_g = min(kRowGroup, N - g * kRowGroup);
    const uint8_t* gc = codes + (size_t)g * kRowGroup * row_codes;
    const uint8_t* gm = meta + (size_t)g * kRowGroup * row_meta;
    const uint4 q = *(const uint4*)(gc + ((size_t)c * n_g + r) * 16);
    const uint32_t dw[4] = {q.x, q.y, q.z, q.w};
    float d8 = 0.0f;  // bin8: this unit's block scale, base + step * c
    if constexpr (F == QG_BIN8) {
        const int full = row_meta >> 4, rem = row_meta & 15;
        const int u = c >> 4, i = c & 15;
        const uint8_t* pm = u < full ? gm + ((size_t)u * n_g + r) * 16 + i
                                     : gm + (size_t)full * n_g * 16 + (size_t)r * rem + i;
        const size_t span = ((size_t)N * row_meta + 15) / 16 * 16;
        const float2 ab = *(const float2*)(meta + span + (size_t)row * 8);
        d8 = bin8_scale(ab.x, ab.y, *pm);
    }
    float* o = out + (size_t)row * K + (size_t)c * CPC;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        float w[CPD];
        Unit<F>::decode(dw[d], w);
        if constexpr (F != QG_Q8_0) {
#pragma unroll
            for (int i = 0; i < CPD; ++i) w[i] *= 512.0f;  // exact: back to integer codes
        }
#pragma unroll
        for (int i = 0; i < CPD; ++i) {
            const int col = c * CPC + d * CPD + i;
            const int blk = col / T::BLOCK;
            float v;
            if constexpr (F == QG_Q8_0) {
                v = w[i] * h2f(meta_u16(gm, n_g, r, 2 * blk, row_meta));
            } else if constexpr (F == QG_Q4_0) {
                v = (w[i] - 8.0f) * h2f(meta_u16(gm, n_g, r, 2 * blk, row_meta));
            } else if constexpr (F == QG_Q4_1) {
                // n*d is exact, so fma and multiply-then-add round identically
                v = fmaf(w[i], h2f(meta_u16(gm, n_g, r, 4 * blk, row_meta)),
                         h2f(meta_u16(gm, n_g, r, 4 * blk + 2, row_meta)));
            } else if constexpr (F == QG_Q4_K || F == QG_Q2_K) {
                const int j = (col / 32) & 7;
                const int bit = 12 * j;
                const uint32_t two = meta_u16(gm, n_g, r, 16 * blk + (bit >> 3), row_meta);
                const uint32_t pj = (two >> (bit & 7)) & 0xFFFu;
                const float dd = h2f(meta_u16(gm, n_g, r, 16 * blk + 12, row_meta));
                const float dm = h2f(meta_u16(gm, n_g, r, 16 * blk + 14, row_meta));
                v = fmaf(w[i], (float)(pj & 63u) * dd, -((float)(pj >> 6) * dm));
            } else if constexpr (F == QG_TERN) {
                v = (w[i] - 1.0f) * h2f(meta_u16(gm, n_g, r, 2 * blk, row_meta));
            } else if constexpr (F == QG_BIN8) {
                v = (2.0f * w[i] - 1.0f) * d8;
            } else {
                v = (2.0f * w[i] - 1.0f) * h2f(meta_u16(gm, n_g, r, 2 * blk, row_meta));
            }
            o[d * CPD + i] = v;
        }
    }
}

// tern3: one thread per (row, 64-weight group): its three code dwords, its
// scale and its block's tail field.
__global__ void __launch_bounds__(256)
dequant_tern3_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
                     float* __restrict__ out, int N, int K) {
    const int ng = K / 64;                        // groups per row
    const int row_codes = 12 * ng, row_meta = 3 * ng;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= (int64_t)N * ng) return;
    const int row = (int)(id / ng), c = (int)(id - (int64_t)row * ng);
    const int g = row / kRowGroup, r = row - g * kRowGroup;
    const int n_g = min(kRowGroup, N - g * kRowGroup);
    const uint8_t* gc = codes + (size_t)g * kRowGroup * row_codes;
    const uint8_t* gm = meta + (size_t)g * kRowGroup * row_meta;
    const int blk = c >> 2, s = c & 3;
    const float d = h2f(meta_u16(gm, n_g, r, 12 * blk + 2 * s, row_meta));
    const uint32_t field = meta_u16(gm, n_g, r, 12 * blk + 8, row_meta) |
                           (meta_u16(gm, n_g, r, 12 * blk + 10, row_meta) << 16);
    float* o = out + (size_t)row * K + (size_t)c * 64;
#pragma unroll
    for (int e = 0; e < 3; ++e) {
        const int off = 12 * c + 4 * e;  // never crosses a 16-byte unit; code rows have no short unit
        const uint32_t v = *(const uint32_t*)(gc + ((size_t)(off >> 4) * n_g + r) * 16 + (off & 15));
        float w[20];
        tern3_digits(v, w);
#pragma unroll
        for (int i = 0; i < 20; ++i) o[20 * e + i] = (512.0f * w[i] - 1.0f) * d;  // exact: back to f - 1
    }
    float w[4];
    tern3_tail(field, s, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[60 + i] = (512.0f * w[i] - 1.0f) * d;
}

// ---------------------------------------------------------------- launchers

}  // namespace

int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) {
            (void)hipGetLastError();
            c = 256;
        }
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

namespace {

// The plain GEMV as a kernel set for the shared dispatch.
template <int F, int B, int W, int KCS>
struct PlainGemv {
    static hipError_t launch(dim3 grid, dim3 block, hipStream_t st, const uint8_t* codes, const uint8_t* meta,
                             const float* x, float* y, int N, int K) {
        hipLaunchKernelGGL((gemv_dpp_kernel<F, B, W, KCS>), grid, block, 0, st, codes, meta, x, y, N, K);
        return hipGetLastError();
    }
    static int resident() { return resident_blocks(gemv_dpp_kernel<F, B, W, KCS>, W * 64); }
};

template <int F>
hipError_t launch_dequant_f(const uint8_t* codes, const uint8_t* meta, float* out, int N, int K, hipStream_t st) {
    const int64_t n = (int64_t)N * (K / Fmt<F>::CPC);
    const int64_t grid = (n + 255) / 256;
    hipLaunchKernelGGL((dequant_kernel<F>), dim3((unsigned)grid), dim3(256), 0, st, codes, meta, out, N, K);
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
        case QG_BIN8: return launch_dequant_f<QG_BIN8>(codes, meta, out, N, K, st);
        case QG_TERN3: {
            const int64_t n = (int64_t)N * (K / 64);
            hipLaunchKernelGGL(dequant_tern3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, codes,
                               meta, out, N, K);
            return hipGetLastError();
        }
        default: return launch_dequant_f<QG_BIN>(codes, meta, out, N, K, st);
    }
}

constexpr int64_t kMaxGemvK = (int64_t)1 << 26;

// K splits for a GEMV: 4 or 2 when the row groups times the splits still fit
// the compute units (so the split grid fills at most the chip once) and K
// splits into whole 256-column pieces, from batch 5 up; else 1.  Measured on
// Q4_K (both launches): 1024 x 4096 at batch 8 6.4 against 8.1 us single
// pass, at batch 5 5.6 against 6.0, at batch 3 5.9 against 5.2 (a loss);
// 1024 x 14336 at batch 8 11.1 against 24.4; at batch 1, and at 4096 rows,
// splitting gains less than the second launch costs.
int splitk_parts(int64_t N, int64_t K, int B) {
    if (B < 5) return 1;
    const int64_t groups = (N + kRowGroup - 1) / kRowGroup;
    const int cus = device_cus();
    for (int S : {4, 2})
        if (K % (256 * S) == 0 && groups * S <= cus) return S;
    return 1;
}

}  // namespace

int check_gemv_args(int fmt, const void* w, const float* x, const float* y, int64_t N, int64_t K, int B) {
    int rc = check_matrix(fmt, N, K);
    if (rc) return rc;
    if (!w || !x || !y) return fail(QG_EINVAL, "null w, x or y");
    if (B < 1 || B > QG_MAX_BATCH) return fail(QG_ERANGE, "B=%d must be in [1, %d]", B, QG_MAX_BATCH);
    // offsets inside a 16-row group are 32-bit
    if (K > kMaxGemvK) return fail(QG_ESHAPE, "K=%lld exceeds the GEMV limit %lld", (long long)K, (long long)kMaxGemvK);
    if (!aligned(w, 16)) return fail(QG_EALIGN, "w must be 16-byte aligned");
    if (!aligned(x, 16)) return fail(QG_EALIGN, "x must be 16-byte aligned");
    if (!aligned(y, 4)) return fail(QG_EALIGN, "y must be 4-byte aligned");
    // every workgroup reads all of x and writes its own rows of y: no overlap
    const size_t yb = (size_t)B * N * 4, xb = (size_t)B * K * 4, wb = qg_packed_size(fmt, N, K);
    if (overlap(y, yb, x, xb) || overlap(y, yb, w, wb)) return fail(QG_EINVAL, "y must not overlap x or w");
    return QG_OK;
}

}  // namespace qg

using namespace qg;

extern "C" {

size_t qgemv_workspace_size(int fmt, int64_t N, int64_t K, int B) {
    if (!format_info(fmt) || N < 1 || N >= ((int64_t)1 << 31) || K < 1 || K > kMaxGemvK || B < 1 || B > QG_MAX_BATCH ||
        qg_packed_size(fmt, N, K) == 0)
        return 0;
    const int S = splitk_parts(N, K, B);
    return S > 1 ? (size_t)S * B * N * 4 : 0;
}

int qgemv(int fmt, const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
          void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    int rc = check_gemv_args(fmt, w, x, y, N, K, B);
    if (rc) return rc;
    const uint8_t* codes = static_cast<const uint8_t*>(w);
    const uint8_t* meta = codes + qg_codes_plane_size(fmt, N, K);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int S = splitk_parts(N, K, B);
    const size_t need = S > 1 ? (size_t)S * B * N * 4 : 0;
    hipError_t e;
    if (need > 0 && ws && ws_bytes >= need) {
        if (!aligned(ws, 16)) return fail(QG_EALIGN, "ws must be 16-byte aligned");
        const size_t yb = (size_t)B * N * 4, xb = (size_t)B * K * 4, wb = qg_packed_size(fmt, N, K);
        if (overlap(ws, need, x, xb) || overlap(ws, need, y, yb) || overlap(ws, need, w, wb))
            return fail(QG_EINVAL, "ws must not overlap w, x or y");
        e = launch_gemv_splitk(fmt, (int)N, (int)K, B, S, st, codes, meta, x, static_cast<float*>(ws), y);
    } else {
        // no workspace (or too small): the single-pass kernel
        e = core::launch_dpp<PlainGemv>(fmt, (int)N, (int)K, B, st, codes, meta, x, y, (int)N, (int)K);
    }
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
QG_GEMV_ALIAS(qgemv_tern3, QG_TERN3)
QG_GEMV_ALIAS(qgemv_bin, QG_BIN)
QG_GEMV_ALIAS(qgemv_bin8, QG_BIN8)
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
