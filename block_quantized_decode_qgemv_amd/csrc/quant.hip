// Device quantizer and re-quantizer for gfx950.
//
// The same quantizers as the host reference quantizer (handbook page,
// section "GGUF 的量化格式": per-32 Q8_0 / Q4_0 / Q4_1 and the two-level
// K-quant; Q2_K is that construction with 2-bit codes), run on weights that
// are already in HBM, and written straight into the packed two-plane,
// 16-row-interleaved layout.  The Flash-MoE page runs 2-bit experts made
// from its 4-bit ones by an offline re-quantization step (sections
// "性能表现" and "项目结构"); qrequant does that on the device: decode the
// source format, then quantize to the target one.
//
// One thread per (row, block).  Every step follows the host quantizer's
// order of operations with IEEE fp32 division and no contraction, so the
// bytes equal the host quantizer's.  Errors found on the device (a
// non-finite weight, a scale that overflows fp16) are reported through a
// caller-provided status word.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "internal.h"

#pragma clang fp contract(off)

namespace qg {
namespace {

// fp32 -> fp16 bits: round to nearest even, subnormals kept, overflow -> inf.
__device__ uint16_t to_f16(float f) {
    const uint32_t x = __float_as_uint(f);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7FFFFFFFu;
    if (ax >= 0x7F800000u) return (uint16_t)(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
    if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // >= 65520 rounds to inf
    const uint32_t e32 = ax >> 23;
    if (e32 >= 113) {  // normal fp16
        uint32_t h = ((e32 - 112) << 10) | ((ax & 0x7FFFFFu) >> 13);
        const uint32_t rem = ax & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
        return (uint16_t)(sign | h);
    }
    if (e32 < 102) return (uint16_t)sign;  // below 2^-25: rounds to zero
    const uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;
    const uint32_t shift = 126 - e32;  // 14 .. 24
    uint32_t h = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (h & 1u))) ++h;
    return (uint16_t)(sign | h);
}

// fp16 bits -> fp32 (exact; the hardware conversion keeps subnormals)
__device__ float from_f16(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// A scale or min through fp16 storage; false when it overflows.
__device__ bool store_f16(float v, uint16_t* bits, float* stored) {
    *bits = to_f16(v);
    if ((*bits & 0x7C00u) == 0x7C00u) return false;
    *stored = from_f16(*bits);
    return true;
}

__device__ float clampf(float v, float lo, float hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Byte position of byte j of row n in a plane of rb bytes per row, rows
// interleaved by 16 (16-byte unit u of the group's rows contiguous, unit
// after unit, then each row's short last unit, row after row).
__device__ size_t plane_pos(int64_t n, int64_t N, size_t rb, size_t j) {
    const int64_t g = n / 16;
    const int r = (int)(n % 16);
    const int n_g = (int)(N - 16 * g < 16 ? N - 16 * g : 16);
    const size_t units = rb / 16;
    const size_t base = (size_t)(16 * g) * rb;
    if (j < units * 16) return base + ((j / 16) * n_g + r) * 16 + j % 16;
    return base + units * n_g * 16 + (size_t)r * (rb % 16) + (j - units * 16);
}

// Writes `len` bytes (a multiple of 16 or a divisor of 16, at j aligned to
// min(len, 16)) so that no write straddles a 16-byte unit.
__device__ void put_bytes(uint8_t* plane, int64_t n, int64_t N, size_t rb, size_t j, const uint8_t* src, int len) {
    for (int o = 0; o < len; ++o) plane[plane_pos(n, N, rb, j + o)] = src[o];
}

__device__ void report(int* status, int code) { atomicMin(status, code); }

// The block's weights, read from global memory (cached) each time they are
// needed, with -0 turned into +0; no per-thread copy of the block.
struct Src {
    const float* p;
    __device__ float operator[](int k) const { return p[k] + 0.0f; }
};

template <int F> struct DevQuant;

template <> struct DevQuant<QG_Q8_0> {
    static constexpr int BLOCK = 32, CB = 32, MB = 2;
    __device__ static bool run(Src v, uint8_t* cb, uint8_t* mb) {
        float a = 0.0f;
        for (int i = 0; i < 32; ++i) { const float m = fabsf(v[i]); if (m > a) a = m; }
        uint16_t dbits; float d;
        if (!store_f16(a / 127.0f, &dbits, &d)) return false;
        mb[0] = (uint8_t)(dbits & 0xFF); mb[1] = (uint8_t)(dbits >> 8);
        for (int i = 0; i < 32; ++i) {
            const float q = d == 0.0f ? 0.0f : clampf(rintf(v[i] / d), -127.0f, 127.0f);
            cb[i] = (uint8_t)(int8_t)q;
        }
        return true;
    }
};

template <> struct DevQuant<QG_Q4_0> {
    static constexpr int BLOCK = 32, CB = 16, MB = 2;
    __device__ static bool run(Src v, uint8_t* cb, uint8_t* mb) {
        int j = 0;
        for (int i = 1; i < 32; ++i) if (fabsf(v[i]) > fabsf(v[j])) j = i;
        uint16_t dbits; float d;
        if (!store_f16(v[j] / -8.0f, &dbits, &d)) return false;
        mb[0] = (uint8_t)(dbits & 0xFF); mb[1] = (uint8_t)(dbits >> 8);
        for (int i = 0; i < 32; i += 2) {
            const float c0 = d == 0.0f ? 0.0f : clampf(rintf(v[i] / d), -8.0f, 7.0f);
            const float c1 = d == 0.0f ? 0.0f : clampf(rintf(v[i + 1] / d), -8.0f, 7.0f);
            cb[i / 2] = (uint8_t)(((int)c0 + 8) | (((int)c1 + 8) << 4));
        }
        return true;
    }
};

template <> struct DevQuant<QG_Q4_1> {
    static constexpr int BLOCK = 32, CB = 16, MB = 4;
    __device__ static bool run(Src v, uint8_t* cb, uint8_t* mb) {
        float lo = v[0], hi = v[0];
        for (int i = 1; i < 32; ++i) { if (v[i] < lo) lo = v[i]; if (v[i] > hi) hi = v[i]; }
        uint16_t dbits, mbits; float d, m;
        if (!store_f16((hi - lo) / 15.0f, &dbits, &d)) return false;
        if (!store_f16(lo, &mbits, &m)) return false;
        mb[0] = (uint8_t)(dbits & 0xFF); mb[1] = (uint8_t)(dbits >> 8);
        mb[2] = (uint8_t)(mbits & 0xFF); mb[3] = (uint8_t)(mbits >> 8);
        for (int i = 0; i < 32; i += 2) {
            const float n0 = d == 0.0f ? 0.0f : clampf(rintf((v[i] - m) / d), 0.0f, 15.0f);
            const float n1 = d == 0.0f ? 0.0f : clampf(rintf((v[i + 1] - m) / d), 0.0f, 15.0f);
            cb[i / 2] = (uint8_t)((int)n0 | ((int)n1 << 4));
        }
        return true;
    }
};

// Two-level K-quant over a 256-weight super-block, codes in [0, QMAX].
template <int QMAX> struct DevKQuant {
    static constexpr int BLOCK = 256, BITS = QMAX == 15 ? 4 : 2, PER_BYTE = 8 / BITS;
    static constexpr int CB = 256 / PER_BYTE, MB = 16;
    __device__ static bool run(Src v, uint8_t* cb, uint8_t* mb) {
        float sc[8], mn[8];
        float scmax = 0.0f, mnmax = 0.0f;
        for (int j = 0; j < 8; ++j) {
            float lo = v[32 * j], hi = v[32 * j];
            for (int i = 1; i < 32; ++i) {
                const float x = v[32 * j + i];
                if (x < lo) lo = x;
                if (x > hi) hi = x;
            }
            if (!(lo < 0.0f)) lo = 0.0f;  // min clamped to <= 0
            sc[j] = (hi - lo) / (float)QMAX;
            mn[j] = -lo;
            if (j == 0 || sc[j] > scmax) scmax = sc[j];
            if (j == 0 || mn[j] > mnmax) mnmax = mn[j];
        }
        uint16_t dbits, dmbits; float D, M;
        if (!store_f16(scmax / 63.0f, &dbits, &D)) return false;
        if (!store_f16(mnmax / 63.0f, &dmbits, &M)) return false;
        uint32_t s[8], t[8];
        float S[8], Mn[8];
        for (int j = 0; j < 8; ++j) {
            s[j] = D == 0.0f ? 1u : (uint32_t)clampf(rintf(sc[j] / D), 1.0f, 63.0f);
            t[j] = M == 0.0f ? 0u : (uint32_t)clampf(rintf(mn[j] / M), 0.0f, 63.0f);
            S[j] = (float)s[j] * D;
            Mn[j] = (float)t[j] * M;
        }
        for (int m = 0; m < 4; ++m) {
            const uint32_t v24 = (s[2 * m] | (t[2 * m] << 6)) | ((s[2 * m + 1] | (t[2 * m + 1] << 6)) << 12);
            mb[3 * m] = (uint8_t)(v24 & 0xFF);
            mb[3 * m + 1] = (uint8_t)((v24 >> 8) & 0xFF);
            mb[3 * m + 2] = (uint8_t)((v24 >> 16) & 0xFF);
        }
        mb[12] = (uint8_t)(dbits & 0xFF); mb[13] = (uint8_t)(dbits >> 8);
        mb[14] = (uint8_t)(dmbits & 0xFF); mb[15] = (uint8_t)(dmbits >> 8);
        for (int i = 0; i < CB; ++i) cb[i] = 0;
        for (int i = 0; i < 256; ++i) {
            const int j = i / 32;
            const float q = S[j] == 0.0f ? 0.0f : clampf(rintf((v[i] + Mn[j]) / S[j]), 0.0f, (float)QMAX);
            cb[i / PER_BYTE] |= (uint8_t)((uint32_t)q << (BITS * (i % PER_BYTE)));
        }
        return true;
    }
};
template <> struct DevQuant<QG_Q4_K> : DevKQuant<15> {};
template <> struct DevQuant<QG_Q2_K> : DevKQuant<3> {};

// One thread per (row, block), grid-stride over N * K / BLOCK blocks.
template <int F>
__global__ void __launch_bounds__(256)
quant_kernel(const float* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ out, int* __restrict__ status) {
    using Q = DevQuant<F>;
    const int64_t nb = K / Q::BLOCK;
    const size_t row_codes = (size_t)nb * Q::CB, row_meta = (size_t)nb * Q::MB;
    uint8_t* codes = out;
    uint8_t* meta = out + (size_t)N * row_codes;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < N * nb;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = i / nb, b = i % nb;
        const Src v{w + n * K + b * Q::BLOCK};
        bool finite = true;
        for (int k = 0; k < Q::BLOCK; ++k) finite = finite && isfinite(v.p[k]);
        if (!finite) {
            report(status, QG_EINVAL);
            continue;
        }
        uint8_t cb[Q::CB], mb[Q::MB];
        if (!Q::run(v, cb, mb)) {
            report(status, QG_ERANGE);
            continue;
        }
        put_bytes(codes, n, N, row_codes, (size_t)b * Q::CB, cb, Q::CB);
        put_bytes(meta, n, N, row_meta, (size_t)b * Q::MB, mb, Q::MB);
    }
}

__global__ void clear_status_kernel(int* status) { *status = QG_OK; }

template <int F>
hipError_t launch_quant_f(const float* w, int64_t N, int64_t K, uint8_t* out, int* status, hipStream_t st) {
    const int64_t items = N * (K / DevQuant<F>::BLOCK);
    const int64_t want = (items + 255) / 256;
    const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL((quant_kernel<F>), dim3(grid), dim3(256), 0, st, w, N, K, out, status);
    return hipGetLastError();
}

hipError_t launch_quant(int fmt, const float* w, int64_t N, int64_t K, uint8_t* out, int* status, hipStream_t st) {
    hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, st, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (fmt) {
        case QG_Q8_0: return launch_quant_f<QG_Q8_0>(w, N, K, out, status, st);
        case QG_Q4_0: return launch_quant_f<QG_Q4_0>(w, N, K, out, status, st);
        case QG_Q4_1: return launch_quant_f<QG_Q4_1>(w, N, K, out, status, st);
        case QG_Q4_K: return launch_quant_f<QG_Q4_K>(w, N, K, out, status, st);
        default: return launch_quant_f<QG_Q2_K>(w, N, K, out, status, st);
    }
}

int check_quant(int fmt, int64_t N, int64_t K, const void* out, const int* status) {
    if (fmt == QG_TERN || fmt == QG_BIN || fmt == QG_BIN8 || fmt == QG_TERN3)
        return fail(QG_EUNSUPPORTED, "format %d has no quantizer (it packs given codes)", fmt);
    int rc = check_matrix(fmt, N, K);
    if (rc) return rc;
    if (!out || !status) return fail(QG_EINVAL, "null out or status");
    if (!aligned(out, 16)) return fail(QG_EALIGN, "out must be 16-byte aligned");
    if (!aligned(status, 4)) return fail(QG_EALIGN, "status must be 4-byte aligned");
    return QG_OK;
}

}  // namespace
}  // namespace qg

using namespace qg;

extern "C" {

int qquant_device(int fmt, const float* w, int64_t N, int64_t K, void* out, int* status, void* stream) {
    clear_error();
    int rc = check_quant(fmt, N, K, out, status);
    if (rc) return rc;
    if (!w) return fail(QG_EINVAL, "null w");
    if (!aligned(w, 4)) return fail(QG_EALIGN, "w must be 4-byte aligned");
    const size_t ob = qg_packed_size(fmt, N, K), wb = (size_t)N * (size_t)K * 4;
    if (overlap(out, ob, w, wb) || overlap(status, 4, w, wb) || overlap(status, 4, out, ob))
        return fail(QG_EINVAL, "w, out and status must not overlap");
    hipError_t e = launch_quant(fmt, w, N, K, static_cast<uint8_t*>(out), status, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QG_EHIP, "quantizer launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

size_t qrequant_workspace_size(int64_t N, int64_t K) {
    if (N < 1 || K < 1 || N >= (int64_t)1 << 31 || K > (int64_t)1 << 30) return 0;
    return (size_t)N * (size_t)K * sizeof(float);
}

int qrequant(int src_fmt, const void* src, int dst_fmt, void* dst, int64_t N, int64_t K, void* workspace,
             size_t ws_bytes, int* status, void* stream) {
    clear_error();
    int rc = check_quant(dst_fmt, N, K, dst, status);
    if (rc) return rc;
    rc = check_matrix(src_fmt, N, K);
    if (rc) return rc;
    if (!src || !workspace) return fail(QG_EINVAL, "null src or workspace");
    if (!aligned(src, 16) || !aligned(workspace, 16)) return fail(QG_EALIGN, "src and workspace must be 16-byte aligned");
    const size_t need = qrequant_workspace_size(N, K);
    if (ws_bytes < need) return fail(QG_ERANGE, "workspace of %zu bytes is below the %zu needed", ws_bytes, need);
    const uint8_t* s = static_cast<const uint8_t*>(src);
    const uint8_t* d = static_cast<const uint8_t*>(dst);
    const size_t src_bytes = qg_packed_size(src_fmt, N, K), dst_bytes = qg_packed_size(dst_fmt, N, K);
    const uint8_t* t = static_cast<const uint8_t*>(workspace);
    if (overlap(s, src_bytes, d, dst_bytes) || overlap(t, need, d, dst_bytes) || overlap(t, need, s, src_bytes) ||
        overlap(status, 4, d, dst_bytes) || overlap(status, 4, t, need))
        return fail(QG_EINVAL, "src, dst, workspace and status must not overlap");
    float* tmp = static_cast<float*>(workspace);
    rc = qg_dequant(src_fmt, src, tmp, N, K, stream);
    if (rc) return rc;
    hipError_t e = launch_quant(dst_fmt, tmp, N, K, static_cast<uint8_t*>(dst), status, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QG_EHIP, "quantizer launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // extern "C"
