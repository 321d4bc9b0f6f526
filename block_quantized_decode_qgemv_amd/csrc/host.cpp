// Host half of libqgemv.so: sizes, errors, argument checks, and the reference
// quantizer / packers.
//
// The quantizers restate the handbook page "端侧推理：llama.cpp 与 GGUF、MLX、
// ExecuTorch", section "GGUF 的量化格式" (Q8_0, Q4_0, Q4_1 and the simplified
// two-level Q4_K), with every scale and min stored as fp16 and the codes
// computed against the stored values; Q2_K is the same K-quant construction
// with 2-bit codes.  All arithmetic is IEEE fp32 in the order written
// (compiled with -ffp-contract=off), rounding is half-to-even, and a zero
// divisor yields the zero code.  Byte layout as documented in qgemv.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <thread>
#include <vector>

#include "internal.h"

namespace qg {

namespace {

const FormatInfo kFormats[] = {
    {32, 32, 2},    // Q8_0
    {32, 16, 2},    // Q4_0
    {32, 16, 4},    // Q4_1
    {256, 128, 16}, // Q4_K
    {256, 64, 16},  // Q2_K
    {128, 32, 2},   // TERN
    {128, 16, 2},   // BIN
    {128, 16, 1},   // BIN8 (plus the per-row plane, see qg_packed_size)
    {256, 48, 12},  // TERN3: four 64-weight scale groups per block
};

thread_local char g_last_error[512] = "";

// fp32 -> fp16 bits, round to nearest even, subnormals kept, overflow -> inf.
uint16_t f32_to_f16(float f) {
    uint32_t x;
    std::memcpy(&x, &f, 4);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7FFFFFFFu;
    if (ax >= 0x7F800000u) return (uint16_t)(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
    if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // >= 65520 rounds to inf
    const uint32_t e32 = ax >> 23;
    if (e32 >= 113) {  // normal fp16 (>= 2^-14)
        uint32_t h = ((e32 - 112) << 10) | ((ax & 0x7FFFFFu) >> 13);
        const uint32_t rem = ax & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
        return (uint16_t)(sign | h);
    }
    if (e32 < 102) return (uint16_t)sign;  // below 2^-25: rounds to zero
    const uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;
    const uint32_t shift = 126 - e32;  // 14 .. 24: value / 2^-24 = mant >> shift
    uint32_t h = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (h & 1u))) ++h;
    return (uint16_t)(sign | h);
}

float f16_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 0x1Fu;
    const uint32_t m = h & 0x3FFu;
    uint32_t x;
    if (e == 0) {
        if (m == 0) {
            x = sign;
        } else {  // subnormal: normalise
            int sh = 0;
            uint32_t mm = m;
            while (!(mm & 0x400u)) { mm <<= 1; ++sh; }
            x = sign | ((uint32_t)(113 - sh) << 23) | ((mm & 0x3FFu) << 13);
        }
    } else if (e == 31) {
        x = sign | 0x7F800000u | (m << 13);
    } else {
        x = sign | ((e + 112) << 23) | (m << 13);
    }
    float f;
    std::memcpy(&f, &x, 4);
    return f;
}

float clampf(float v, float lo, float hi) { return v < lo ? lo : (v > hi ? hi : v); }

// One scale/min through fp16 storage; false when it overflows.
bool store_f16(float v, uint16_t* bits, float* stored) {
    *bits = f32_to_f16(v);
    if ((*bits & 0x7C00u) == 0x7C00u) return false;
    *stored = f16_to_f32(*bits);
    return true;
}

void put_u16(uint8_t* p, uint16_t v) {
    p[0] = (uint8_t)(v & 0xFF);
    p[1] = (uint8_t)(v >> 8);
}

// Per-row quantizers.  `w` is one row of K canonical (finite, no -0) values;
// `codes` and `meta` point at the row's slice of each plane.
int quant_row_q8_0(const float* w, int64_t K, uint8_t* codes, uint8_t* meta) {
    for (int64_t b = 0; b < K / 32; ++b) {
        const float* v = w + 32 * b;
        float a = 0.0f;
        for (int i = 0; i < 32; ++i) { const float m = std::fabs(v[i]); if (m > a) a = m; }
        uint16_t dbits; float d;
        if (!store_f16(a / 127.0f, &dbits, &d)) return QG_ERANGE;
        put_u16(meta + 2 * b, dbits);
        for (int i = 0; i < 32; ++i) {
            const float q = d == 0.0f ? 0.0f : clampf(std::nearbyint(v[i] / d), -127.0f, 127.0f);
            codes[32 * b + i] = (uint8_t)(int8_t)q;
        }
    }
    return QG_OK;
}

int quant_row_q4_0(const float* w, int64_t K, uint8_t* codes, uint8_t* meta) {
    for (int64_t b = 0; b < K / 32; ++b) {
        const float* v = w + 32 * b;
        int j = 0;
        for (int i = 1; i < 32; ++i) if (std::fabs(v[i]) > std::fabs(v[j])) j = i;
        uint16_t dbits; float d;
        if (!store_f16(v[j] / -8.0f, &dbits, &d)) return QG_ERANGE;
        put_u16(meta + 2 * b, dbits);
        for (int i = 0; i < 32; i += 2) {
            const float c0 = d == 0.0f ? 0.0f : clampf(std::nearbyint(v[i] / d), -8.0f, 7.0f);
            const float c1 = d == 0.0f ? 0.0f : clampf(std::nearbyint(v[i + 1] / d), -8.0f, 7.0f);
            codes[16 * b + i / 2] = (uint8_t)(((int)c0 + 8) | (((int)c1 + 8) << 4));
        }
    }
    return QG_OK;
}

int quant_row_q4_1(const float* w, int64_t K, uint8_t* codes, uint8_t* meta) {
    for (int64_t b = 0; b < K / 32; ++b) {
        const float* v = w + 32 * b;
        float lo = v[0], hi = v[0];
        for (int i = 1; i < 32; ++i) { if (v[i] < lo) lo = v[i]; if (v[i] > hi) hi = v[i]; }
        uint16_t dbits, mbits; float d, m;
        if (!store_f16((hi - lo) / 15.0f, &dbits, &d)) return QG_ERANGE;
        if (!store_f16(lo, &mbits, &m)) return QG_ERANGE;
        put_u16(meta + 4 * b, dbits);
        put_u16(meta + 4 * b + 2, mbits);
        for (int i = 0; i < 32; i += 2) {
            const float n0 = d == 0.0f ? 0.0f : clampf(std::nearbyint((v[i] - m) / d), 0.0f, 15.0f);
            const float n1 = d == 0.0f ? 0.0f : clampf(std::nearbyint((v[i + 1] - m) / d), 0.0f, 15.0f);
            codes[16 * b + i / 2] = (uint8_t)((int)n0 | ((int)n1 << 4));
        }
    }
    return QG_OK;
}

// Two-level K-quant, weight codes in [0, qmax] (15 for Q4_K, 3 for Q2_K).
int quant_row_kquant(const float* w, int64_t K, uint8_t* codes, uint8_t* meta, int qmax) {
    const int code_bits = qmax == 15 ? 4 : 2;
    const int per_byte = 8 / code_bits;
    for (int64_t sb = 0; sb < K / 256; ++sb) {
        const float* v = w + 256 * sb;
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
            sc[j] = (hi - lo) / (float)qmax;
            mn[j] = -lo;
            if (j == 0 || sc[j] > scmax) scmax = sc[j];
            if (j == 0 || mn[j] > mnmax) mnmax = mn[j];
        }
        uint16_t dbits, dmbits; float D, M;
        if (!store_f16(scmax / 63.0f, &dbits, &D)) return QG_ERANGE;
        if (!store_f16(mnmax / 63.0f, &dmbits, &M)) return QG_ERANGE;
        uint32_t s[8], t[8];
        float S[8], Mn[8];
        for (int j = 0; j < 8; ++j) {
            s[j] = D == 0.0f ? 1u : (uint32_t)clampf(std::nearbyint(sc[j] / D), 1.0f, 63.0f);
            t[j] = M == 0.0f ? 0u : (uint32_t)clampf(std::nearbyint(mn[j] / M), 0.0f, 63.0f);
            S[j] = (float)s[j] * D;
            Mn[j] = (float)t[j] * M;
        }
        uint8_t* mb = meta + 16 * sb;
        for (int m = 0; m < 4; ++m) {
            const uint32_t pa = s[2 * m] | (t[2 * m] << 6);
            const uint32_t pb = s[2 * m + 1] | (t[2 * m + 1] << 6);
            const uint32_t v24 = pa | (pb << 12);
            mb[3 * m] = (uint8_t)(v24 & 0xFF);
            mb[3 * m + 1] = (uint8_t)((v24 >> 8) & 0xFF);
            mb[3 * m + 2] = (uint8_t)((v24 >> 16) & 0xFF);
        }
        put_u16(mb + 12, dbits);
        put_u16(mb + 14, dmbits);
        uint8_t* cb = codes + (256 / per_byte) * sb;
        std::memset(cb, 0, 256 / per_byte);
        for (int i = 0; i < 256; ++i) {
            const int j = i / 32;
            const float q = S[j] == 0.0f ? 0.0f
                                         : clampf(std::nearbyint((v[i] + Mn[j]) / S[j]), 0.0f, (float)qmax);
            cb[i / per_byte] |= (uint8_t)((uint32_t)q << (code_bits * (i % per_byte)));
        }
    }
    return QG_OK;
}

// Row-major bytes of one row group (n_g rows of rb bytes) -> the 16-row
// interleaved order: 16-byte unit u of every row contiguous, unit after unit,
// then each row's short last unit (rb % 16 bytes), row after row.
void interleave_group(const uint8_t* rows, int n_g, size_t rb, uint8_t* dst) {
    const size_t units = rb / 16, rem = rb % 16;
    for (size_t u = 0; u < units; ++u)
        for (int r = 0; r < n_g; ++r) std::memcpy(dst + (u * n_g + r) * 16, rows + r * rb + u * 16, 16);
    uint8_t* tail = dst + units * n_g * 16;
    for (int r = 0; r < n_g; ++r) std::memcpy(tail + r * rem, rows + r * rb + units * 16, rem);
}

int quant_row(int fmt, const float* w, int64_t K, uint8_t* codes, uint8_t* meta) {
    switch (fmt) {
        case QG_Q8_0: return quant_row_q8_0(w, K, codes, meta);
        case QG_Q4_0: return quant_row_q4_0(w, K, codes, meta);
        case QG_Q4_1: return quant_row_q4_1(w, K, codes, meta);
        case QG_Q4_K: return quant_row_kquant(w, K, codes, meta, 15);
        case QG_Q2_K: return quant_row_kquant(w, K, codes, meta, 3);
        default: return QG_EINVAL;
    }
}

// Codes are validated before anything is written (the packers' error
// contract): the index of the first value of v[0 .. n) outside [lo, hi], or -1.
template <typename T>
int64_t first_out_of_range(const T* v, int64_t n, int lo, int hi) {
    for (int64_t i = 0; i < n; ++i)
        if ((int)v[i] < lo || (int)v[i] > hi) return i;
    return -1;
}

}  // namespace

const FormatInfo* format_info(int fmt) {
    if (fmt < QG_Q8_0 || fmt > QG_TERN3) return nullptr;
    return &kFormats[fmt];
}

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_last_error[0] = '\0'; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return na > 0 && nb > 0 && pa < pb + nb && pb < pa + na;
}

int check_matrix(int fmt, int64_t N, int64_t K) {
    const FormatInfo* fi = format_info(fmt);
    if (!fi) return fail(QG_EINVAL, "unknown format %d", fmt);
    if (N < 1) return fail(QG_ESHAPE, "N=%lld must be >= 1", (long long)N);
    if (K < fi->block || K % fi->block)
        return fail(QG_ESHAPE, "K=%lld is not a positive multiple of the block size %d", (long long)K, fi->block);
    if (N >= (int64_t)1 << 31 || K > (int64_t)1 << 30)  // kernels take N and K as int
        return fail(QG_ESHAPE, "N=%lld, K=%lld exceed the supported range (N < 2^31, K <= 2^30)", (long long)N,
                    (long long)K);
    return QG_OK;
}

}  // namespace qg

using namespace qg;

extern "C" {

size_t qg_packed_size(int fmt, int64_t N, int64_t K) {
    const FormatInfo* fi = format_info(fmt);
    if (!fi || N < 1 || K < fi->block || K % fi->block) return 0;
    const size_t meta = (size_t)N * (size_t)(K / fi->block) * (size_t)fi->meta_bytes;
    if (fmt == QG_BIN8)  // meta padded to 16, then (base, step) per row
        return qg_codes_plane_size(fmt, N, K) + (meta + 15) / 16 * 16 + (size_t)N * 8;
    return qg_codes_plane_size(fmt, N, K) + meta;
}

size_t qg_codes_plane_size(int fmt, int64_t N, int64_t K) {
    const FormatInfo* fi = format_info(fmt);
    if (!fi || N < 1 || K < fi->block || K % fi->block) return 0;
    return (size_t)N * (size_t)(K / fi->block) * (size_t)fi->code_bytes;
}

size_t qg_codes_plane_offset(int fmt, int64_t N, int64_t K) { return qg_codes_plane_size(fmt, N, K); }

int qg_block_size(int fmt) {
    const FormatInfo* fi = format_info(fmt);
    return fi ? fi->block : 0;
}

const char* qg_strerror(int code) {
    switch (code) {
        case QG_OK: return "ok";
        case QG_EINVAL: return "invalid argument";
        case QG_ESHAPE: return "invalid shape";
        case QG_EALIGN: return "misaligned pointer";
        case QG_ERANGE: return "value out of range";
        case QG_EHIP: return "HIP runtime error";
        case QG_EUNSUPPORTED: return "unsupported";
        default: return "unknown error";
    }
}

const char* qg_last_error(void) { return g_last_error; }

const char* qg_version(void) { return "qgemv 0.1 (gfx950)"; }

int qquant(int fmt, const float* w_host, int64_t N, int64_t K, void* out_host, int n_threads) {
    clear_error();
    if (fmt == QG_TERN || fmt == QG_BIN || fmt == QG_BIN8 || fmt == QG_TERN3)
        return fail(QG_EINVAL, "format %d packs given codes: use qpack_tern / qpack_bin / qpack_bin8 / qpack_tern3",
                    fmt);
    int rc = check_matrix(fmt, N, K);
    if (rc) return rc;
    if (!w_host || !out_host) return fail(QG_EINVAL, "null pointer");
    const FormatInfo* fi = format_info(fmt);
    const size_t row_codes = (size_t)(K / fi->block) * fi->code_bytes;
    const size_t row_meta = (size_t)(K / fi->block) * fi->meta_bytes;
    uint8_t* codes = static_cast<uint8_t*>(out_host);
    uint8_t* meta = codes + (size_t)N * row_codes;
    if (n_threads < 1) n_threads = 1;

    const int64_t groups = (N + 15) / 16;
    if ((int64_t)n_threads > groups) n_threads = (int)groups;
    std::vector<int> status(n_threads, QG_OK);
    std::vector<int64_t> bad_row(n_threads, -1);
    auto work = [&](int tid) {
        std::vector<float> row((size_t)K);
        std::vector<uint8_t> gc(16 * row_codes), gm(16 * row_meta);
        for (int64_t g = tid; g < groups; g += n_threads) {
            const int n_g = (int)std::min<int64_t>(16, N - 16 * g);
            for (int i = 0; i < n_g; ++i) {
                const int64_t r = 16 * g + i;
                const float* src = w_host + (size_t)r * K;
                for (int64_t k = 0; k < K; ++k) {
                    if (!std::isfinite(src[k])) { status[tid] = QG_EINVAL; bad_row[tid] = r; return; }
                    row[k] = src[k] + 0.0f;  // -0 -> +0
                }
                const int s = quant_row(fmt, row.data(), K, gc.data() + i * row_codes, gm.data() + i * row_meta);
                if (s != QG_OK) { status[tid] = s; bad_row[tid] = r; return; }
            }
            interleave_group(gc.data(), n_g, row_codes, codes + (size_t)(16 * g) * row_codes);
            interleave_group(gm.data(), n_g, row_meta, meta + (size_t)(16 * g) * row_meta);
        }
    };
    if (n_threads == 1) {
        work(0);
    } else {
        std::vector<std::thread> pool;
        for (int t = 0; t < n_threads; ++t) pool.emplace_back(work, t);
        for (auto& th : pool) th.join();
    }
    for (int t = 0; t < n_threads; ++t) {
        if (status[t] == QG_EINVAL) return fail(QG_EINVAL, "non-finite weight in row %lld", (long long)bad_row[t]);
        if (status[t] != QG_OK)
            return fail(status[t], "a scale or min of row %lld overflows fp16", (long long)bad_row[t]);
    }
    return QG_OK;
}

int qpack_tern(const int8_t* t, const uint16_t* scale_f16, int64_t N, int64_t K, void* out_host) {
    clear_error();
    int rc = check_matrix(QG_TERN, N, K);
    if (rc) return rc;
    if (!t || !scale_f16 || !out_host) return fail(QG_EINVAL, "null pointer");
    if (const int64_t i = first_out_of_range(t, N * K, -1, 1); i >= 0)
        return fail(QG_EINVAL, "ternary code %d at (%lld, %lld)", t[i], (long long)(i / K), (long long)(i % K));
    const size_t row_codes = (size_t)K / 4, row_meta = (size_t)(K / 128) * 2;
    uint8_t* codes = static_cast<uint8_t*>(out_host);
    uint8_t* meta = codes + (size_t)N * row_codes;
    std::vector<uint8_t> gc(16 * row_codes), gm(16 * row_meta);
    for (int64_t g = 0; g < (N + 15) / 16; ++g) {
        const int n_g = (int)std::min<int64_t>(16, N - 16 * g);
        for (int i = 0; i < n_g; ++i) {
            const int64_t r = 16 * g + i;
            for (int64_t k = 0; k < K; k += 4) {
                uint8_t byte = 0;
                for (int j = 0; j < 4; ++j) {
                    const int v = t[(size_t)r * K + k + j];  // validated above
                    byte |= (uint8_t)((v + 1) << (2 * j));
                }
                gc[i * row_codes + k / 4] = byte;
            }
            for (int64_t b = 0; b < K / 128; ++b) put_u16(gm.data() + i * row_meta + 2 * b, scale_f16[(size_t)r * (K / 128) + b]);
        }
        interleave_group(gc.data(), n_g, row_codes, codes + (size_t)(16 * g) * row_codes);
        interleave_group(gm.data(), n_g, row_meta, meta + (size_t)(16 * g) * row_meta);
    }
    return QG_OK;
}

int qpack_tern3(const int8_t* t, const uint16_t* scale_f16, int64_t N, int64_t K, void* out_host) {
    clear_error();
    int rc = check_matrix(QG_TERN3, N, K);
    if (rc) return rc;
    if (!t || !scale_f16 || !out_host) return fail(QG_EINVAL, "null pointer");
    if (const int64_t i = first_out_of_range(t, N * K, -1, 1); i >= 0)
        return fail(QG_EINVAL, "ternary code %d at (%lld, %lld)", t[i], (long long)(i / K), (long long)(i % K));
    const int64_t nb = K / 256;
    const size_t row_codes = (size_t)nb * 48, row_meta = (size_t)nb * 12;
    uint8_t* codes = static_cast<uint8_t*>(out_host);
    uint8_t* meta = codes + (size_t)N * row_codes;
    std::vector<uint8_t> gc(16 * row_codes), gm(16 * row_meta);
    for (int64_t g = 0; g < (N + 15) / 16; ++g) {
        const int n_g = (int)std::min<int64_t>(16, N - 16 * g);
        for (int i = 0; i < n_g; ++i) {
            const int64_t r = 16 * g + i;
            const int8_t* tr = t + (size_t)r * K;
            for (int64_t b = 0; b < nb; ++b) {
                uint8_t* cb = gc.data() + i * row_codes + 48 * b;
                uint8_t* mb = gm.data() + i * row_meta + 12 * b;
                uint32_t field = 0;
                for (int s = 0; s < 4; ++s) {
                    const int8_t* ts = tr + 256 * b + 64 * s;  // one 64-weight scale group
                    // byte m: the base-3 digits of columns 5m .. 5m + 4 (column 5m + l has weight 3^l)
                    for (int m = 0; m < 12; ++m) {
                        unsigned v = 0;
                        for (int l = 4; l >= 0; --l) v = 3 * v + (unsigned)(ts[5 * m + l] + 1);
                        cb[12 * s + m] = (uint8_t)v;
                    }
                    // columns 60..63: 2-bit fields, field byte l at bits 2s
                    for (int l = 0; l < 4; ++l) field |= (uint32_t)(ts[60 + l] + 1) << (8 * l + 2 * s);
                    put_u16(mb + 2 * s, scale_f16[(size_t)r * (K / 64) + 4 * b + s]);
                }
                for (int l = 0; l < 4; ++l) mb[8 + l] = (uint8_t)(field >> (8 * l));
            }
        }
        interleave_group(gc.data(), n_g, row_codes, codes + (size_t)(16 * g) * row_codes);
        interleave_group(gm.data(), n_g, row_meta, meta + (size_t)(16 * g) * row_meta);
    }
    return QG_OK;
}

int qpack_bin(const uint8_t* bits, const uint16_t* scale_f16, int64_t N, int64_t K, void* out_host) {
    clear_error();
    int rc = check_matrix(QG_BIN, N, K);
    if (rc) return rc;
    if (!bits || !scale_f16 || !out_host) return fail(QG_EINVAL, "null pointer");
    if (const int64_t i = first_out_of_range(bits, N * K, 0, 1); i >= 0)
        return fail(QG_EINVAL, "1-bit code %u at (%lld, %lld)", bits[i], (long long)(i / K), (long long)(i % K));
    const size_t row_codes = (size_t)K / 8, row_meta = (size_t)(K / 128) * 2;
    uint8_t* codes = static_cast<uint8_t*>(out_host);
    uint8_t* meta = codes + (size_t)N * row_codes;
    std::vector<uint8_t> gc(16 * row_codes), gm(16 * row_meta);
    for (int64_t g = 0; g < (N + 15) / 16; ++g) {
        const int n_g = (int)std::min<int64_t>(16, N - 16 * g);
        for (int i = 0; i < n_g; ++i) {
            const int64_t r = 16 * g + i;
            for (int64_t k = 0; k < K; k += 8) {
                uint8_t byte = 0;
                for (int j = 0; j < 8; ++j) {
                    const unsigned v = bits[(size_t)r * K + k + j];  // validated above
                    byte |= (uint8_t)(v << j);
                }
                gc[i * row_codes + k / 8] = byte;
            }
            for (int64_t b = 0; b < K / 128; ++b) put_u16(gm.data() + i * row_meta + 2 * b, scale_f16[(size_t)r * (K / 128) + b]);
        }
        interleave_group(gc.data(), n_g, row_codes, codes + (size_t)(16 * g) * row_codes);
        interleave_group(gm.data(), n_g, row_meta, meta + (size_t)(16 * g) * row_meta);
    }
    return QG_OK;
}

int qpack_bin8(const uint8_t* bits, const uint16_t* scale_f16, int64_t N, int64_t K, void* out_host) {
    clear_error();
    int rc = check_matrix(QG_BIN8, N, K);
    if (rc) return rc;
    if (!bits || !scale_f16 || !out_host) return fail(QG_EINVAL, "null pointer");
    if (const int64_t i = first_out_of_range(bits, N * K, 0, 1); i >= 0)
        return fail(QG_EINVAL, "1-bit code %u at (%lld, %lld)", bits[i], (long long)(i / K), (long long)(i % K));
    for (int64_t i = 0; i < N * (K / 128); ++i)
        if (!std::isfinite(f16_to_f32(scale_f16[i])))
            return fail(QG_EINVAL, "non-finite scale in row %lld", (long long)(i / (K / 128)));
    const int64_t nb = K / 128;
    const size_t row_codes = (size_t)K / 8, row_meta = (size_t)nb;
    uint8_t* codes = static_cast<uint8_t*>(out_host);
    uint8_t* meta = codes + (size_t)N * row_codes;
    const size_t meta_span = ((size_t)N * row_meta + 15) / 16 * 16;
    uint8_t* pairs = meta + meta_span;
    std::memset(meta + (size_t)N * row_meta, 0, meta_span - (size_t)N * row_meta);
    std::vector<uint8_t> gc(16 * row_codes), gm(16 * row_meta);
    std::vector<float> d((size_t)nb);
    for (int64_t g = 0; g < (N + 15) / 16; ++g) {
        const int n_g = (int)std::min<int64_t>(16, N - 16 * g);
        for (int i = 0; i < n_g; ++i) {
            const int64_t r = 16 * g + i;
            for (int64_t k = 0; k < K; k += 8) {
                uint8_t byte = 0;
                for (int j = 0; j < 8; ++j) {
                    const unsigned v = bits[(size_t)r * K + k + j];  // validated above
                    byte |= (uint8_t)(v << j);
                }
                gc[i * row_codes + k / 8] = byte;
            }
            // the row's block scales as 8-bit codes of base + step * c
            float lo = 0.0f, hi = 0.0f;
            for (int64_t b = 0; b < nb; ++b) {
                d[b] = f16_to_f32(scale_f16[(size_t)r * nb + b]);  // finite: validated above
                if (b == 0 || d[b] < lo) lo = d[b];
                if (b == 0 || d[b] > hi) hi = d[b];
            }
            const float step = (hi - lo) / 255.0f;
            for (int64_t b = 0; b < nb; ++b)
                gm[i * row_meta + b] =
                    step == 0.0f ? 0 : (uint8_t)clampf(std::nearbyint((d[b] - lo) / step), 0.0f, 255.0f);
            std::memcpy(pairs + (size_t)r * 8, &lo, 4);
            std::memcpy(pairs + (size_t)r * 8 + 4, &step, 4);
        }
        interleave_group(gc.data(), n_g, row_codes, codes + (size_t)(16 * g) * row_codes);
        interleave_group(gm.data(), n_g, row_meta, meta + (size_t)(16 * g) * row_meta);
    }
    return QG_OK;
}

}  // extern "C"
