// Split-K GEMV kernels (see gemv_splitk.h): the partial sums of the
// register-x kernel over one piece of K per workgroup, and the fixed-order
// reduction of the pieces.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemv_core.h"
#include "gemv_dispatch.h"
#include "gemv_splitk.h"
#include "internal.h"

namespace qg {
namespace {

using namespace core;

// Row groups that fill a quarter of the compute units or fewer leave most of
// the chip idle when a batch makes the launch VALU-bound.  Split K: workgroup
// (g, s) sums row group g over code units [s * cps, (s + 1) * cps) into
// part[s][b][n]; the second launch adds the S partials of each output in
// order s = 0 .. S-1 (deterministic, no atomics).

template <int F, int B, int W, int KCS>
__global__ void __launch_bounds__(W * 64)
gemv_splitk_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
                   const float* __restrict__ x, float* __restrict__ part, int N, int K, int cps) {
    __shared__ float red[W * kRowGroup * B];
    const int g = blockIdx.x, s = blockIdx.y;
    float* ps = part + (size_t)s * B * N;
    GemvDpp<F, B, W, KCS>::run_group(
        codes, meta, N, K, g, [&](int b) { return x + (size_t)b * K; }, B,
        [&](auto sums, int n_g, int tid) {
            for (int t = tid; t < kRowGroup * B; t += W * 64)
                if (t / B < n_g) ps[(size_t)(t % B) * N + g * kRowGroup + t / B] = sums(t);
        },
        0, red, nullptr, 0.0f, nullptr, s * cps, (s + 1) * cps);
}

__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, float* __restrict__ y, int S, int total) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    float v = part[i];
    for (int s = 1; s < S; ++s) v += part[(size_t)s * total + i];
    y[i] = v;
}

// The split-K partial GEMV as a kernel set for the shared dispatch: its grid
// gains a second dimension, the S splits (the wave choice sees one split's
// row length).
template <int F, int B, int W, int KCS>
struct SplitGemv {
    static hipError_t launch(dim3 grid, dim3 block, hipStream_t st, const uint8_t* codes, const uint8_t* meta,
                             const float* x, float* part, int N, int K, int cps, int S) {
        hipLaunchKernelGGL((gemv_splitk_kernel<F, B, W, KCS>), dim3(grid.x, S), block, 0, st, codes, meta, x, part,
                           N, K, cps);
        return hipGetLastError();
    }
    static int resident() { return resident_blocks(gemv_splitk_kernel<F, B, W, KCS>, W * 64); }
};


// Columns per 16-byte code unit of a (validated) format.
int unit_columns(int fmt) {
    switch (fmt) {
        case QG_Q8_0: return Fmt<QG_Q8_0>::CPC;
        case QG_Q4_0: return Fmt<QG_Q4_0>::CPC;
        case QG_Q4_1: return Fmt<QG_Q4_1>::CPC;
        case QG_Q4_K: return Fmt<QG_Q4_K>::CPC;
        case QG_Q2_K: return Fmt<QG_Q2_K>::CPC;
        case QG_TERN: return Fmt<QG_TERN>::CPC;
        case QG_BIN8: return Fmt<QG_BIN8>::CPC;
        case QG_TERN3: return Fmt<QG_TERN3>::CPC;
        default: return Fmt<QG_BIN>::CPC;
    }
}

}  // namespace

hipError_t launch_gemv_splitk(int fmt, int N, int K, int B, int S, hipStream_t st, const uint8_t* codes,
                              const uint8_t* meta, const float* x, float* part, float* y) {
    const int cps = K / S / unit_columns(fmt);  // code units per piece
    // the wave choice sees one piece's row length
    hipError_t e = launch_dpp<SplitGemv>(fmt, N, K / S, B, st, codes, meta, x, part, N, K, cps, S);
    if (e != hipSuccess) return e;
    const int total = B * N;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((total + 255) / 256), dim3(256), 0, st, part, y, S, total);
    return hipGetLastError();
}

}  // namespace qg
