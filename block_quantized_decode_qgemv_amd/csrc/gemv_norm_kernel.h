// Kernels of the RMS-normalising GEMV (see gemv_norm.hip), shared by the two
// translation units that instantiate them: gemv_norm.hip (gain vector) and
// gemv_norm_unit.hip (unit gain), compiled in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemv_core.h"
#include "gemv_dispatch.h"
#include "internal.h"

namespace qg {
namespace norm {

using namespace core;


// Minimum waves per SIMD to compile for.  Q4_K at batch 8 needs 130 VGPRs
// with the norm's registers, which leaves room for one 8-wave workgroup per
// compute unit; capped at 128 (no spill) it keeps two, like the plain kernel.
template <int F, int B>
constexpr int norm_waves_per_eu() {
    return F == QG_Q4_K && B == 8 ? 4 : 1;
}

template <int F, int B, int W, int KCS, bool GAMMA>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(norm_waves_per_eu<F, B>())))
gemv_rmsnorm_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
                    const float* __restrict__ x, const float* __restrict__ gamma, float eps,
                    float* __restrict__ y, int N, int K) {
    const int g = blockIdx.x;
    GemvDpp<F, B, W, KCS>::template run_rmsnorm<GAMMA>(
        codes, meta, N, K, g, [&](int b) { return x + (size_t)b * K; }, B, gamma, eps,
        [&](auto sums, int n_g, int tid) {
            for (int t = tid; t < kRowGroup * B; t += W * 64)
                if (t / B < n_g) y[(size_t)(t % B) * N + g * kRowGroup + t / B] = sums(t);
        });
}

template <int F, int B, int W, int KCS, bool GAMMA>
struct RmsNormGemvG {
    static hipError_t launch(dim3 grid, dim3 block, hipStream_t st, const uint8_t* codes, const uint8_t* meta,
                             const float* x, const float* gamma, float eps, float* y, int N, int K) {
        hipLaunchKernelGGL((gemv_rmsnorm_kernel<F, B, W, KCS, GAMMA>), grid, block, 0, st, codes, meta, x, gamma,
                           eps, y, N, K);
        return hipGetLastError();
    }
    static int resident() { return resident_blocks(gemv_rmsnorm_kernel<F, B, W, KCS, GAMMA>, W * 64); }
};
// with a gain vector, and with unit gain (gamma folded into W)
template <int F, int B, int W, int KCS> struct RmsNormGemv : RmsNormGemvG<F, B, W, KCS, true> {};
template <int F, int B, int W, int KCS> struct RmsNormUnitGemv : RmsNormGemvG<F, B, W, KCS, false> {};

}  // namespace norm

// The unit-gain launch, instantiated in gemv_norm_unit.hip; arguments
// already validated by qgemv_rmsnorm.
hipError_t launch_rmsnorm_unit(int fmt, int N, int K, int B, hipStream_t st, const uint8_t* codes,
                               const uint8_t* meta, const float* x, float eps, float* y);

}  // namespace qg
