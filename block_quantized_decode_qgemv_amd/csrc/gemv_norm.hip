// GEMV on RMS-normalised activations: Y[b] = W * rmsnorm(X[b]), with
// rmsnorm(x)_k = x_k * gamma_k / sqrt(mean_k x_k^2 + eps).
//
// The Flash-MoE page runs RMS normalisation on the GPU in two passes (a
// sum-of-squares reduction, then its application; section "Metal 计算着色器")
// and keeps the combine + norm on the GPU so that it feeds the next layer's
// projection directly (section "延迟 GPU 专家计算").  Here both passes fold
// into the projection that consumes the normalised vector: the waves that
// load x for the register-x GEMV also sum its squares, gamma multiplies x in
// registers, and each batch row's 1/rms scales its finished row sums
// (GemvDpp::run_rmsnorm in gemv_core.h).  The normalised vector is never
// written, and the call costs one launch like the plain GEMV.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "gemv_core.h"
#include "gemv_dispatch.h"
#include "internal.h"

namespace qg {
namespace {

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

}  // namespace
}  // namespace qg

using namespace qg;

extern "C" int qgemv_rmsnorm(int fmt, const void* w, const float* x, const float* gamma, float eps, float* y,
                             int64_t N, int64_t K, int B, void* stream) {
    clear_error();
    int rc = check_gemv_args(fmt, w, x, y, N, K, B);
    if (rc) return rc;
    if (gamma && !aligned(gamma, 16)) return fail(QG_EALIGN, "gamma must be 16-byte aligned");
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(QG_ERANGE, "eps=%g must be finite and >= 0", (double)eps);
    if (gamma && overlap(y, (size_t)B * N * 4, gamma, (size_t)K * 4))
        return fail(QG_EINVAL, "y must not overlap gamma");
    const uint8_t* codes = static_cast<const uint8_t*>(w);
    const uint8_t* meta = codes + qg_codes_plane_size(fmt, N, K);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = gamma ? core::launch_dpp<RmsNormGemv>(fmt, (int)N, (int)K, B, st, codes, meta, x, gamma, eps, y,
                                                         (int)N, (int)K)
                         : core::launch_dpp<RmsNormUnitGemv>(fmt, (int)N, (int)K, B, st, codes, meta, x, gamma, eps,
                                                             y, (int)N, (int)K);
    if (e != hipSuccess) return fail(QG_EHIP, "GEMV launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}
