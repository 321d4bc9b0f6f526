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

#include "gemv_norm_kernel.h"
#include "internal.h"

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
    hipError_t e = gamma ? core::launch_dpp<norm::RmsNormGemv>(fmt, (int)N, (int)K, B, st, codes, meta, x, gamma,
                                                               eps, y, (int)N, (int)K)
                         : launch_rmsnorm_unit(fmt, (int)N, (int)K, B, st, codes, meta, x, eps, y);
    if (e != hipSuccess) return fail(QG_EHIP, "GEMV launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}
