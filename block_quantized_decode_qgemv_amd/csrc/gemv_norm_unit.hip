// Unit-gain instances of the RMS-normalising GEMV (gamma folded into the
// weights), in a translation unit of their own so that the library's two
// largest instance sets compile in parallel.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemv_norm_kernel.h"
#include "internal.h"

namespace qg {

hipError_t launch_rmsnorm_unit(int fmt, int N, int K, int B, hipStream_t st, const uint8_t* codes,
                               const uint8_t* meta, const float* x, float eps, float* y) {
    return core::launch_dpp<norm::RmsNormUnitGemv>(fmt, N, K, B, st, codes, meta, x, (const float*)nullptr, eps, y,
                                                   N, K);
}

}  // namespace qg
