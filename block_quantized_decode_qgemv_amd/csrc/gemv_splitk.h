// Split-K GEMV (gemv_splitk.hip): for row-starved launches at batch 5 and
// up, K is cut into S pieces of whole 256-column spans; workgroup (g, s) sums
// row group g over piece s into part[s][B][N] (a caller workspace of
// S * B * N floats), then a second launch adds the S partials of each output
// in order s = 0 .. S-1 into y (deterministic, no atomics).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qg {

// Format, shape, batch and S (2 or 4, K % (256 S) == 0) are validated by the caller.
hipError_t launch_gemv_splitk(int fmt, int N, int K, int B, int S, hipStream_t st, const uint8_t* codes,
                              const uint8_t* meta, const float* x, float* part, float* y);

}  // namespace qg
