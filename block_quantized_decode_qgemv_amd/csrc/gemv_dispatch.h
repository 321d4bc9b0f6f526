// Launch-time choices of the register-x GEMV, shared by the entry points
// that use it (plain and RMS-normalising).  A kernel set KS<F, B, W, KCS>
// provides, for one configuration:
//   static hipError_t launch(dim3 grid, dim3 block, hipStream_t st, args...);
//   static int resident();   // workgroups one compute unit holds at once
#pragma once

#include <hip/hip_runtime.h>

#include "gemv_core.h"
#include "internal.h"

namespace qg {
namespace core {

// Resident workgroups of KS<F, B, W>, queried once per configuration.
template <template <int, int, int, int> class KS, int F, int B, int W>
int dpp_resident() {
    static const int n = [] {
        const int b = KS<F, B, W, dpp_lane_units<F, B>()>::resident();
        return b < 1 ? 1 : b;
    }();
    return n;
}

// Waves per workgroup: start from the fewest that cover a row in one slice
// (pick_waves_dpp), then halve while too few workgroups fit on a compute unit:
// one when the grid has at most one workgroup per compute unit, else two, so
// that a workgroup's reduction and tail overlap another's streaming.
template <template <int, int, int, int> class KS, int F, int B>
int choose_waves_dpp(int N, int K) {
    constexpr int MW = dpp_max_waves<F, B>();
    const int groups = (N + kRowGroup - 1) / kRowGroup;
    const int need = groups > device_cus() ? 2 : 1;
    int w = pick_waves_dpp<F, dpp_lane_units<F, B>()>(K, MW);
    for (; w > 1; w /= 2) {
        int res = 1;
        switch (w) {
            case 2: res = dpp_resident<KS, F, B, 2>(); break;
            case 4: res = dpp_resident<KS, F, B, 4>(); break;
            case 8: res = dpp_resident<KS, F, B, 8>(); break;
            default:
                if constexpr (MW == 16) res = dpp_resident<KS, F, B, 16>();
                break;
        }
        if (res >= need) break;
    }
    return w;
}

template <template <int, int, int, int> class KS, int F, int B, int W, class... Args>
hipError_t launch_dpp_w(int N, hipStream_t st, Args... args) {
    const int grid = (N + kRowGroup - 1) / kRowGroup;
    return KS<F, B, W, dpp_lane_units<F, B>()>::launch(dim3(grid), dim3(W * 64), st, args...);
}

template <template <int, int, int, int> class KS, int F, int B, class... Args>
hipError_t launch_dpp_b(int N, int K, hipStream_t st, Args... args) {
    static_assert(B <= dpp_max_batch<F>(), "every batch runs the register-x kernel");
    constexpr int MW = dpp_max_waves<F, B>();
    switch (choose_waves_dpp<KS, F, B>(N, K)) {
        case 1: return launch_dpp_w<KS, F, B, 1>(N, st, args...);
        case 2: return launch_dpp_w<KS, F, B, 2>(N, st, args...);
        case 4: return launch_dpp_w<KS, F, B, 4>(N, st, args...);
        case 8: return launch_dpp_w<KS, F, B, 8>(N, st, args...);
        default:
            if constexpr (MW == 16) return launch_dpp_w<KS, F, B, 16>(N, st, args...);
            return hipErrorInvalidConfiguration;  // never chosen
    }
}

template <template <int, int, int, int> class KS, int F, class... Args>
hipError_t launch_dpp_f(int N, int K, int B, hipStream_t st, Args... args) {
    switch (B) {
        case 1: return launch_dpp_b<KS, F, 1>(N, K, st, args...);
        case 2: return launch_dpp_b<KS, F, 2>(N, K, st, args...);
        case 3: return launch_dpp_b<KS, F, 3>(N, K, st, args...);
        case 4: return launch_dpp_b<KS, F, 4>(N, K, st, args...);
        case 5: return launch_dpp_b<KS, F, 5>(N, K, st, args...);
        case 6: return launch_dpp_b<KS, F, 6>(N, K, st, args...);
        case 7: return launch_dpp_b<KS, F, 7>(N, K, st, args...);
        default: return launch_dpp_b<KS, F, 8>(N, K, st, args...);
    }
}

// Dispatch on the format (validated by the caller), then the batch.
template <template <int, int, int, int> class KS, class... Args>
hipError_t launch_dpp(int fmt, int N, int K, int B, hipStream_t st, Args... args) {
    switch (fmt) {
        case QG_Q8_0: return launch_dpp_f<KS, QG_Q8_0>(N, K, B, st, args...);
        case QG_Q4_0: return launch_dpp_f<KS, QG_Q4_0>(N, K, B, st, args...);
        case QG_Q4_1: return launch_dpp_f<KS, QG_Q4_1>(N, K, B, st, args...);
        case QG_Q4_K: return launch_dpp_f<KS, QG_Q4_K>(N, K, B, st, args...);
        case QG_Q2_K: return launch_dpp_f<KS, QG_Q2_K>(N, K, B, st, args...);
        case QG_TERN: return launch_dpp_f<KS, QG_TERN>(N, K, B, st, args...);
        case QG_BIN8: return launch_dpp_f<KS, QG_BIN8>(N, K, B, st, args...);
        case QG_TERN3: return launch_dpp_f<KS, QG_TERN3>(N, K, B, st, args...);
        default: return launch_dpp_f<KS, QG_BIN>(N, K, B, st, args...);
    }
}

// Occupancy query helper for kernel sets: resident workgroups of `kernel` at
// `threads` per workgroup (1 if the query fails).
template <class Kernel>
int resident_blocks(Kernel kernel, int threads) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kernel, threads, 0) != hipSuccess) {
        (void)hipGetLastError();
        b = 1;
    }
    return b;
}

}  // namespace core
}  // namespace qg
