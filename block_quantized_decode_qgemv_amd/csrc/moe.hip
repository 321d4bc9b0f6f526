// Routed MoE expert layer at decode (Flash-MoE page, sections "模型架构" --
// 512 experts, K active plus one shared, hidden 4096 -- "Metal 计算着色器" --
// fused SwiGLU and the fused combine + residual + sigmoid gate -- and
// "每层流水线" -- softmax + top-K routing; EPM README, section "正確性": the
// routed matmul semantics).  Here every step stays on the GPU (the Flash-MoE
// page routes on the CPU between command buffers) because every expert is
// resident in HBM:
//
//   1. route: one workgroup computes each token's softmax over E logits, its
//      top-K experts (ties to the lower index) and weights, and
//      sigmoid(shared-gate logit); then it groups the (token, k) pairs into
//      work items -- one expert with at most 2 tokens, in order of first
//      appearance -- and appends the shared expert as ceil(T/2) items;
//   2. gate/up: one grouped GEMV over the items (x rows gathered by token);
//      gate and up rows are interleaved (row 2i = gate i, row 2i+1 = up i), so
//      each 16-row group holds 8 (gate, up) pairs and the epilogue writes
//      h = silu(gate) * up directly (fused SwiGLU);
//   3. down: one grouped GEMV of each item's h rows; the epilogue scales by
//      the token's routing weight (sigmoid gate for the shared expert) and
//      writes a per-(token, slot) partial output;
//   4. combine: out = residual + sum of the K routed partials + the shared
//      partial, in that fixed order (deterministic; no float atomics).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "gemv_core.h"
#include "internal.h"

namespace qg {
namespace {

using namespace core;

constexpr int kMaxT = 8, kMaxTopK = 8, kMaxE = 4096;
constexpr int kItemInts = 8;  // expert, count, tok[2], kslot[2], wt[2] (as float bits)

// Workspace layout, byte offsets (each region 256-byte aligned).
struct MoeLayout {
    int max_items;
    size_t items, h, partial, total;
    MoeLayout(int T, int H, int I, int top_k) {
        max_items = T * top_k + (T + 1) / 2;
        auto up = [](size_t v) { return (v + 255) / 256 * 256; };
        items = 0;
        h = up(items + (size_t)(1 + max_items) * kItemInts * 4);
        partial = up(h + (size_t)max_items * 2 * I * 4);
        total = up(partial + (size_t)T * (top_k + 1) * H * 4);
    }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// ------------------------------------------------------------------ route
// items[0] = number of items; item j at items + 8*(1+j):
//   {expert, count, tok0, tok1, kslot0, kslot1, wt0 bits, wt1 bits}

__global__ void __launch_bounds__(512)
moe_route_kernel(const float* __restrict__ logits, const float* __restrict__ shared_logit, int T, int E,
                 int top_k, unsigned flags, int* __restrict__ items) {
    __shared__ int sel_e[kMaxT * kMaxTopK];
    __shared__ float sel_w[kMaxT * kMaxTopK];
    __shared__ float sig[kMaxT];
    __shared__ int sub_base[kMaxT * kMaxTopK];
    __shared__ int n_routed;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    if (wave < T) {
        const float* l = logits + (size_t)wave * E;
        float m = -INFINITY;
        for (int i = lane; i < E; i += 64) m = fmaxf(m, l[i]);
        m = wave_max(m);
        float s = 0.0f;
        for (int i = lane; i < E; i += 64) s += expf(l[i] - m);
        s = wave_sum(s);
        int chosen[kMaxTopK];
        float wsum = 0.0f;
        for (int k = 0; k < top_k; ++k) {
            // (value, index) keys in a total order: larger value first, then
            // the lower index; NaN counts as -inf and "no candidate" (index
            // kNone) loses to everything, so the pick is always a valid expert
            constexpr int kNone = 0x7fffffff;
            float best = -INFINITY;
            int bi = kNone;
            for (int i = lane; i < E; i += 64) {
                bool taken = false;
                for (int j = 0; j < k; ++j) taken |= chosen[j] == i;
                const float v = __builtin_isnan(l[i]) ? -INFINITY : l[i];
                if (!taken && (bi == kNone || v > best || (v == best && i < bi))) { best = v; bi = i; }
            }
#pragma unroll
            for (int msk = 32; msk >= 1; msk >>= 1) {
                const float ov = __shfl_xor(best, msk);
                const int oi = __shfl_xor(bi, msk);
                if (oi != kNone && (bi == kNone || ov > best || (ov == best && oi < bi))) { best = ov; bi = oi; }
            }
            chosen[k] = bi;
            const float p = expf(best - m) / s;
            wsum += p;
            if (lane == 0) {
                sel_e[wave * top_k + k] = bi;
                sel_w[wave * top_k + k] = p;
            }
        }
        if (lane == 0) {
            if (flags & QG_MOE_RENORM)
                for (int k = 0; k < top_k; ++k) sel_w[wave * top_k + k] /= wsum;
            sig[wave] = 1.0f / (1.0f + expf(-shared_logit[wave]));
        }
    }
    __syncthreads();

    // group the pairs q = t*top_k + k by expert, in order of first appearance
    const int P = T * top_k;
    int e = 0, pos = 0, cnt = 0;
    bool leader = false;
    if (tid < P) {
        e = sel_e[tid];
        leader = true;
        for (int q = 0; q < P; ++q) {
            const bool same = sel_e[q] == e;
            cnt += same;
            if (q < tid && same) { leader = false; ++pos; }
        }
    }
    __syncthreads();
    if (tid < P && leader) {
        // items of the experts that appear first before this one
        int base = 0;
        for (int q = 0; q < tid; ++q) {
            const int eq = sel_e[q];
            bool first = true;
            int c = 0;
            for (int r = 0; r < P; ++r) {
                c += sel_e[r] == eq;
                first &= !(r < q && sel_e[r] == eq);
            }
            if (first) base += (c + 1) / 2;
        }
        sub_base[tid] = base;
    }
    if (tid == 0) {
        int total = 0;
        for (int q = 0; q < P; ++q) {
            bool first = true;
            int c = 0;
            for (int r = 0; r < P; ++r) {
                c += sel_e[r] == sel_e[q];
                first &= !(r < q && sel_e[r] == sel_e[q]);
            }
            if (first) total += (c + 1) / 2;
        }
        n_routed = total;
    }
    __syncthreads();
    if (tid < P) {
        int lead = tid;
        for (int q = 0; q < tid; ++q)
            if (sel_e[q] == e) { lead = q; break; }
        const int item = sub_base[lead] + pos / 2, slot = pos % 2;
        int* it = items + kItemInts * (1 + item);
        if (slot == 0) {
            it[0] = e;
            it[1] = min(2, cnt - pos);
        }
        it[2 + slot] = tid / top_k;
        it[4 + slot] = tid % top_k;
        it[6 + slot] = __float_as_int(sel_w[tid]);
    }
    // the shared expert (index E): tokens (2j, 2j+1), weight sigmoid(s_t)
    if (tid < (T + 1) / 2) {
        const int j = tid;
        int* it = items + kItemInts * (1 + n_routed + j);
        const int c = min(2, T - 2 * j);
        it[0] = E;
        it[1] = c;
        it[2] = 2 * j;
        it[3] = c > 1 ? 2 * j + 1 : 2 * j;
        it[4] = top_k;
        it[5] = top_k;
        it[6] = __float_as_int(sig[2 * j]);
        it[7] = __float_as_int(c > 1 ? sig[2 * j + 1] : 0.0f);
    }
    if (tid == 0) items[0] = n_routed + (T + 1) / 2;
}

// ------------------------------------------------------- grouped GEMVs

struct Item {
    int expert, count, tok[2], kslot[2];
    float wt[2];
};

__device__ __forceinline__ Item read_item(const int* items, int j) {
    const int* it = items + kItemInts * (1 + j);
    Item r;
    r.expert = it[0];
    r.count = it[1];
    r.tok[0] = it[2];
    r.tok[1] = it[3];
    r.kslot[0] = it[4];
    r.kslot[1] = it[5];
    r.wt[0] = __int_as_float(it[6]);
    r.wt[1] = __int_as_float(it[7]);
    return r;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// gate/up rows interleaved: group g holds gate rows 8g..8g+7 (rows 2i) and up
// rows (rows 2i+1); h[item][b][8g + i] = silu(gate) * up
template <int F, int W, int KCS>
__global__ void __launch_bounds__(W * 64)
moe_gate_up_kernel(const uint8_t* __restrict__ wgu, size_t expert_bytes, size_t codes_bytes, int H, int I,
                   const float* __restrict__ x, const int* __restrict__ items, float* __restrict__ h) {
    const int j = blockIdx.y;
    if (j >= items[0]) return;  // uniform: unused item slot
    const Item it = read_item(items, j);
    const uint8_t* codes = wgu + (size_t)it.expert * expert_bytes;
    const uint8_t* meta = codes + codes_bytes;
    const int g = blockIdx.x;
    float* hj = h + (size_t)j * 2 * I;
    auto xrow = [&](int b) { return x + (size_t)it.tok[b] * H; };
    auto epi = [&](int B) {
        return [=](auto sums, int) {
            for (int t = threadIdx.x; t < 8 * B; t += W * 64) {
                const int i = t / B, b = t % B;
                if (b < it.count) hj[(size_t)b * I + 8 * g + i] = silu(sums((2 * i) * B + b)) * sums((2 * i + 1) * B + b);
            }
        };
    };
    if (it.count == 1) GemvDpp<F, 1, W, KCS>::run(codes, meta, 2 * I, H, g, xrow, 1, epi(1));
    else GemvDpp<F, 2, W, KCS>::run(codes, meta, 2 * I, H, g, xrow, 2, epi(2));
}

// down: partial[tok][kslot][row] = weight * (W_down h)[row]
template <int F, int W, int KCS>
__global__ void __launch_bounds__(W * 64)
moe_down_kernel(const uint8_t* __restrict__ wdn, size_t expert_bytes, size_t codes_bytes, int H, int I,
                int top_k, const int* __restrict__ items, const float* __restrict__ h, float* __restrict__ partial) {
    const int j = blockIdx.y;
    if (j >= items[0]) return;
    const Item it = read_item(items, j);
    const uint8_t* codes = wdn + (size_t)it.expert * expert_bytes;
    const uint8_t* meta = codes + codes_bytes;
    const int g = blockIdx.x;
    const float* hj = h + (size_t)j * 2 * I;
    auto xrow = [&](int b) { return hj + (size_t)b * I; };
    auto epi = [&](int B) {
        return [=](auto sums, int n_g) {
            for (int t = threadIdx.x; t < kRowGroup * B; t += W * 64) {
                const int rw = t / B, b = t % B;
                // selects, not it.tok[b]: a runtime index would put the item in scratch
                const int tok = b ? it.tok[1] : it.tok[0], ks = b ? it.kslot[1] : it.kslot[0];
                const float wt = b ? it.wt[1] : it.wt[0];
                if (b < it.count && rw < n_g)
                    partial[((size_t)tok * (top_k + 1) + ks) * H + kRowGroup * g + rw] = wt * sums(t);
            }
        };
    };
    if (it.count == 1) GemvDpp<F, 1, W, KCS>::run(codes, meta, H, I, g, xrow, 1, epi(1));
    else GemvDpp<F, 2, W, KCS>::run(codes, meta, H, I, g, xrow, 2, epi(2));
}

// out = residual + sum_k partial[k] (k = 0 .. top_k, the last being the
// shared expert), in that order
__global__ void __launch_bounds__(256)
moe_combine_kernel(const float* __restrict__ residual, const float* __restrict__ partial, float* __restrict__ out,
                   int T, int H, int top_k) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * H) return;
    const int t = idx / H, c = idx - t * H;
    float v = residual[idx];
    for (int k = 0; k <= top_k; ++k) v += partial[((size_t)t * (top_k + 1) + k) * H + c];
    out[idx] = v;
}

// ------------------------------------------------------------- launchers

template <int F, int W, int KCS>
hipError_t launch_gate_up_w(const uint8_t* wgu, int H, int I, const float* x, const int* items, float* h,
                            int max_items, hipStream_t st) {
    const size_t eb = qg_packed_size(F, 2 * (int64_t)I, H), cb = qg_codes_plane_size(F, 2 * (int64_t)I, H);
    hipLaunchKernelGGL((moe_gate_up_kernel<F, W, KCS>), dim3(2 * I / kRowGroup, max_items), dim3(W * 64), 0, st,
                       wgu, eb, cb, H, I, x, items, h);
    return hipGetLastError();
}

template <int F, int W, int KCS>
hipError_t launch_down_w(const uint8_t* wdn, int H, int I, int top_k, const int* items, const float* h,
                         float* partial, int max_items, hipStream_t st) {
    const size_t eb = qg_packed_size(F, H, I), cb = qg_codes_plane_size(F, H, I);
    hipLaunchKernelGGL((moe_down_kernel<F, W, KCS>), dim3(H / kRowGroup, max_items), dim3(W * 64), 0, st,
                       wdn, eb, cb, H, I, top_k, items, h, partial);
    return hipGetLastError();
}

template <int F>
hipError_t launch_moe(const uint8_t* wgu, const uint8_t* wdn, int E, int H, int I, int top_k, const float* x,
                      const float* residual, const float* logits, const float* slogit, int T, unsigned flags,
                      float* out, uint8_t* ws, hipStream_t st) {
    // register-x GEMVs (items carry at most 2 tokens)
    constexpr int KCS = dpp_lane_units<F>();
    static_assert(dpp_max_batch<F>() >= 2, "two tokens per item");
    const MoeLayout L(T, H, I, top_k);
    int* items = reinterpret_cast<int*>(ws + L.items);
    float* h = reinterpret_cast<float*>(ws + L.h);
    float* partial = reinterpret_cast<float*>(ws + L.partial);
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(512), 0, st, logits, slogit, T, E, top_k, flags, items);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (pick_waves_dpp<F, KCS>(H)) {
        case 1: e = launch_gate_up_w<F, 1, KCS>(wgu, H, I, x, items, h, L.max_items, st); break;
        case 2: e = launch_gate_up_w<F, 2, KCS>(wgu, H, I, x, items, h, L.max_items, st); break;
        case 4: e = launch_gate_up_w<F, 4, KCS>(wgu, H, I, x, items, h, L.max_items, st); break;
        case 8: e = launch_gate_up_w<F, 8, KCS>(wgu, H, I, x, items, h, L.max_items, st); break;
        default: e = launch_gate_up_w<F, 16, KCS>(wgu, H, I, x, items, h, L.max_items, st); break;
    }
    if (e != hipSuccess) return e;
    switch (pick_waves_dpp<F, KCS>(I)) {
        case 1: e = launch_down_w<F, 1, KCS>(wdn, H, I, top_k, items, h, partial, L.max_items, st); break;
        case 2: e = launch_down_w<F, 2, KCS>(wdn, H, I, top_k, items, h, partial, L.max_items, st); break;
        case 4: e = launch_down_w<F, 4, KCS>(wdn, H, I, top_k, items, h, partial, L.max_items, st); break;
        case 8: e = launch_down_w<F, 8, KCS>(wdn, H, I, top_k, items, h, partial, L.max_items, st); break;
        default: e = launch_down_w<F, 16, KCS>(wdn, H, I, top_k, items, h, partial, L.max_items, st); break;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((T * H + 255) / 256), dim3(256), 0, st, residual, partial, out, T, H,
                       top_k);
    return hipGetLastError();
}

}  // namespace
}  // namespace qg

using namespace qg;

extern "C" {

size_t moe_expert_ffn_workspace_size(int T, int E, int H, int I, int top_k) {
    if (T < 1 || T > kMaxT || E < 1 || E > kMaxE || H < 256 || I < 256 || H % 256 || I % 256 || top_k < 1 ||
        top_k > kMaxTopK || top_k > E)
        return 0;
    return MoeLayout(T, H, I, top_k).total;
}

int moe_expert_ffn(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k,
                   const float* x, const float* residual, const float* router_logits,
                   const float* shared_gate_logit, int T, unsigned flags, float* out,
                   void* workspace, size_t ws_bytes, void* stream) {
    clear_error();
    if (fmt != QG_Q4_K && fmt != QG_Q2_K) return fail(QG_EINVAL, "moe_expert_ffn takes Q4_K or Q2_K experts");
    if (!w_gate_up || !w_down || !x || !residual || !router_logits || !shared_gate_logit || !out || !workspace)
        return fail(QG_EINVAL, "null pointer");
    if (T < 1 || T > kMaxT) return fail(QG_ERANGE, "T=%d must be in [1, %d]", T, kMaxT);
    if (E < 1 || E > kMaxE) return fail(QG_ERANGE, "E=%d must be in [1, %d]", E, kMaxE);
    if (top_k < 1 || top_k > kMaxTopK || top_k > E)
        return fail(QG_ERANGE, "top_k=%d must be in [1, min(E, %d)]", top_k, kMaxTopK);
    if (H < 256 || H % 256 || I < 256 || I % 256)
        return fail(QG_ESHAPE, "H=%d and I=%d must be positive multiples of 256", H, I);
    if (flags & ~QG_MOE_RENORM) return fail(QG_EINVAL, "unknown flags 0x%x", flags);
    if (!aligned(w_gate_up, 16) || !aligned(w_down, 16) || !aligned(x, 16) || !aligned(workspace, 16))
        return fail(QG_EALIGN, "weights, x and workspace must be 16-byte aligned");
    if (!aligned(residual, 4) || !aligned(router_logits, 4) || !aligned(shared_gate_logit, 4) || !aligned(out, 4))
        return fail(QG_EALIGN, "residual, logits and out must be 4-byte aligned");
    const size_t need = MoeLayout(T, H, I, top_k).total;
    if (ws_bytes < need) return fail(QG_ERANGE, "workspace of %zu bytes is below the %zu needed", ws_bytes, need);
    if ((const void*)out == (const void*)x || (const void*)out == (const void*)residual)
        return fail(QG_EINVAL, "out must not alias x or residual");
    const uint8_t* wgu = static_cast<const uint8_t*>(w_gate_up);
    const uint8_t* wdn = static_cast<const uint8_t*>(w_down);
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    hipError_t e = fmt == QG_Q4_K
        ? launch_moe<QG_Q4_K>(wgu, wdn, E, H, I, top_k, x, residual, router_logits, shared_gate_logit, T, flags, out, ws, st)
        : launch_moe<QG_Q2_K>(wgu, wdn, E, H, I, top_k, x, residual, router_logits, shared_gate_logit, T, flags, out, ws, st);
    if (e != hipSuccess) return fail(QG_EHIP, "MoE launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // extern "C"
