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
//      appearance -- and appends the shared expert as ceil(T/2) items (a
//      single token needs no routing launch: the gate/up workgroups route it);
//   2. gate/up: one grouped GEMV over the items (x rows gathered by token);
//      gate and up rows are interleaved (row 2i = gate i, row 2i+1 = up i), so
//      each 16-row group holds 8 (gate, up) pairs and the epilogue writes
//      h = silu(gate) * up directly (fused SwiGLU);
//   3. down + combine: for each 16 output rows, one or a few workgroups that
//      share the tokens; for each of its tokens in turn (or two or three at
//      once) a workgroup runs the down projection of the token's K + 1 slots,
//      each in its own wave group, scales it by the slot's routing weight
//      (sigmoid gate for the shared expert), and writes out = residual + the
//      K routed sums + the shared sum, in that fixed order (deterministic; no
//      float atomics and no partial results leaving the workgroup).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "gemv_core.h"
#include "internal.h"

// Workspace of moe_expert_ffn_noalloc (callers that cannot allocate): a
// stated maximum, held by every device the library runs on until the
// process ends.
constexpr size_t kNoAllocScratchBytes = (size_t)2 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace qg {
namespace {

using namespace core;

constexpr int kMaxT = 8, kMaxTopK = 8, kMaxE = 4096;
// Up to this many experts, a single token's route is computed inside the
// gate/up workgroups (8 logits per lane) instead of by a routing launch.
constexpr int kRouteInGateUpMaxE = 512;
// Down workgroups per 16-row group when the down takes one token at a time
// (a single token, or odd T where three slot groups do not fit a workgroup);
// each takes its share of the T tokens in turn.  Measured for the layer at
// T = 2..8 against every power of two of tokens per workgroup, same machine:
// Q4_K is fastest with 4 tokens per workgroup (T = 8: 65.3 us against 67.8
// with one token per workgroup), Q2_K with two workgroups whatever T (T = 4:
// 31.0 against 33.7 with one).
template <int F>
int down_token_groups(int T) {
    return F == QG_Q2_K ? (T < 2 ? T : 2) : (T + 3) / 4;
}
constexpr int kItemInts = 8;  // expert, count, tok[2], kslot[2], wt[2] (as float bits)

// Workspace layout, byte offsets (each region 256-byte aligned).
struct MoeLayout {
    int max_items;
    size_t items, hsel, h, total;
    MoeLayout(int T, int H, int I, int top_k) {
        (void)H;
        max_items = T * top_k + (T + 1) / 2;
        auto up = [](size_t v) { return (v + 255) / 256 * 256; };
        items = 0;
        hsel = up(items + (size_t)(1 + max_items) * kItemInts * 4);  // [T][top_k + 1]: 2 * item + b
        h = up(hsel + (size_t)T * (top_k + 1) * 4);
        total = up(h + (size_t)max_items * 2 * I * 4);
    }
};

// ------------------------------------------------------------------ route
// items[0] = number of items; item j at items + 8*(1+j):
//   {expert, count, tok0, tok1, kslot0, kslot1, wt0 bits, wt1 bits}

// In-row DPP steps (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror) leave each 16-lane row's result in all its lanes; the four row
// results are then read into scalars and combined.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false); }
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float rl(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return fmaxf(fmaxf(rl(v, 0), rl(v, 16)), fmaxf(rl(v, 32), rl(v, 48)));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return (rl(v, 0) + rl(v, 16)) + (rl(v, 32) + rl(v, 48));
}

// One token's logits in a wave's registers: lane owns experts lane + 64 m.
// A NaN logit counts as -inf; experts past E hold NaN, which the selection
// below never picks.
template <int MPL>
__device__ __forceinline__ void load_logits(const float* __restrict__ l, int E, int lane, float (&v)[MPL]) {
#pragma unroll
    for (int m = 0; m < MPL; ++m) {
        const int i = lane + 64 * m;
        const float x = i < E ? l[i] : 0.0f;
        v[m] = i < E ? (__builtin_isnan(x) ? -INFINITY : x) : __builtin_nanf("");
    }
}

// The first `rounds` rounds of the top-K selection: round k takes the largest
// remaining logit (a wave maximum; NaN, for experts past E and experts
// already taken, is passed over by fmaxf and equals nothing) and, between
// equal logits (-0 equal to +0), the lowest expert index -- the lowest m
// whose ballot is non-empty, then that ballot's lowest lane.  Lane k keeps
// round k's expert (my_e) and logit (my_v).  rounds <= E.
template <int MPL>
__device__ __forceinline__ void top_rounds(float (&v)[MPL], int rounds, int lane, int& my_e, float& my_v) {
    my_e = 0;
    my_v = -INFINITY;
    for (int k = 0; k < rounds; ++k) {
        float lm = v[0];
#pragma unroll
        for (int m = 1; m < MPL; ++m) lm = fmaxf(lm, v[m]);
        const float wm = wave_max_dpp(lm);  // the same in every lane
        int win = -1;
#pragma unroll
        for (int m = 0; m < MPL; ++m) {
            const uint64_t bal = __ballot(v[m] == wm);  // uniform
            if (bal) {
                win = (int)__builtin_ctzll(bal) + 64 * m;
                break;
            }
        }
#pragma unroll
        for (int m = 0; m < MPL; ++m) v[m] = lane + 64 * m == win ? __builtin_nanf("") : v[m];  // taken
        if (lane == k) {
            my_e = win < 0 ? 0 : win;
            my_v = wm;
        }
    }
}

// One token's route, computed by one wave: softmax statistics, then top_k
// rounds of a wave argmax; returns, in lane k < top_k, the k-th expert
// (my_e) and its routing weight (my_w), and the sigmoid of the shared-gate
// logit in every lane.
template <int MPL>  // experts per lane: E <= 64 * MPL
__device__ __forceinline__ void route_token(const float* __restrict__ l, float sl, int E, int top_k, unsigned flags,
                                            int lane, int& my_e, float& my_w, float& sig) {
    float v[MPL];
    load_logits<MPL>(l, E, lane, v);
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < MPL; ++m) mx = fmaxf(mx, v[m]);
    mx = wave_max_dpp(mx);
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < MPL; ++m)
        if (lane + 64 * m < E) s += expf(v[m] - mx);
    s = wave_sum_dpp(s);
    float my_v;
    top_rounds<MPL>(v, top_k, lane, my_e, my_v);
    // the weights, off the rounds' dependency chain: lane k turns its logit
    // into a probability; the renormalising sum adds them in round order
    const float my_p = expf(my_v - mx) / s;
    float wsum = 0.0f;
    if (flags & QG_MOE_RENORM)
        for (int k = 0; k < top_k; ++k) wsum += rl(my_p, k);
    my_w = (flags & QG_MOE_RENORM) ? my_p / wsum : my_p;
    sig = 1.0f / (1.0f + expf(-sl));
}

template <int MPL>  // experts per lane: E <= 64 * MPL
__global__ void __launch_bounds__(512)
moe_route_kernel(const float* __restrict__ logits, const float* __restrict__ shared_logit, int T, int E,
                 int top_k, unsigned flags, int* __restrict__ items, int* __restrict__ hsel) {
    __shared__ int sel_e[kMaxT * kMaxTopK];
    __shared__ float sel_w[kMaxT * kMaxTopK];
    __shared__ float sig[kMaxT];
    __shared__ uint64_t expert_pairs[kMaxE];  // only the chosen experts' entries are touched
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // (1) one wave per token
    if (wave < T) {
        int my_e;
        float my_w, sg;
        route_token<MPL>(logits + (size_t)wave * E, shared_logit[wave], E, top_k, flags, lane, my_e, my_w, sg);
        if (lane < top_k) {
            sel_e[wave * top_k + lane] = my_e;
            sel_w[wave * top_k + lane] = my_w;
        }
        if (lane == 0) sig[wave] = sg;
    }
    __syncthreads();

    // (2) wave 0 groups the pairs q = t*top_k + k (lane q) by expert, in order of
    // first appearance, into items of at most two tokens
    if (wave == 0) {
        const int P = T * top_k;  // <= 64
        const bool act = lane < P;
        const int e = act ? sel_e[lane] : 0;
        // the set of pairs that chose each expert, as a lane mask in LDS: cleared,
        // then or-ed by every pair (LDS operations of one wave run in order)
        if (act) expert_pairs[e] = 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (act) __hip_atomic_fetch_or(&expert_pairs[e], 1ull << lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const uint64_t same = act ? expert_pairs[e] : 0;
        const int cnt = __popcll(same);                                  // pairs of this expert
        const int pos = __popcll(same & ((1ull << lane) - 1));          // earlier pairs of it
        const int lead = act ? __builtin_ctzll(same) : lane;             // its first pair
        const int nit = (act && pos == 0) ? (cnt + 1) / 2 : 0;  // items of this expert, at its first pair
        // items of experts first seen before the lead pair (exclusive scan over
        // lanes), and all items.  Inclusive scan by DPP: shifts within each
        // 16-lane row (lanes without a source add 0), then the row totals by
        // row broadcasts (rows 1 and 3 add lane 15 of the row before, rows 2
        // and 3 add lane 31); 0.2 us faster per routing launch than lane
        // shuffles through LDS, same records.
        int incl = nit;
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);   // row_shr:1
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);   // row_shr:2
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);   // row_shr:4
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);   // row_shr:8
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x142, 0xA, 0xF, false);  // row_bcast:15
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x143, 0xC, 0xF, false);  // row_bcast:31
        const int base = __shfl(incl - nit, lead);
        const int n_routed = __shfl(incl, 63);
        if (act) {
            const int item = base + pos / 2, slot = pos % 2;
            int* it = items + kItemInts * (1 + item);
            const int tok = lane / top_k, ks = lane % top_k;
            const int wbits = __float_as_int(sel_w[lane]);
            hsel[tok * (top_k + 1) + ks] = 2 * item + slot;
            if (slot == 0) {
                const int c = min(2, cnt - pos);
                it[0] = e;
                it[1] = c;
                it[2] = tok;
                it[4] = ks;
                it[6] = wbits;
                if (c == 1) { it[3] = tok; it[5] = ks; it[7] = 0; }  // unused second slot
            } else {
                it[3] = tok;
                it[5] = ks;
                it[7] = wbits;
            }
        }
        // the shared expert (index E): tokens (2j, 2j+1), weight sigmoid(s_t)
        if (lane < (T + 1) / 2) {
            const int j = lane;
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
        if (lane < T) hsel[lane * (top_k + 1) + top_k] = 2 * (n_routed + lane / 2) + (lane & 1);
        if (lane == 0) items[0] = n_routed + (T + 1) / 2;
    }
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
// rows (rows 2i+1); h[item][b][8g + i] = silu(gate) * up.  NORM 1 or 2: the token
// rows are RMS-normalised on the way in (gain gamma, eps), as in the
// normalising GEMV.
//
// RMPL > 0 (a single token, E <= 64 * RMPL): no routing launch precedes the
// kernel; the items are the token's top_k experts in order, then the shared
// expert, and workgroup column j routes the token itself (one wave, the
// routing launch's per-token rounds, only those up to slot j) to find its
// expert; workgroup (0, 0)
// also writes the routing records the down kernel reads (items, hsel), the
// same records the routing launch writes for one token.
template <int F, int W, int KCS, int NORM, int RMPL>
__global__ void __launch_bounds__(W * 64)
moe_gate_up_kernel(const uint8_t* __restrict__ wgu, size_t expert_bytes, size_t codes_bytes, int H, int I,
                   const float* __restrict__ x, const float* __restrict__ gamma, float eps,
                   int* __restrict__ items, float* __restrict__ h, const float* __restrict__ logits,
                   const float* __restrict__ shared_logit, int E, int top_k, unsigned flags,
                   int* __restrict__ hsel) {
    const int j = blockIdx.y;
    Item it;
    if constexpr (RMPL > 0) {
        __shared__ int route_e[kMaxTopK];
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        it.expert = E;  // slot top_k: the shared expert, no routing needed
        if (j < top_k) {  // uniform across the workgroup
            if (wave == 0) {
                int my_e;
                float my_w, sg;
                if (blockIdx.x == 0 && j == 0) {
                    route_token<RMPL>(logits, shared_logit[0], E, top_k, flags, lane, my_e, my_w, sg);
                } else {
                    // only slot j's expert is needed here: rounds 0 .. j, no weights
                    float v[RMPL], my_v;
                    load_logits<RMPL>(logits, E, lane, v);
                    top_rounds<RMPL>(v, j + 1, lane, my_e, my_v);
                }
                if (lane < top_k) route_e[lane] = my_e;
                if (blockIdx.x == 0 && j == 0) {
                    // one token: item k is slot k's expert, then the shared one
                    if (lane <= top_k) {
                        int* rec = items + kItemInts * (1 + lane);
                        rec[0] = lane < top_k ? my_e : E;
                        rec[1] = 1;
                        rec[2] = rec[3] = 0;
                        rec[4] = rec[5] = lane;
                        rec[6] = __float_as_int(lane < top_k ? my_w : sg);
                        rec[7] = 0;
                        hsel[lane] = 2 * lane;
                    }
                    if (lane == 0) items[0] = top_k + 1;
                }
            }
            __syncthreads();
            it.expert = route_e[j];
        }
        it.count = 1;
        it.tok[0] = it.tok[1] = 0;
        it.kslot[0] = it.kslot[1] = j;
        it.wt[0] = it.wt[1] = 0.0f;
    } else {
        if (j >= items[0]) return;  // uniform: unused item slot
        it = read_item(items, j);
    }
    const uint8_t* codes = wgu + (size_t)it.expert * expert_bytes;
    const uint8_t* meta = codes + codes_bytes;
    const int g = blockIdx.x;
    float* hj = h + (size_t)j * 2 * I;
    auto xrow = [&](int b) { return x + (size_t)it.tok[b] * H; };
    auto epi = [&](int B) {
        return [=](auto sums, int, int tid) {
            for (int t = tid; t < 8 * B; t += W * 64) {
                const int i = t / B, b = t % B;
                if (b < it.count) hj[(size_t)b * I + 8 * g + i] = silu(sums((2 * i) * B + b)) * sums((2 * i + 1) * B + b);
            }
        };
    };
    if constexpr (NORM != 0) {
        if (it.count == 1)
            GemvDpp<F, 1, W, KCS>::template run_rmsnorm<NORM == 1>(codes, meta, 2 * I, H, g, xrow, 1, gamma, eps, epi(1));
        else
            GemvDpp<F, 2, W, KCS>::template run_rmsnorm<NORM == 1>(codes, meta, 2 * I, H, g, xrow, 2, gamma, eps, epi(2));
    } else {
        if (it.count == 1) GemvDpp<F, 1, W, KCS>::run(codes, meta, 2 * I, H, g, xrow, 1, epi(1));
        else GemvDpp<F, 2, W, KCS>::run(codes, meta, 2 * I, H, g, xrow, 2, epi(2));
    }
}

// down + combine: one workgroup per 16-row group g and token t, or per g and a
// run of tokens taken TP at a time (t0 = TP * blockIdx.y, then TP * gridDim.y
// further, the LDS arrays reused after a barrier).  Its waves form TP x
// (top_k + 1) groups of WD waves; group (u, s) runs the down projection of
// token t0 + u's slot s (the K routed experts, then the shared one) on its h
// row and scales it by the slot's weight; then out = residual + the slot sums
// in slot order, per token.  A token pair sharing an item reads that expert's
// down rows twice, but no partial leaves the workgroup.
template <int F, int WD, int KCS, int TP>
__global__ void __launch_bounds__(1024)
moe_down_kernel(const uint8_t* __restrict__ wdn, size_t expert_bytes, size_t codes_bytes, int H, int I, int T,
                int top_k, const int* __restrict__ items, const int* __restrict__ hsel,
                const float* __restrict__ h, const float* __restrict__ residual, float* __restrict__ out) {
    __shared__ float red[TP][kMaxTopK + 1][WD * kRowGroup];
    __shared__ float slot_sum[TP][kMaxTopK + 1][kRowGroup];
    const int g = blockIdx.x;
    const int grp = threadIdx.x / (64 * WD);  // wave group, uniform per wave
    const int tp = TP == 1 ? 0 : grp / (top_k + 1), s = grp - tp * (top_k + 1);
    // TP tokens at a time: t0 = TP * blockIdx.y, then TP * gridDim.y further (uniform loop)
    for (int t0 = TP * blockIdx.y; t0 < T; t0 += TP * gridDim.y) {
        // a group past the last token runs the GEMV over an empty column range
        // (no loads; every group must run it: it synchronizes the workgroup),
        // its sums unused
        const bool live = TP == 1 || t0 + tp < T;
        const int t = TP == 1 ? t0 : min(t0 + tp, T - 1);
        const int hs = hsel[t * (top_k + 1) + s];
        const int* it = items + kItemInts * (1 + (hs >> 1));
        const float wt = __int_as_float(it[6 + (hs & 1)]);
        const uint8_t* codes = wdn + (size_t)it[0] * expert_bytes;
        const uint8_t* meta = codes + codes_bytes;
        const float* xr = h + (size_t)hs * I;
        GemvDpp<F, 1, WD, KCS>::run_group(
            codes, meta, H, I, g, [&](int) { return xr; }, 1,
            [&](auto sum, int, int tid) {
                if (tid < kRowGroup) slot_sum[tp][s][tid] = wt * sum(tid);
            },
            grp * WD, &red[tp][s][0], nullptr, 0.0f, nullptr, 0, live ? -1 : 0);
        __syncthreads();
        if (threadIdx.x < TP * kRowGroup) {
            const int u = TP == 1 ? 0 : threadIdx.x / kRowGroup, r = threadIdx.x - u * kRowGroup;
            if (TP == 1 || t0 + u < T) {
                const size_t o = (size_t)(t0 + u) * H + (size_t)kRowGroup * g + r;
                float v = residual[o];
                for (int k = 0; k <= top_k; ++k) v += slot_sum[u][k][r];
                out[o] = v;
            }
        }
        __syncthreads();  // red and slot_sum are reused by the next tokens
    }
}

// ------------------------------------------------------------- launchers

template <int F, int W, int KCS, int NORM, int RMPL>
hipError_t launch_gate_up_w(const uint8_t* wgu, int H, int I, const float* x, const float* gamma, float eps,
                            int* items, float* h, int max_items, const float* logits, const float* slogit, int E,
                            int top_k, unsigned flags, int* hsel, hipStream_t st) {
    const size_t eb = qg_packed_size(F, 2 * (int64_t)I, H), cb = qg_codes_plane_size(F, 2 * (int64_t)I, H);
    hipLaunchKernelGGL((moe_gate_up_kernel<F, W, KCS, NORM, RMPL>), dim3(2 * I / kRowGroup, max_items), dim3(W * 64),
                       0, st, wgu, eb, cb, H, I, x, gamma, eps, items, h, logits, slogit, E, top_k, flags, hsel);
    return hipGetLastError();
}

template <int F, int KCS, int NORM, int RMPL>
hipError_t launch_gate_up(const uint8_t* wgu, int H, int I, const float* x, const float* gamma, float eps, int* items,
                          float* h, int max_items, const float* logits, const float* slogit, int E, int top_k,
                          unsigned flags, int* hsel, hipStream_t st) {
    switch (pick_waves_dpp<F, KCS>(H)) {
        case 1: return launch_gate_up_w<F, 1, KCS, NORM, RMPL>(wgu, H, I, x, gamma, eps, items, h, max_items, logits,
                                                               slogit, E, top_k, flags, hsel, st);
        case 2: return launch_gate_up_w<F, 2, KCS, NORM, RMPL>(wgu, H, I, x, gamma, eps, items, h, max_items, logits,
                                                               slogit, E, top_k, flags, hsel, st);
        case 4: return launch_gate_up_w<F, 4, KCS, NORM, RMPL>(wgu, H, I, x, gamma, eps, items, h, max_items, logits,
                                                               slogit, E, top_k, flags, hsel, st);
        case 8: return launch_gate_up_w<F, 8, KCS, NORM, RMPL>(wgu, H, I, x, gamma, eps, items, h, max_items, logits,
                                                               slogit, E, top_k, flags, hsel, st);
        default: return launch_gate_up_w<F, 16, KCS, NORM, RMPL>(wgu, H, I, x, gamma, eps, items, h, max_items,
                                                                 logits, slogit, E, top_k, flags, hsel, st);
    }
}

template <int F, int WD, int KCS, int TP = 1>
hipError_t launch_down_w(const uint8_t* wdn, int H, int I, int top_k, int T, const int* items, const int* hsel,
                         const float* h, const float* residual, float* out, hipStream_t st, int ty = 0) {
    const size_t eb = qg_packed_size(F, H, I), cb = qg_codes_plane_size(F, H, I);
    if (ty <= 0) ty = down_token_groups<F>(T);
    hipLaunchKernelGGL((moe_down_kernel<F, WD, KCS, TP>), dim3(H / kRowGroup, ty), dim3(TP * (top_k + 1) * WD * 64), 0,
                       st, wdn, eb, cb, H, I, T, top_k, items, hsel, h, residual, out);
    return hipGetLastError();
}

template <int MPL>
hipError_t launch_route(const float* logits, const float* slogit, int T, int E, int top_k, unsigned flags,
                        int* items, int* hsel, hipStream_t st) {
    hipLaunchKernelGGL(moe_route_kernel<MPL>, dim3(1), dim3(512), 0, st, logits, slogit, T, E, top_k, flags, items,
                       hsel);
    return hipGetLastError();
}

template <int F, int NORM>
hipError_t launch_moe(const uint8_t* wgu, const uint8_t* wdn, int E, int H, int I, int top_k, const float* x,
                      const float* gamma, float eps, const float* residual, const float* logits,
                      const float* slogit, int T, unsigned flags, float* out, uint8_t* ws, hipStream_t st) {
    // register-x GEMVs (items carry at most 2 tokens)
    constexpr int KCS = dpp_lane_units<F, 2>();
    // gate/up from two tokens up: lane parts twice as wide where the format
    // allows (Q4_K: half the waves, 9 KB in flight per wave).  Layer at T = 2 /
    // 4 / 8: 22.8 / 34.6 / 57.7 us against 23.2 / 36.4 / 61.1 (same machine);
    // a single token measured 12.57 against 12.33 us and keeps the usual width.
    constexpr int KGU = 2 * KCS <= 8 && dpp_units_ok<F>(2 * KCS) ? 2 * KCS : KCS;
    static_assert(dpp_max_batch<F>() >= 2, "two tokens per item");
    const MoeLayout L(T, H, I, top_k);
    int* items = reinterpret_cast<int*>(ws + L.items);
    int* hsel = reinterpret_cast<int*>(ws + L.hsel);
    float* h = reinterpret_cast<float*>(ws + L.h);
    hipError_t e;
    if (T == 1 && E <= kRouteInGateUpMaxE) {
        // one token: the gate/up workgroups route it themselves (no routing launch)
        e = launch_gate_up<F, KCS, NORM, kRouteInGateUpMaxE / 64>(wgu, H, I, x, gamma, eps, items, h, L.max_items,
                                                                 logits, slogit, E, top_k, flags, hsel, st);
    } else {
        if (E <= 64) e = launch_route<1>(logits, slogit, T, E, top_k, flags, items, hsel, st);
        else if (E <= 128) e = launch_route<2>(logits, slogit, T, E, top_k, flags, items, hsel, st);
        else if (E <= 256) e = launch_route<4>(logits, slogit, T, E, top_k, flags, items, hsel, st);
        else if (E <= 512) e = launch_route<8>(logits, slogit, T, E, top_k, flags, items, hsel, st);
        else if (E <= 1024) e = launch_route<16>(logits, slogit, T, E, top_k, flags, items, hsel, st);
        else if (E <= 2048) e = launch_route<32>(logits, slogit, T, E, top_k, flags, items, hsel, st);
        else e = launch_route<64>(logits, slogit, T, E, top_k, flags, items, hsel, st);
        if (e != hipSuccess) return e;
        e = launch_gate_up<F, KGU, NORM, 0>(wgu, H, I, x, gamma, eps, items, h, L.max_items, logits, slogit, E, top_k,
                                            flags, hsel, st);
    }
    if (e != hipSuccess) return e;
    // down from two tokens up: two or three tokens at a time, each slot's row
    // in one wave of the widest lane parts (Q4_K at I = 1024: 9 KB in flight
    // per wave instead of 4.6 KB), the tokens' slot groups side by side in one
    // workgroup per row group, which takes them in turn.  Three at a time
    // where that takes fewer rounds than two (a last round may hold an idle
    // group), two where the rounds tie.  Two against one at T = 2 / 4 / 6 / 8:
    // layer 23.2 / 36.9 / 49.1 / 60.5 us against 24.4 / 39.2 / 52.4 / 64.7;
    // three against the choice before it at T = 3 / 5 / 6 / 7 / 8: 27.4 /
    // 40.7 / 44.0 / 53.3 / 56.6 us against 30.1 / 43.5 / 46.1 / 55.7 / 57.2,
    // and 37.2 against 34.4 us at T = 4 (same-machine A/B runs).  Odd T
    // without room for three slot groups keeps one token at a time.
    // (the gate/up's width: Q4_K twice the usual, Q2_K the usual; for Q2_K
    // at T = 3 / 6 / 8: 24.8 / 39.7 / 50.2 us against 25.4 / 41.7 / 52.4 one
    // token at a time, T = 2, 4, 5, 7 within 1 %)
    constexpr int KW = KGU;
    if constexpr (KW <= 8 && dpp_units_ok<F>(KW)) {
        if (T >= 2 && pick_waves_dpp<F, KW>(I) == 1) {
            if (T >= 3 && 3 * (top_k + 1) <= 16 && (T + 2) / 3 < (T + 1) / 2)
                return launch_down_w<F, 1, KW, 3>(wdn, H, I, top_k, T, items, hsel, h, residual, out, st, 1);
            if (T % 2 == 0 && 2 * (top_k + 1) <= 16)
                return launch_down_w<F, 1, KW, 2>(wdn, H, I, top_k, T, items, hsel, h, residual, out, st, 1);
        }
    }
    // down: where a slot would get one wave, half-width lane parts give it
    // two (Q2_K, I = 1024: single-token layer 12.4 -> 11.9 us, T = 8 equal)
    if constexpr (KCS >= 2 && dpp_units_ok<F>(KCS / 2)) {
        if (pick_waves_dpp<F, KCS>(I) == 1 && pick_waves_dpp<F, KCS / 2>(I) >= 2 && 2 * (top_k + 1) <= 16)
            return launch_down_w<F, 2, KCS / 2>(wdn, H, I, top_k, T, items, hsel, h, residual, out, st);
    }
    // down waves per slot: what the row needs, within 16 waves for top_k + 1 slots
    int wd = pick_waves_dpp<F, KCS>(I);
    while (wd > 1 && (top_k + 1) * wd > 16) wd /= 2;
    switch (wd) {
        case 1: return launch_down_w<F, 1, KCS>(wdn, H, I, top_k, T, items, hsel, h, residual, out, st);
        case 2: return launch_down_w<F, 2, KCS>(wdn, H, I, top_k, T, items, hsel, h, residual, out, st);
        case 4: return launch_down_w<F, 4, KCS>(wdn, H, I, top_k, T, items, hsel, h, residual, out, st);
        default: return launch_down_w<F, 8, KCS>(wdn, H, I, top_k, T, items, hsel, h, residual, out, st);
    }
}

// ------------------------------------------- no-allocation workspace
//
// moe_expert_ffn_noalloc takes its workspace from the file-scope device array
// `scratch` (top of this file) instead of a caller buffer.  In host code that
// name is a host-side stand-in, not device memory: host code uses only the
// address hipGetSymbolAddress returns for the current device (each device
// holds its own copy of the array at its own address), resolved once per
// device.
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];  // per device; guarded by scratch_mu

// The current device's scratch address, resolving it on the first call on
// that device; QG_OK or QG_EHIP with the detail recorded.
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QG_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(QG_EUNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(QG_EHIP, "hipGetSymbolAddress of the MoE scratch failed: %s", hipGetErrorString(e));
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return QG_OK;
}

}  // namespace
}  // namespace qg

using namespace qg;

extern "C" {

size_t moe_expert_ffn_workspace_size(int T, int E, int H, int I, int top_k) {
    if (T < 1 || T > kMaxT || E < 1 || E > kMaxE || H < 256 || I < 256 || H % 256 || I % 256 ||
        H > (1 << 26) || I > (1 << 26) || top_k < 1 ||
        top_k > kMaxTopK || top_k > E)
        return 0;
    return MoeLayout(T, H, I, top_k).total;
}

int moe_expert_ffn_workspace_layout(int T, int E, int H, int I, int top_k, size_t* hsel_offset, size_t* h_offset) {
    clear_error();
    if (!hsel_offset || !h_offset) return fail(QG_EINVAL, "null offset pointer");
    if (moe_expert_ffn_workspace_size(T, E, H, I, top_k) == 0)
        return fail(QG_ERANGE, "T=%d E=%d H=%d I=%d top_k=%d is not a valid layer", T, E, H, I, top_k);
    const MoeLayout L(T, H, I, top_k);
    *hsel_offset = L.hsel;
    *h_offset = L.h;
    return QG_OK;
}

}  // extern "C"

namespace {

// Host validation shared by the MoE entry points (QG_OK or the error set):
// the layer's shape and its caller buffers, then the workspace.
int check_moe_layer(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k,
                    const float* x, const float* residual, const float* router_logits,
                    const float* shared_gate_logit, int T, unsigned flags, float* out) {
    if (fmt != QG_Q4_K && fmt != QG_Q2_K) return fail(QG_EINVAL, "moe_expert_ffn takes Q4_K or Q2_K experts");
    if (!w_gate_up || !w_down || !x || !residual || !router_logits || !shared_gate_logit || !out)
        return fail(QG_EINVAL, "null pointer");
    if (T < 1 || T > kMaxT) return fail(QG_ERANGE, "T=%d must be in [1, %d]", T, kMaxT);
    if (E < 1 || E > kMaxE) return fail(QG_ERANGE, "E=%d must be in [1, %d]", E, kMaxE);
    if (top_k < 1 || top_k > kMaxTopK || top_k > E)
        return fail(QG_ERANGE, "top_k=%d must be in [1, min(E, %d)]", top_k, kMaxTopK);
    if (H < 256 || H % 256 || I < 256 || I % 256 || H > (1 << 26) || I > (1 << 26))
        return fail(QG_ESHAPE, "H=%d and I=%d must be multiples of 256 in [256, 2^26]", H, I);
    if (flags & ~QG_MOE_RENORM) return fail(QG_EINVAL, "unknown flags 0x%x", flags);
    if (!aligned(w_gate_up, 16) || !aligned(w_down, 16) || !aligned(x, 16))
        return fail(QG_EALIGN, "weights and x must be 16-byte aligned");
    if (!aligned(residual, 4) || !aligned(router_logits, 4) || !aligned(shared_gate_logit, 4) || !aligned(out, 4))
        return fail(QG_EALIGN, "residual, logits and out must be 4-byte aligned");
    const size_t act = (size_t)T * H * 4;
    if (overlap(out, act, x, act) || overlap(out, act, residual, act))
        return fail(QG_EINVAL, "out must not overlap x or residual");
    return QG_OK;
}

int check_moe_workspace(int E, int H, int I, int top_k, const float* x, const float* residual,
                        const float* router_logits, const float* shared_gate_logit, int T, float* out,
                        void* workspace, size_t ws_bytes) {
    if (!workspace) return fail(QG_EINVAL, "null workspace");
    if (!aligned(workspace, 16)) return fail(QG_EALIGN, "the workspace must be 16-byte aligned");
    const size_t need = MoeLayout(T, H, I, top_k).total;
    if (ws_bytes < need) return fail(QG_ERANGE, "workspace of %zu bytes is below the %zu needed", ws_bytes, need);
    const size_t act = (size_t)T * H * 4;
    if (overlap(workspace, need, x, act) || overlap(workspace, need, residual, act) ||
        overlap(workspace, need, out, act) || overlap(workspace, need, router_logits, (size_t)T * E * 4) ||
        overlap(workspace, need, shared_gate_logit, (size_t)T * 4))
        return fail(QG_EINVAL, "workspace must not overlap the inputs or out");
    return QG_OK;
}

int check_moe_args(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k,
                   const float* x, const float* residual, const float* router_logits,
                   const float* shared_gate_logit, int T, unsigned flags, float* out, void* workspace,
                   size_t ws_bytes) {
    const int rc = check_moe_layer(fmt, w_gate_up, w_down, E, H, I, top_k, x, residual, router_logits,
                                   shared_gate_logit, T, flags, out);
    if (rc) return rc;
    return check_moe_workspace(E, H, I, top_k, x, residual, router_logits, shared_gate_logit, T, out, workspace,
                               ws_bytes);
}

// NORM: 0 plain, 1 RMS norm with a gain vector, 2 RMS norm with unit gain
template <int NORM>
int moe_call(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k, const float* x,
             const float* gamma, float eps, const float* residual, const float* router_logits,
             const float* shared_gate_logit, int T, unsigned flags, float* out, void* workspace, void* stream) {
    const uint8_t* wgu = static_cast<const uint8_t*>(w_gate_up);
    const uint8_t* wdn = static_cast<const uint8_t*>(w_down);
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    hipError_t e = fmt == QG_Q4_K
        ? launch_moe<QG_Q4_K, NORM>(wgu, wdn, E, H, I, top_k, x, gamma, eps, residual, router_logits,
                                    shared_gate_logit, T, flags, out, ws, st)
        : launch_moe<QG_Q2_K, NORM>(wgu, wdn, E, H, I, top_k, x, gamma, eps, residual, router_logits,
                                    shared_gate_logit, T, flags, out, ws, st);
    if (e != hipSuccess) return fail(QG_EHIP, "MoE launch failed: %s", hipGetErrorString(e));
    return QG_OK;
}

}  // namespace

extern "C" {

int moe_expert_ffn(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k,
                   const float* x, const float* residual, const float* router_logits,
                   const float* shared_gate_logit, int T, unsigned flags, float* out,
                   void* workspace, size_t ws_bytes, void* stream) {
    clear_error();
    const int rc = check_moe_args(fmt, w_gate_up, w_down, E, H, I, top_k, x, residual, router_logits,
                                  shared_gate_logit, T, flags, out, workspace, ws_bytes);
    if (rc) return rc;
    return moe_call<0>(fmt, w_gate_up, w_down, E, H, I, top_k, x, nullptr, 0.0f, residual, router_logits,
                           shared_gate_logit, T, flags, out, workspace, stream);
}

int moe_expert_ffn_noalloc(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k,
                           const float* x, const float* residual, const float* router_logits,
                           const float* shared_gate_logit, int T, unsigned flags, float* out, void* stream) {
    clear_error();
    int rc = check_moe_layer(fmt, w_gate_up, w_down, E, H, I, top_k, x, residual, router_logits, shared_gate_logit,
                             T, flags, out);
    if (rc) return rc;
    const size_t need = MoeLayout(T, H, I, top_k).total;
    if (need > kNoAllocScratchBytes)
        return fail(QG_ERANGE, "the layer needs %zu bytes of workspace, above the %zu of the no-allocation scratch",
                    need, kNoAllocScratchBytes);
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    rc = check_moe_workspace(E, H, I, top_k, x, residual, router_logits, shared_gate_logit, T, out, ws,
                             kNoAllocScratchBytes);
    if (rc) return rc;
    // every workspace word a kernel reads is written earlier in the same call
    // (routing records, h rows), so the scratch needs no clearing
    return moe_call<0>(fmt, w_gate_up, w_down, E, H, I, top_k, x, nullptr, 0.0f, residual, router_logits,
                       shared_gate_logit, T, flags, out, ws, stream);
}

int moe_expert_ffn_rmsnorm(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k,
                           const float* x, const float* gamma, float eps, const float* residual,
                           const float* router_logits, const float* shared_gate_logit, int T, unsigned flags,
                           float* out, void* workspace, size_t ws_bytes, void* stream) {
    clear_error();
    const int rc = check_moe_args(fmt, w_gate_up, w_down, E, H, I, top_k, x, residual, router_logits,
                                  shared_gate_logit, T, flags, out, workspace, ws_bytes);
    if (rc) return rc;
    if (gamma && !aligned(gamma, 16)) return fail(QG_EALIGN, "gamma must be 16-byte aligned");
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(QG_ERANGE, "eps=%g must be finite and >= 0", (double)eps);
    if (gamma && (overlap(gamma, (size_t)H * 4, out, (size_t)T * H * 4) ||
                  overlap(gamma, (size_t)H * 4, workspace, MoeLayout(T, H, I, top_k).total)))
        return fail(QG_EINVAL, "gamma must not overlap out or the workspace");
    if (!gamma)  // unit gain: the gain folded into the gate/up weights
        return moe_call<2>(fmt, w_gate_up, w_down, E, H, I, top_k, x, gamma, eps, residual, router_logits,
                           shared_gate_logit, T, flags, out, workspace, stream);
    return moe_call<1>(fmt, w_gate_up, w_down, E, H, I, top_k, x, gamma, eps, residual, router_logits,
                       shared_gate_logit, T, flags, out, workspace, stream);
}

}  // extern "C"
