// Routed MoE expert layer (Flash-MoE page, sections "模型架构", "Metal 计算着色器",
// "每层流水线").  Entry points are declared in qgemv.h; kernels follow.
#include <hip/hip_runtime.h>

#include "internal.h"

using namespace qg;

extern "C" {

size_t moe_expert_ffn_workspace_size(int T, int E, int H, int I, int top_k) {
    (void)T; (void)E; (void)H; (void)I; (void)top_k;
    return 0;
}

int moe_expert_ffn(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k,
                   const float* x, const float* residual, const float* router_logits,
                   const float* shared_gate_logit, int T, unsigned flags, float* out,
                   void* workspace, size_t ws_bytes, void* stream) {
    (void)fmt; (void)w_gate_up; (void)w_down; (void)E; (void)H; (void)I; (void)top_k; (void)x;
    (void)residual; (void)router_logits; (void)shared_gate_logit; (void)T; (void)flags; (void)out;
    (void)workspace; (void)ws_bytes; (void)stream;
    clear_error();
    return fail(QG_EUNSUPPORTED, "moe_expert_ffn is not built yet");
}

}  // extern "C"
