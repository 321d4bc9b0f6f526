/*
 * qgemv.h -- C ABI of the block-quantized decode GEMV library (libqgemv.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  Handbook page "端侧推理：llama.cpp 与 GGUF、MLX、
 * ExecuTorch", section "速度上限：带宽 ÷ 权重字节数" and its self-test answers:
 * at batch-1 decode every output is the dot product of one quantized weight
 * row with the activation vector, y = W x, and every weight is read once per
 * token.  Batch B stacks activation rows: Y[b][n] = sum_k W[n][k] * X[b][k].
 * The block formats are those of the same page, section "GGUF 的量化格式"
 * (Q8_0, Q4_0, Q4_1, Q4_K), plus Q2_K, ternary weights in 2-bit fields,
 * ternary weights packed in base 3 at 1.875 bits per weight, and 1-bit sign
 * weights (with fp16 block scales, or 8-bit per-row affine ones) from the
 * low-bit README page's kernel table, and the
 * Flash-MoE page's 2-bit experts.  The MoE layer follows the Flash-MoE page,
 * sections "模型架构", "Metal 计算着色器" and "每层流水线".
 *
 * Conventions for every function:
 *   - extern "C", returns int: QG_OK (0) or a negative QG_E* code, never
 *     throws, never aborts.  qg_last_error() then holds a thread-local
 *     message for the failing call.
 *   - Arguments are validated on the host before anything is launched; on
 *     a validation error no output is touched.
 *   - Device functions are asynchronous on `stream` (a hipStream_t; NULL is
 *     the null stream).  A launch failure returns QG_EHIP; a fault during
 *     execution surfaces at the caller's next synchronisation.
 *   - All buffers are caller-owned.  The library allocates nothing, keeps no
 *     pointer after returning, and has no global state or environment-driven
 *     behaviour, so it is thread-safe.  Buffers must stay alive until the
 *     stream work that uses them completes.
 *
 * Packed matrix layout (one [N][K] matrix, format f with block size bs):
 *   [codes plane][meta plane], codes plane = N*(K/bs)*code_bytes bytes,
 *   meta plane = N*(K/bs)*meta_bytes bytes; total qg_packed_size() =
 *   N*K*bpw/8 exactly (BIN8: plus its per-row plane below).  Each plane is the row-major image of its rows (row n:
 *   its blocks' code bytes, resp. meta bytes, in block order) interleaved by
 *   groups of 16 rows (the low-bit README page's row repack for dot-product
 *   lanes): group g holds rows 16g .. 16g+n_g-1 (n_g = min(16, N-16g)) and
 *   starts at byte 16*g*row_bytes; within it, 16-byte unit u of row r sits at
 *   (u*n_g + r)*16, and when row_bytes is not a multiple of 16 the rows' short
 *   last units (L = row_bytes % 16 bytes) follow the full units at
 *   full_units*n_g*16 + r*L.
 *     format  bs   code B  meta B  bpw    meta entry
 *     Q8_0    32   32      2       8.5    fp16 d; codes int8
 *     Q4_0    32   16      2       4.5    fp16 d (signed); nibble = code + 8
 *     Q4_1    32   16      4       5.0    fp16 d, fp16 m
 *     Q4_K    256  128     16      4.5    96-bit field of 8 pairs s_j|t_j<<6
 *     Q2_K    256  64      16      2.5      (12 bits each, LSB first), then
 *                                           fp16 d, fp16 dmin
 *     TERN    128  32      2       2.125  fp16 scale; 2-bit field = t + 1
 *     BIN     128  16      2       1.125  fp16 scale; bit 1 = +1, 0 = -1
 *     BIN8    128  16      1       1.0625 scale code c; bits as BIN
 *     TERN3   256  48      12      1.875  4 fp16 scales (one per 64), then a
 *                                           32-bit field of 2-bit codes
 *   TERN3 (the low-bit page's lossless base-3 ternary with a scale per 64
 *   weights, kernel table, ternary Q2_0 row): f = t + 1 as for TERN; for the
 *   64-weight group s of a block, code byte 12s + m (m < 12) is
 *   sum_{l<5} f(64s + 5m + l) * 3^l (<= 242), and f(64s + 60 + l) sits
 *   at bits 2s..2s+1 of byte l of the meta entry's field (bytes 8..11).
 *   BIN8 adds a third plane: the meta plane is zero-padded to a multiple of
 *   16 bytes and followed by N rows of (base, step), two little-endian fp32;
 *   the block scale is fp32(base + fp32(step * c)) (see qpack_bin8).
 *   Nibble i of a block sits in byte i>>1 (low nibble for even i); 2-bit field
 *   i in byte i>>2 at bits 2*(i&3); bit i in byte i>>3 at bit i&7.  All
 *   multi-byte values are little-endian.  Decoded weights:
 *     Q8_0 q*d; Q4_0 (n-8)*d; Q4_1 n*d+m; Q4_K/Q2_K n*(s_j*d) - t_j*dmin;
 *     TERN, TERN3 (f-1)*scale; BIN, BIN8 (2*bit-1)*scale.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QG_Q8_0 = 0,
    QG_Q4_0 = 1,
    QG_Q4_1 = 2,
    QG_Q4_K = 3,
    QG_Q2_K = 4,
    QG_TERN = 5,
    QG_BIN = 6,
    QG_BIN8 = 7,
    QG_TERN3 = 8
} qg_format;

enum {
    QG_OK = 0,
    QG_EINVAL = -1,      /* null pointer, bad enum, non-finite quantizer input */
    QG_ESHAPE = -2,      /* N < 1, K not a positive multiple of the block, ... */
    QG_EALIGN = -3,      /* a pointer misses its required alignment            */
    QG_ERANGE = -4,      /* B out of range, a scale overflowing fp16, ...      */
    QG_EHIP = -5,        /* a HIP launch or runtime call failed                */
    QG_EUNSUPPORTED = -6 /* a valid request the library does not implement     */
};

/* Flags for moe_expert_ffn. */
#define QG_MOE_RENORM 1u /* divide the top-K routing weights by their sum */

/* Largest batch (activation rows) one GEMV call accepts. */
#define QG_MAX_BATCH 8

/* ------------------------------------------------------------------ sizes */

/* Bytes of a packed [N][K] matrix (== N*K*bpw/8), or 0 if the format is
 * unknown, N < 1 or K is not a positive multiple of the block size. */
size_t qg_packed_size(int fmt, int64_t N, int64_t K);

/* Bytes of the codes plane, i.e. the offset of the meta plane (0 if invalid). */
size_t qg_codes_plane_size(int fmt, int64_t N, int64_t K);

/* The same value, named for the layout [codes plane][meta plane]: the byte
 * offset at which the codes plane ends and the meta plane begins (the codes
 * plane itself starts at offset 0).  0 if invalid. */
size_t qg_codes_plane_offset(int fmt, int64_t N, int64_t K);

/* Weights per block (32, 256 or 128; TERN3 256, holding four scale groups
 * of 64) or 0 for an unknown format. */
int qg_block_size(int fmt);

/* ------------------------------------------------------------------- GEMV */

/* Device scratch the GEMV can use, in bytes: S * B * N * 4 when the shape
 * is split along K (S = 4 or 2 pieces of whole 256-column spans, chosen
 * when the row groups times S still fit the device's compute units and the
 * batch is 5 or more, so the launch is VALU-bound on a few compute units --
 * e.g. 1024 x 4096 at batch 8), else 0.  The split follows the handbook
 * page's decode bound ("速度上限：带宽 ÷ 权重字节数"): the bytes are the same,
 * the split only spreads them over more of the chip.  0 also for arguments
 * qgemv rejects. */
size_t qgemv_workspace_size(int fmt, int64_t N, int64_t K, int B);

/* Y[b][n] = sum_k W[n][k] * X[b][k] for b < B, n < N, in fp32 with fp32
 * accumulation (handbook page, "速度上限：带宽 ÷ 权重字节数": y = W x).
 *   w   DEVICE, packed [N][K] matrix of format fmt, 16-byte aligned.
 *   x   DEVICE, fp32 [B][K] row-major, 16-byte aligned.
 *   y   DEVICE, fp32 [B][N] row-major, 4-byte aligned; overwritten; must not
 *       overlap x or w (QG_EINVAL).
 *   1 <= N < 2^31; K a positive multiple of the block size, at most
 *   2^26 (offsets inside a 16-row group are 32-bit);
 *   1 <= B <= 8.
 *   ws  DEVICE scratch of >= qgemv_workspace_size() bytes, 16-byte aligned,
 *       not overlapping w, x or y: the split-K partial sums (two launches:
 *       the pieces, then their fixed-order sum).  NULL, or a smaller
 *       ws_bytes, runs the single-pass kernel instead (same accuracy bound,
 *       its own summation order).  Its contents are scratch.
 * Accuracy: |y - y_exact| <= 2e-5 * sum_k |W[n][k] X[b][k]| + 1e-7, where
 * y_exact is the exact sum over the decoded weights.  Results are
 * deterministic: the same inputs give the same bits on every call.
 * Errors: QG_EINVAL (null w/x/y, unknown fmt; a used ws overlapping w, x or
 * y), QG_ESHAPE, QG_ERANGE (B), QG_EALIGN (also a used ws), QG_EHIP. */
int qgemv(int fmt, const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
          void* ws, size_t ws_bytes, void* stream);

/* The same call with the format fixed by the name. */
int qgemv_q8_0(const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
               void* ws, size_t ws_bytes, void* stream);
int qgemv_q4_0(const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
               void* ws, size_t ws_bytes, void* stream);
int qgemv_q4_1(const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
               void* ws, size_t ws_bytes, void* stream);
int qgemv_q4k(const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
              void* ws, size_t ws_bytes, void* stream);
int qgemv_q2k(const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
              void* ws, size_t ws_bytes, void* stream);
int qgemv_tern(const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
               void* ws, size_t ws_bytes, void* stream);
int qgemv_bin(const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
              void* ws, size_t ws_bytes, void* stream);
int qgemv_bin8(const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
               void* ws, size_t ws_bytes, void* stream);
int qgemv_tern3(const void* w, const float* x, float* y, int64_t N, int64_t K, int B,
                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------- GEMV on normalised x */

/* Y[b][n] = sum_k W[n][k] * xhat[b][k] with the RMS normalisation
 *   xhat[b][k] = X[b][k] * gamma[k] / sqrt(mean_k X[b][k]^2 + eps)
 * of each activation row folded into the GEMV (Flash-MoE page: RMS
 * normalisation in two passes, sum of squares then application, section
 * "Metal 计算着色器"; the norm feeding the next projection on the GPU, section
 * "延迟 GPU 专家计算").  The sum of squares is taken while x is loaded, gamma
 * scales x in registers and 1/rms scales each row sum, so no normalised copy
 * of x is written.
 *   gamma  DEVICE, fp32 [K], 16-byte aligned, not overlapping y; or NULL
 *          for unit gain, when the caller has folded gamma into the weights
 *          (quantizing W * diag(gamma) instead of W): then no gamma is read.
 *   eps    finite, >= 0 (a zero row with eps = 0 gives non-finite y, as the
 *          definition does).
 *   w, x, y, N, K, B, stream: as for qgemv.
 * Accuracy: |error| <= 3e-5 * sum_k |W[n][k] xhat[b][k]| + 1e-7: the qgemv
 * bound on xhat plus the fp32 sum of squares, square root and gamma product.
 * Deterministic.  Errors: as qgemv, plus QG_EALIGN (gamma), QG_EINVAL
 * (gamma overlaps y), QG_ERANGE (eps). */
int qgemv_rmsnorm(int fmt, const void* w, const float* x, const float* gamma, float eps, float* y,
                  int64_t N, int64_t K, int B, void* stream);

/* ----------------------------------------------------------------- dequant */

/* Device dequantization of a packed [N][K] matrix to fp32 out[N][K]
 * (row-major, 4-byte aligned), with the decoded-weight formulas above.
 * Every value is bit-exact: each product is exact in fp32 and the only
 * rounding is Q4_1's "+m" and the K-quants' "-t*dmin".  Same pointer rules
 * and errors as qgemv. */
int qg_dequant(int fmt, const void* w, float* out, int64_t N, int64_t K, void* stream);

/* ------------------------------------------------------ reference quantizer */

/* Host quantizer: fp32 w_host[N][K] (row-major) -> packed bytes in out_host
 * (qg_packed_size() bytes).  Q8_0, Q4_0, Q4_1 follow the handbook page's
 * quantizer listing (section "GGUF 的量化格式"), Q4_K its simplified K-quant,
 * Q2_K the same construction with 2-bit codes; every scale and min is stored
 * as fp16 (round to nearest even) and the codes are computed against the
 * stored values; rounding is half-to-even; a zero scale gives the zero code.
 * Signed zeros in the input are treated as +0.  n_threads <= 0 means 1.
 * Both pointers are HOST memory.  Errors: QG_EINVAL (null, non-finite input,
 * fmt is TERN/BIN/BIN8/TERN3 -- use their qpack_*), QG_ESHAPE, QG_ERANGE (a
 * scale or min overflows fp16).  After QG_EINVAL for a non-finite weight or
 * QG_ERANGE, out_host is unspecified (rows are quantized as they are read). */
int qquant(int fmt, const float* w_host, int64_t N, int64_t K, void* out_host, int n_threads);

/* Device quantizer: the same quantizers as qquant (byte-identical output),
 * run on weights already in device memory.
 *   w       DEVICE fp32 [N][K] row-major, 4-byte aligned.
 *   out     DEVICE, qg_packed_size(fmt, N, K) bytes, 16-byte aligned.
 *   status  DEVICE int, 4-byte aligned: set to QG_OK by the call, then to a
 *           negative code if a block fails on the device -- QG_EINVAL (a
 *           non-finite weight) or QG_ERANGE (a scale or min overflows fp16);
 *           with several failures it holds the smallest code.  The blocks
 *           that fail leave their bytes of out unspecified.
 * w, out and status must not overlap (QG_EINVAL).
 * fmt Q8_0, Q4_0, Q4_1, Q4_K or Q2_K (the 1-bit and ternary formats:
 * QG_EUNSUPPORTED; the
 * pages give no ternarizer or binarizer).  Asynchronous on `stream`; read
 * status after synchronising.  Host errors: QG_EINVAL, QG_ESHAPE, QG_EALIGN,
 * QG_EUNSUPPORTED, QG_EHIP. */
int qquant_device(int fmt, const float* w, int64_t N, int64_t K, void* out, int* status, void* stream);

/* Device re-quantizer: decode a packed src matrix (any format) and quantize
 * it to dst_fmt, as qg_dequant followed by qquant_device -- e.g. 4-bit
 * experts re-quantized to 2 bits, which the Flash-MoE page does offline
 * (sections "性能表现" and "项目结构": its 2-bit experts come from the
 * 4-bit ones).
 *   src        DEVICE packed [N][K] of src_fmt, 16-byte aligned.
 *   dst        DEVICE packed [N][K] of dst_fmt, 16-byte aligned.
 *   workspace  DEVICE scratch of >= qrequant_workspace_size(N, K) bytes
 *              (the decoded fp32 matrix), 16-byte aligned.
 *   status     as for qquant_device.
 * src, dst, workspace and status must not overlap (QG_EINVAL).  Errors: as
 * qg_dequant and qquant_device, plus QG_ERANGE (workspace too small). */
size_t qrequant_workspace_size(int64_t N, int64_t K);
int qrequant(int src_fmt, const void* src, int dst_fmt, void* dst, int64_t N, int64_t K, void* workspace,
             size_t ws_bytes, int* status, void* stream);

/* Host packers for the trained low-bit formats (the pages give no
 * ternarizer/binarizer): t[N][K] int8 in {-1,0,1} or bits[N][K] uint8 in
 * {0,1}, plus scale_f16[N][K/128] fp16 bit patterns -> packed bytes.
 * Errors: QG_EINVAL (null pointer, a code out of range), QG_ESHAPE; every
 * code is checked before any byte of out_host is written. */
int qpack_tern(const int8_t* t, const uint16_t* scale_f16, int64_t N, int64_t K, void* out_host);
int qpack_bin(const uint8_t* bits, const uint16_t* scale_f16, int64_t N, int64_t K, void* out_host);

/* Host packer for QG_TERN3 (layout above): t[N][K] int8 in {-1,0,1} and
 * scale_f16[N][K/64] fp16 bit patterns (one scale per 64 weights) -> packed
 * bytes; lossless (qg_dequant gives t * scale exactly).  K a multiple of 256.
 * Errors: QG_EINVAL (null pointer, a code out of range), QG_ESHAPE. */
int qpack_tern3(const int8_t* t, const uint16_t* scale_f16, int64_t N, int64_t K, void* out_host);

/* Host packer for QG_BIN8, the 1-bit format whose block scales are 8-bit
 * codes of a per-row affine map (low-bit README page, kernel table, the
 * Q1_0 bit-plane row).  Takes the same bits and fp16 block scales as
 * qpack_bin and re-codes each row's scales d_j as
 *   base = min_j d_j, step = (max_j d_j - base) / 255      (fp32),
 *   c_j  = clamp(round_half_even((d_j - base) / step), 0, 255), 0 if step = 0,
 * decoded as d_j' = fp32(base + fp32(step * c_j)).  Layout: the codes plane
 * (as QG_BIN), the meta plane (one byte c_j per 128-weight block, rows
 * interleaved by 16 as usual) zero-padded to a multiple of 16 bytes, then N
 * rows of (base, step) as two little-endian fp32, row-major.
 * Errors: as qpack_bin, plus QG_EINVAL for a non-finite scale. */
int qpack_bin8(const uint8_t* bits, const uint16_t* scale_f16, int64_t N, int64_t K, void* out_host);

/* --------------------------------------------------------------- MoE layer */

/* Routed expert layer for T decode tokens (Flash-MoE page, sections "模型架构",
 * "Metal 计算着色器", "每层流水线"; the routed matmul semantics of the EPM
 * README, section "正確性").  For each token t:
 *   p = softmax(router_logits[t]);  e_1..e_K = the top_k largest p (ties to
 *   the lower expert index);  w_k = p[e_k] (divided by sum_k p[e_k] when
 *   QG_MOE_RENORM is set);  for each selected expert e and the shared expert
 *   (index E): h = silu(W_gate,e x_t) * (W_up,e x_t), o_e = W_down,e h;
 *   out[t] = residual[t] + sum_k w_k o_{e_k} + sigmoid(shared_gate_logit[t]) o_E.
 *   fmt        QG_Q4_K or QG_Q2_K.
 *   w_gate_up  DEVICE, (E+1) consecutive packed [2I][H] matrices whose row 2i
 *              is gate row i and row 2i+1 is up row i; expert E is shared.
 *   w_down     DEVICE, (E+1) consecutive packed [H][I] matrices.
 *   x, residual  DEVICE fp32 [T][H] (residual may alias x); out DEVICE fp32
 *              [T][H] (must not overlap x or residual).
 *   router_logits DEVICE fp32 [T][E]; shared_gate_logit DEVICE fp32 [T].
 *   workspace  DEVICE scratch >= moe_expert_ffn_workspace_size() bytes,
 *              16-byte aligned, overlapping no input and not out.
 *   1 <= T <= 8, 1 <= top_k <= min(E, 8), 1 <= E <= 4096, H and I
 *   multiples of 256 in [256, 2^26].  Deterministic (fixed-order sums, no
 *   float atomics).
 * Errors: QG_EINVAL, QG_ESHAPE, QG_ERANGE, QG_EALIGN, QG_EHIP. */
size_t moe_expert_ffn_workspace_size(int T, int E, int H, int I, int top_k);

/* Where a finished moe_expert_ffn (or moe_expert_ffn_rmsnorm) call leaves its
 * intermediate results in the workspace, for stage-wise checks (EPM README,
 * section "正確性": the SwiGLU intermediate of one implementation fed into the
 * other's down projection localises a difference).  For the same
 * (T, E, H, I, top_k), once the call's stream work has completed:
 *   int32 hsel[T][top_k + 1] at byte *hsel_offset: hsel[t][k] is the h row of
 *     token t's slot k (slots 0..top_k-1: the routed experts in descending
 *     weight; slot top_k: the shared expert);
 *   fp32 h[rows][I] at byte *h_offset: row r holds silu(W_gate x_t) *
 *     (W_up x_t) of the expert and token that r was assigned to.
 * hsel_offset and h_offset are HOST pointers receiving the byte offsets.
 * The contents are scratch: valid only until the workspace is used again.
 * Returns QG_OK, or QG_ERANGE / QG_EINVAL for arguments that
 * moe_expert_ffn_workspace_size rejects (it returns 0 for them). */
int moe_expert_ffn_workspace_layout(int T, int E, int H, int I, int top_k, size_t* hsel_offset, size_t* h_offset);

int moe_expert_ffn(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k,
                   const float* x, const float* residual, const float* router_logits,
                   const float* shared_gate_logit, int T, unsigned flags, float* out,
                   void* workspace, size_t ws_bytes, void* stream);

/* The same layer for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * it takes no workspace argument and allocates nothing.  Its workspace is a
 * library-owned device array of QG_MOE_NOALLOC_SCRATCH_BYTES (2 MiB) per
 * device, held until the process ends; a layer whose
 * moe_expert_ffn_workspace_size exceeds that returns QG_ERANGE.  Every call
 * on one device shares that device's array, so calls that overlap on one
 * device (concurrent streams, or host threads) race and must be serialised
 * by the caller.  Every other argument, the result and the errors are those
 * of moe_expert_ffn (bit-identical output). */
#define QG_MOE_NOALLOC_SCRATCH_BYTES ((size_t)2 << 20)
int moe_expert_ffn_noalloc(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k,
                           const float* x, const float* residual, const float* router_logits,
                           const float* shared_gate_logit, int T, unsigned flags, float* out, void* stream);

/* The same layer fed through an RMS norm: every expert (routed and shared)
 * sees xhat[t][k] = x[t][k] * gamma[k] / sqrt(mean_k x[t][k]^2 + eps)
 * instead of x, the norm folded into the gate/up GEMVs as in qgemv_rmsnorm
 * (Flash-MoE page: the RMS norm's two passes, section "Metal 计算着色器";
 * the norm in the layer's GPU pipeline ahead of routing and the experts,
 * section "每层流水线").  In a pre-norm block residual is the un-normalised
 * x itself (it may alias x); router_logits are the router projection of
 * xhat, e.g. from qgemv_rmsnorm with the same gamma and eps.
 *   gamma  DEVICE fp32 [H], 16-byte aligned, overlapping neither out nor
 *          the workspace; or NULL for unit gain (the gain folded into every
 *          expert's gate/up weights); eps finite, >= 0.
 *   Every other argument as for moe_expert_ffn (same workspace size).
 * Accuracy: the moe_expert_ffn bound with the gate/up GEMV bound widened to
 * 3e-5 * sum_k |W[n][k] xhat[t][k]| + 1e-7 (the qgemv_rmsnorm bound).
 * Errors: as moe_expert_ffn, plus QG_EALIGN (gamma), QG_EINVAL (gamma
 * overlaps out or the workspace), QG_ERANGE (eps). */
int moe_expert_ffn_rmsnorm(int fmt, const void* w_gate_up, const void* w_down, int E, int H, int I, int top_k,
                           const float* x, const float* gamma, float eps, const float* residual,
                           const float* router_logits, const float* shared_gate_logit, int T, unsigned flags,
                           float* out, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ measurement */

/* Streaming-read probe: reads `bytes` bytes of DEVICE memory at `buf` with
 * 128-bit non-temporal loads, the access pattern of the GEMV weight stream,
 * and touches *sink (DEVICE, 4 bytes) only when a data-dependent value that
 * never occurs is met, so the loads cannot be dropped.  It exists to measure
 * the HBM read rate that the GEMV is compared with (the handbook page's
 * decode bound, section "速度上限：带宽 ÷ 权重字节数", divides the weight bytes
 * by that rate).  buf 16-byte aligned, bytes a positive multiple of 16;
 * otherwise QG_EALIGN / QG_ESHAPE.  Asynchronous on `stream`. */
int qg_hbm_read_probe(const void* buf, size_t bytes, unsigned* sink, void* stream);

/* ------------------------------------------------------------------ errors */

/* Static description of an error code. */
const char* qg_strerror(int code);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* qg_last_error(void);
/* Library version string. */
const char* qg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
