/*
 * rq_fp8.h - C ABI of the MI355X (gfx950) W8A8 FP8 linear library.
 *
 * The library computes the FP8 post-training-quantized linear used for OneRec-V2
 * serving.  Page "Quantized Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈",
 * section 关键证据, states the method: weights quantized offline per output channel,
 * activations quantized per token at run time, an FP8 matrix product accumulated in
 * FP32, and the result cast back to FP16 before the next layer; it is applied to the
 * attention q/k/v/o linears, the dense FFN linears and the sparse-MoE expert grouped
 * GEMM.  Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践" fixes the FP8 range at
 * +/-448 (§1.2, i.e. OCP E4M3), sketches the per-token quantizer (§2.2) and shows the
 * FP16 -> quantize -> FP8 GEMM -> dequantize -> FP16 flow (§2.3, Fig. 2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers to row-major, contiguous memory.  FP16 tensors
 *   are IEEE binary16 bit patterns (uint16_t), FP8 tensors are OCP E4M3 bytes, scales
 *   are FP32 dequantization multipliers (value = decode(byte) * scale).
 * - FP16 and FP8 tensor pointers and the workspace must be 16-byte aligned; scale and
 *   index arrays 4-byte aligned.  Otherwise the call returns RQ_ERR_ALIGN.
 * - K and N must be positive multiples of 16 (RQ_ERR_ALIGN otherwise).  Row counts
 *   (M, T, B) may be 0: the call then validates its arguments and enqueues nothing.
 * - Size limits (RQ_ERR_SHAPE beyond them): K <= 2^22 for the linears, and every FP8
 *   operand of one GEMM (activation rows x K, one expert's N x K) below 2^31 bytes.
 * - The caller owns every buffer; the library never allocates device memory.  Scratch
 *   space comes from the caller's workspace, sized by the *_workspace_size calls.
 * - `stream` is a hipStream_t (NULL = the default stream).  All work is enqueued
 *   asynchronously on it; no call synchronizes the host, the ragged MoE row counts
 *   included.  Concurrent calls must use distinct workspaces.
 * - Arguments are validated on the host before anything is enqueued.  On any error
 *   nothing has been enqueued.  A failing kernel launch returns RQ_ERR_HIP.  A device
 *   other than gfx950 returns RQ_ERR_UNSUPPORTED.
 * - Outputs are deterministic (no floating-point atomics): the same inputs give the
 *   same bytes on every run.  Outputs must not alias inputs.
 *
 * Quantization (rq_fp8_quant_weights, and inside the linears): for each row x of
 * length K, amax = max|x_i|, s = fl32(max(amax, 2^-24) / 448) with a correctly rounded
 * FP32 division, q_i = E4M3(fl32(x_i / s)) rounded to nearest even and saturated at
 * +/-448, the sign kept (-0 -> 0x80).
 *
 * Linear: y[m][n] = fl16(fl32(fl32(acc[m][n] * s_x[m]) * s_w[n])) with
 * acc = sum_k decode(x_q[m][k]) * decode(w_q[n][k]) accumulated in FP32, rounded to
 * nearest even.  There is no bias.
 */
#ifndef RQ_FP8_H
#define RQ_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RQ_OK = 0,
  RQ_ERR_NULL = 1,        /* a required pointer is NULL */
  RQ_ERR_SHAPE = 2,       /* a negative or unsupported size, or an unsupported top_k / E */
  RQ_ERR_ALIGN = 3,       /* K or N not a multiple of 16, or a misaligned pointer */
  RQ_ERR_WORKSPACE = 4,   /* workspace smaller than the *_workspace_size result */
  RQ_ERR_UNSUPPORTED = 5, /* the current device is not gfx950 */
  RQ_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed */
  RQ_ERR_ARG = 7,         /* an unknown act / layout / a_fmt / w_gran value, or a missing topk_w */
  RQ_ERR_SCRATCH = 8      /* rq_fp8_linear_noalloc: the call needs more than RQ_STATIC_SCRATCH_BYTES */
} rq_status;

/* Activation applied to the FP16 input rows before they are quantized.
 * RQ_ACT_SILU_MUL: each input row has 2K values [g (K) | u (K)] and the quantized row is
 * h = fl16(silu(g) * u), silu(g) = g / (1 + exp(-g)) evaluated in FP32.  This is the FFN
 * intermediate between the gate/up and down linears. */
enum { RQ_ACT_NONE = 0, RQ_ACT_SILU_MUL = 1, RQ_ACT_GATE_SILU = 2 };

/* RQ_ACT_GATE_SILU is applied to the OUTPUT instead (the input rows are plain [K] rows): the
 * linear's N output columns come in blocks of 32 alternating gate and up features - output
 * columns [64b, 64b + 32) are the gate values of features [32b, 32b + 32) and columns
 * [64b + 32, 64b + 64) their up values (so the weight rows are interleaved the same way) -
 * and the call writes h [rows][N / 2], h[m][32b + i] = fl16(silu(g) * u) of the FP16 linear
 * outputs g = y[m][64b + i], u = y[m][64b + 32 + i], computed in FP32 exactly as
 * RQ_ACT_SILU_MUL computes it.  The FFN intermediate then never exists at full width in
 * memory: its gate/up GEMM writes h, and the down linear takes h with RQ_ACT_NONE.
 * N must be a multiple of 64 (RQ_ERR_ALIGN otherwise). */

/* MoE input rows: one per token (quantized once, before dispatch) or one per routed
 * slot in the canonical permuted order (see rq_fp8_moe_grouped_linear).
 * RQ_MOE_PLAN_READY, OR'ed into RQ_MOE_IN_PERMUTED, skips building the routing plan: the
 * workspace already holds the plan of these same topk_ids (T, top_k, E), written by an
 * earlier call with the same workspace pointer on the same stream - the usual case being the
 * down-projection call of an expert FFN after its gate/up call.  The plan sits at the front
 * of the workspace at offsets that depend only on (T, top_k, E), so pass the larger of the
 * two calls' workspace sizes to both.  A plan that does not belong to the ids gives wrong
 * rows but no out-of-bounds access (every plan value is clamped where it is used).
 * RQ_ERR_ARG with RQ_MOE_IN_TOKENS. */
enum { RQ_MOE_IN_TOKENS = 0, RQ_MOE_IN_PERMUTED = 1, RQ_MOE_PLAN_READY = 4 };

/* MoE output rows: one per routed slot in the canonical permuted order, or one per
 * token after the routing-weighted combine. */
enum { RQ_MOE_OUT_PERMUTED = 0, RQ_MOE_OUT_COMBINED = 1 };

/* Optional debug outputs (device pointers; any field may be NULL).
 * a_q / a_scale: when given, the activation quantizer writes the E4M3 rows and scales
 *   that the GEMM consumes into these buffers instead of the workspace, so they hold
 *   exactly the GEMM's operand: [rows][K] bytes and [rows] floats.
 * h: FP16 [rows][K], the SiLU*up rows (RQ_ACT_SILU_MUL only). */
typedef struct {
  uint8_t* a_q;
  float* a_scale;
  uint16_t* h;
} rq_debug_out;

/* Offline per-output-channel weight quantization (page "Quantized Inference for
 * OneRec-V2", section 关键证据: weights quantized per channel, offline).
 * w [B][N][K] FP16 -> w_q [B][N][K] E4M3, w_scale [B][N] FP32.  Each of the B*N rows is
 * quantized independently with the row quantizer above, so applied to an [M][K]
 * activation matrix it gives exactly the per-token quantization of rq_fp8_linear.
 * Needs no workspace.  Any B, N >= 0; K > 0, K % 16 == 0. */
int rq_fp8_quant_weights(const uint16_t* w, int64_t B, int64_t N, int64_t K,
                         uint8_t* w_q, float* w_scale, void* stream);

/* Bytes of workspace rq_fp8_linear needs for M rows of K quantized values
 * (the quantized activation bytes and scales, each region 256-byte aligned). */
size_t rq_fp8_linear_workspace_size(int64_t M, int64_t K, int act);

/* Bytes of workspace with which rq_fp8_linear (and rq_fp8_linear_ex with per-channel or
 * per-tensor weight scales) may also split K: the quantized activations as above plus, for few
 * rows (M <= 1024, the weight-streaming regime), FP32 partial sums [parts][M][N].  With such a
 * workspace a linear whose 64 x 128 tile count would leave most of the 256 compute units idle
 * cuts K into 2, 4 or 8 equal parts (each at least 2048 bytes of K), runs them as separate
 * work items and adds the parts in a fixed order in a second kernel that applies the
 * epilogue: outputs stay deterministic, and the part count depends only on M, N and K (the
 * gated and the plain gate/up linear sum alike).  With a smaller workspace (at least
 * rq_fp8_linear_workspace_size) the call does not split.  Returns 0 for invalid sizes. */
size_t rq_fp8_linear_workspace_size_ex(int64_t M, int64_t N, int64_t K, int act);

/* W8A8 FP8 linear (pages: "Quantized Inference for OneRec-V2", section 关键证据;
 * "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.3 and Fig. 2).
 * x [M][K] FP16 (or [M][2K] with RQ_ACT_SILU_MUL) is quantized per token into the
 * workspace (or dbg->a_q / dbg->a_scale), multiplied with w_q [N][K] E4M3 and
 * dequantized with w_scale [N] into y [M][N] FP16.
 * With RQ_ACT_GATE_SILU, y is [M][N / 2] (see above).
 * Two kernels on `stream`: the row quantizer, then the FP8 MFMA GEMM with the
 * scale/FP16 epilogue (three with split-K: the GEMM writes FP32 part sums and a reduce kernel
 * applies the epilogue; see rq_fp8_linear_workspace_size_ex).  dbg may be NULL. */
int rq_fp8_linear(const uint16_t* x, int64_t M, int64_t K, int act,
                  const uint8_t* w_q, const float* w_scale, int64_t N,
                  uint16_t* y, void* workspace, size_t workspace_bytes,
                  const rq_debug_out* dbg, void* stream);

/* rq_fp8_linear for callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same operation with act
 * RQ_ACT_NONE, RQ_ACT_SILU_MUL or RQ_ACT_GATE_SILU, E4M3 activations and per-channel weight
 * scales, and the same kernels, but the quantized activation rows and scales live in a
 * static device buffer of RQ_STATIC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends, so the call itself calls no allocator.  The caller still
 * owns x, w_q, w_scale and y.
 * Limit: rq_fp8_linear_workspace_size(M, K, act) <= RQ_STATIC_SCRATCH_BYTES (for example
 * M = 4096 rows of K = 8192), else RQ_ERR_SCRATCH before anything is enqueued.
 * The call splits K as rq_fp8_linear does with a workspace of
 * rq_fp8_linear_workspace_size_ex bytes whenever the partial sums fit in the buffer too.
 * Every call on one GPU shares that GPU's buffer, which keeps the last call's contents (the
 * quantizer rewrites every byte the GEMM then reads, and the GEMM every partial sum the
 * reduce reads, so nothing needs clearing): calls that
 * overlap on one GPU (concurrent streams, or host threads) race on it and must be ordered
 * by the caller.  The buffer's device address is resolved on the first call on each
 * device. */
#define RQ_STATIC_SCRATCH_BYTES (40u << 20)
int rq_fp8_linear_noalloc(const uint16_t* x, int64_t M, int64_t K, int act,
                          const uint8_t* w_q, const float* w_scale, int64_t N,
                          uint16_t* y, void* stream);

/* Bytes of workspace rq_fp8_moe_grouped_linear needs.  E <= 1024, 1 <= top_k <= E.
 * Besides the row counts and widths (T, top_k, E, K) and the input layout and activation,
 * it takes N and out_layout: with RQ_MOE_OUT_COMBINED the permuted GEMM output
 * [T * top_k][N (N / 2 for RQ_ACT_GATE_SILU)] FP16 also lives in the workspace until the
 * combine has read it. */
size_t rq_fp8_moe_workspace_size(int64_t T, int top_k, int64_t E, int64_t N, int64_t K,
                                 int in_layout, int act, int out_layout);

/* Sparse-MoE expert grouped linear (page "Quantized Inference for OneRec-V2", section
 * 关键证据: the MoE grouped GEMM is on the quantized path; page "FP8量化在生成式推荐系统
 * OneRec-V2中的优化实践", §2.1: the routing gate stays FP16, so its top-k result is an
 * input here).
 *
 * Routing: slot j = t * top_k + k of token t goes to expert topk_ids[t][k] (int32,
 * must lie in [0, E)).  The ids live on the device, so the host cannot check them: a
 * routing-plan kernel sets RQ_FLAG_EXPERT_ID in the device error word (rq_debug_flag) for
 * an id outside [0, E) and maps it into that range so that no kernel reads or writes out of
 * bounds; the outputs of that call are then unspecified.  The canonical
 * permuted order sorts the R = T * top_k slots by (expert, j) ascending; expert e owns
 * permuted rows [offset_e, offset_e + count_e).
 *
 * Input rows: RQ_MOE_IN_TOKENS: x [T][K (or 2K)], one row per token, quantized once
 * per token before dispatch; RQ_MOE_IN_PERMUTED: x [R][K (or 2K)] in canonical order.
 * Permuted row r of expert e computes fl16(dequant(A_r . w_q[e]^T)) with w_q [E][N][K]
 * E4M3 and w_scale [E][N].
 * Output: RQ_MOE_OUT_PERMUTED: y [R][N] FP16 in canonical order;
 * RQ_MOE_OUT_COMBINED: y [T][N] = fl16(sum_k fl32(topk_w[t][k] * y_perm[pos(t,k)])),
 * summed in FP32 in slot order, topk_w [T][top_k] FP16 required.
 * With RQ_ACT_GATE_SILU the output rows are N / 2 wide (see above).
 * Experts with no rows read no weights.  A gate/up + SiLU + down expert FFN is two
 * calls: (TOKENS, NONE, PERMUTED) then (PERMUTED, SILU_MUL, COMBINED), or, with gate/up
 * weight rows interleaved in blocks of 32, (TOKENS, GATE_SILU, PERMUTED) then
 * (PERMUTED, NONE, COMBINED).
 * TOKENS rows are quantized once per token and the result is written to each of the
 * token's top_k permuted rows, so the GEMM reads contiguous rows.
 * dbg->a_q / a_scale: R rows in the permuted order (the GEMM operand, for either input
 * layout); dbg->h: one row per input row (T for TOKENS, R for PERMUTED). */
int rq_fp8_moe_grouped_linear(const uint16_t* x, int in_layout, int act,
                              const int32_t* topk_ids, const uint16_t* topk_w,
                              int64_t T, int top_k,
                              const uint8_t* w_q, const float* w_scale,
                              int64_t E, int64_t N, int64_t K,
                              uint16_t* y, int out_layout,
                              void* workspace, size_t workspace_bytes,
                              const rq_debug_out* dbg, void* stream);

/* Weight-scale granularity (page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1 and
 * §2.2, which quantizes the attention projections per output channel, the dense FFN
 * weights per tensor and the MoE expert weights in 128 x 128 blocks).  Every granularity
 * uses the row formula above over the set of values that shares one scale.  Scale
 * layouts for B (or E) weight matrices [N][K]:
 *   RQ_WSCALE_CHANNEL  [B][N]              one scale per output channel (the default)
 *   RQ_WSCALE_TENSOR   [B]                 one scale per matrix
 *   RQ_WSCALE_BLOCK128 [B][N/128][K/128]   one scale per block of 128 output x 128 input
 *                                          channels; N and K must be multiples of 128
 *                                          (RQ_ERR_ALIGN otherwise)
 * With block scales the linear is y[m][n] = fl16(s_x[m] * sum_j S[n/128][j] * P_j[m][n]),
 * P_j the FP32-accumulated product over K block j: the accumulator is kept relative to the
 * current block's scale (multiplied by S[j-1] / S[j] as block j starts), then scaled by
 * s_x[m] and the last block's scale, each in FP32, and rounded to FP16. */
enum { RQ_WSCALE_CHANNEL = 0, RQ_WSCALE_TENSOR = 1, RQ_WSCALE_BLOCK128 = 2 };

/* Activation format (page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.2, puts
 * activations in E5M2 and weights in E4M3).  RQ_FP8_E5M2: the run-time quantizer writes OCP
 * E5M2 bytes (5 exponent bits, 2 mantissa bits, largest finite 57344) with the row formula
 * above and 57344 in place of 448 - s = fl32(max(amax, 2^-24) / 57344),
 * q = E5M2(fl32(x / s)), rounded to nearest even and saturated at +/-57344 - and the GEMM
 * multiplies them with the E4M3 weights.  Weights are always E4M3. */
enum { RQ_FP8_E4M3 = 0, RQ_FP8_E5M2 = 1 };

/* Weight byte layout, OR'ed into the w_gran argument of rq_fp8_linear_ex and
 * rq_fp8_moe_grouped_linear_ex.  Without it w_q is [B][N][K] (row layout).  With
 * RQ_WLAYOUT_SLABS w_q holds the same bytes in the slab layout rq_fp8_pack_weights writes;
 * K must be a multiple of 64 (RQ_ERR_ALIGN otherwise).  Results are identical bit for bit to
 * those of the row layout: only the addresses at which the GEMM finds the bytes change.  The
 * scales keep their layout. */
enum { RQ_WLAYOUT_SLABS = 0x100 };

/* Offline repacking of quantized weights for the GEMM (a layout of this library; the pages fix
 * none beyond one E4M3 byte per weight).  The GEMM streams each tile's weights as slabs of
 * 128 or 256 rows x 64 K bytes; in the row layout such a slab is 64-byte pieces K bytes apart,
 * which HBM streams markedly slower than a contiguous run.  The slab layout of each of the B
 * matrices [N][K] is [K / 64][N][64]: the 64-byte K slab s of every row, rows in order, then
 * slab s + 1; byte (b, n, k) lands at b * N * K + (k / 64) * 64 * N + 64 * n + k % 64.
 * w_q [B][N][K] -> w_packed, B * N * K bytes, a separate buffer (RQ_ERR_ARG if the two are
 * the same); any B, N >= 0; K > 0 with K % 64 == 0 (RQ_ERR_ALIGN); both pointers 16-byte
 * aligned.  One kernel on `stream`; no workspace. */
int rq_fp8_pack_weights(const uint8_t* w_q, int64_t B, int64_t N, int64_t K, uint8_t* w_packed,
                        void* stream);

/* rq_fp8_quant_weights with the weight-scale granularity w_gran (layouts above).
 * RQ_ERR_ARG for an unknown w_gran.  Per-tensor scales take four short kernels (amax words
 * are kept in w_scale until the last one writes the scales). */
int rq_fp8_quant_weights_ex(const uint16_t* w, int64_t B, int64_t N, int64_t K, int w_gran,
                            uint8_t* w_q, float* w_scale, void* stream);

/* rq_fp8_linear with activations quantized to a_fmt (RQ_FP8_*; dbg->a_q then holds bytes of
 * that format) and weights quantized at granularity w_gran; w_scale has that layout (B = 1).
 * w_gran may carry RQ_WLAYOUT_SLABS (w_q in the slab layout).
 * rq_fp8_linear is this call with RQ_FP8_E4M3 and RQ_WSCALE_CHANNEL.  RQ_ERR_ARG for an
 * unknown a_fmt or w_gran. */
int rq_fp8_linear_ex(const uint16_t* x, int64_t M, int64_t K, int act, int a_fmt,
                     const uint8_t* w_q, const float* w_scale, int w_gran, int64_t N,
                     uint16_t* y, void* workspace, size_t workspace_bytes,
                     const rq_debug_out* dbg, void* stream);

/* rq_fp8_moe_grouped_linear with activations quantized to a_fmt and expert weights quantized
 * at granularity w_gran; w_scale has that layout with B = E.  w_gran may carry
 * RQ_WLAYOUT_SLABS (w_q in the slab layout, B = E).  rq_fp8_moe_grouped_linear is
 * this call with RQ_FP8_E4M3 and RQ_WSCALE_CHANNEL.  The workspace size depends on neither. */
int rq_fp8_moe_grouped_linear_ex(const uint16_t* x, int in_layout, int act, int a_fmt,
                                 const int32_t* topk_ids, const uint16_t* topk_w,
                                 int64_t T, int top_k,
                                 const uint8_t* w_q, const float* w_scale, int w_gran,
                                 int64_t E, int64_t N, int64_t K,
                                 uint16_t* y, int out_layout,
                                 void* workspace, size_t workspace_bytes,
                                 const rq_debug_out* dbg, void* stream);

/* MoE router (page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1: the routing gate
 * stays FP16 and its top-k result is the input of the grouped GEMM above).
 * x [T][K] FP16 token rows, w_gate [E][K] FP16 gate weights.  For each token:
 *   logit[e] = sum_k x[k] * w_gate[e][k]   (FP16 products, FP32 accumulation, any order)
 *   topk_ids[t][0..top_k)                  the top_k experts by logit, larger first, equal
 *                                          logits to the lower expert index (int32)
 *   topk_w[t][i] = fl16(exp(l_i - l_0) / sum_j exp(l_j - l_0))  over the selected logits,
 *                                          computed in FP32 (FP16 out)
 *   logits (optional, may be NULL)         the FP32 logits [T][E] the selection used.
 * topk_ids and topk_w are exactly the inputs rq_fp8_moe_grouped_linear takes.
 * Limits: 1 <= E <= 32, 1 <= top_k <= min(E, 4) (RQ_ERR_SHAPE), K a multiple of 64
 * (RQ_ERR_ALIGN).  One kernel on `stream`; no workspace. */
int rq_moe_router_topk(const uint16_t* x, int64_t T, int64_t K, const uint16_t* w_gate, int64_t E,
                       int top_k, int32_t* topk_ids, uint16_t* topk_w, float* logits, void* stream);

/* Short-context attention core between the QKV and O linears (page "FP8量化在生成式推荐系统
 * OneRec-V2中的优化实践", §3.2: short serving contexts; the core stays FP16, page "Quantized
 * Inference for OneRec-V2", section 关键证据, quantizes only the linears).
 * qkv [requests * length][3 * hidden] FP16: each row is [q | k | v] (the merged QKV linear's
 * output), hidden = heads * head_dim, head h owning columns [h * head_dim, (h + 1) * head_dim)
 * of each part.  Requests are `length` consecutive rows; position i attends causally to
 * positions j <= i of its own request:
 *   s_ij = q_i . k_j / sqrt(head_dim) (FP16 products, FP32 accumulation),
 *   p_ij = softmax_j(s_ij) in FP32,  out_i = fl16(sum_j fl16(p_ij) v_j), FP32 accumulation.
 * out [requests * length][hidden] FP16 (the O linear's input).
 * Limits: 1 <= length <= 32 and head_dim == 128 (RQ_ERR_SHAPE).  One kernel on `stream`. */
int rq_attention_core(const uint16_t* qkv, int64_t requests, int length, int heads, int head_dim,
                      uint16_t* out, void* stream);

/* Batched top-k of FP16 candidate rows, for beam search (page "FP8量化在生成式推荐系统OneRec-V2
 * 中的优化实践", §3.2: a RadixSelect TopK run batched with zero copies; §5.3: TopK results kept
 * in FP16).  scores [rows][n] FP16.  For each row the k candidates ranked first by score -
 * larger first in the IEEE total order (-0 below +0), equal scores ranking the lower index
 * first - go to idx [rows][k] (int32 indices into the row) and vals [rows][k] (their FP16
 * scores), in rank order.  The result is unique, so it is exact.  NaN scores are outside the
 * contract.  Limits: 1 <= k <= min(n, 1024), n <= 2^31 - 1, rows <= 65535 (RQ_ERR_SHAPE).
 * A radix select over the 16-bit score keys in 16384-score segments, one workgroup each;
 * rows longer than one segment run in stages through the workspace (a segment's top k holds
 * every member of the row's top k that lies in it).  The workspace (16-byte aligned) must
 * hold rq_topk_workspace_size bytes (0 when n <= 16384). */
size_t rq_topk_workspace_size(int64_t rows, int64_t n, int k);
int rq_topk(const uint16_t* scores, int64_t rows, int64_t n, int k, int32_t* idx, uint16_t* vals,
            void* workspace, size_t workspace_bytes, void* stream);

/* Kernel-level timing for benchmarks and profilers.  After this call, the next kernel
 * of the given kind that the calling thread enqueues (through any entry point above) is
 * bracketed by hipEventRecord(start_event) just before its launch and
 * hipEventRecord(stop_event) just after it, on the stream it is launched on; the hook
 * then disarms itself.  start_event / stop_event are hipEvent_t handles owned by the
 * caller; passing NULL for both disarms the hook.  Each kind has its own one-shot slot.
 * Returns RQ_ERR_ARG for an unknown kind and RQ_ERR_NULL if only one event is NULL. */
enum {
  RQ_KERNEL_QUANT = 0,
  RQ_KERNEL_GEMM = 1,
  RQ_KERNEL_COMBINE = 2,
  RQ_KERNEL_ROUTER = 3,
  RQ_KERNEL_ATTENTION = 4,
  RQ_KERNEL_TOPK = 5,     /* all kernels of one rq_topk call (every stage) */
  RQ_KERNEL_KINDS = 6
};
int rq_time_next_kernel(int kernel, void* start_event, void* stop_event);

/* Device error word (one per GPU).  Bits: */
enum { RQ_FLAG_EXPERT_ID = 1 /* a routing id outside [0, E) reached rq_fp8_moe_grouped_linear */ };

/* Diagnostic read of the current device's error word: waits for all work on the device
 * (hipDeviceSynchronize), returns the word (>= 0) and, if `clear` is non-zero, resets it to
 * 0.  Returns -1 if a HIP call fails.  Not meant for the hot path: it blocks the host.
 * The word accumulates over calls until it is cleared. */
int rq_debug_flag(int clear);

/* Static description of a status code ("ok", "null pointer", ...). */
const char* rq_status_string(int status);

/* 1 if `device` is a gfx950 GPU the library can run on, 0 if not, -1 on a HIP error. */
int rq_device_supported(int device);

#ifdef __cplusplus
}
#endif

#endif /* RQ_FP8_H */
