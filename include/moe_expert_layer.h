/*
 * moe_expert_layer.h - C ABI of an MI355X (gfx950) library for the forward and backward passes of
 * a Mixture-of-Experts expert layer on one GPU.
 *
 * The layer is the expert part of the EP-MC2 forward on the page "NPU Training Operators - MC2",
 * section 执行路径 (execution path): count slots per expert (step 2), permute token rows into
 * expert-contiguous order (step 6), grouped matmul with the gate/up weights (step 7), SwiGLU
 * (step 8), grouped matmul with the down weights (step 9), and the probs-weighted unpermute
 * (step 10), taken as one device's share with the cross-card All-to-All left out.  The operand set
 * is mc2_fused_expert's on the page "MC2 通算融合" (hwcomputing.csdn.net), section 用法, without
 * the communication group, in the order gate, up, down, plus the routing probabilities of step 10.
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE pointers unless a parameter says "host".  Shapes are row-major and
 *     contiguous; "[A,B]" means A rows of B elements.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns without waiting
 *     for it.  Buffers must stay alive, and must not be written by others, until that work ends.
 *   - The caller allocates and frees all memory, including the workspace, whose size comes from the
 *     matching *_workspace_size call.  The library never allocates device memory in these calls and
 *     keeps no pointer after returning.  One workspace must not serve two calls in flight at once.
 *   - Argument problems that the host can see (null pointers, bad sizes, unsupported dtype, a
 *     workspace that is too small) return an error before anything is enqueued.  Problems only the
 *     device can see (an expert id outside [0, E), a group expert outside [0, E)) are recorded in a
 *     status word at the start of the workspace; moe_query_device_status reads it.  Such slots /
 *     groups are skipped (they contribute nothing), like histc ignoring out-of-range values.
 *   - No C++ exception crosses this interface.  moe_last_error() gives a thread-local message for the
 *     last failing call on the calling thread.
 *
 * Storage formats (moe_problem.dtype):
 *   MOE_F32         float32 x, weights, out; float32 intermediates.
 *   MOE_BF16        bfloat16 x, weights, out; fp32 accumulation; the SwiGLU output h and the
 *                   per-slot expert outputs are rounded to bfloat16 (round to nearest even).
 *   MOE_MXFP8_E4M3  OCP-MX (Microscaling Formats v1.0): E4M3 element bytes with one E8M0 scale byte
 *                   per 32 consecutive elements along the contraction axis; x_scale [T, H/32],
 *                   wg_scale / wu_scale [E, H/32, F], wd_scale [E, F/32, H].  h is MX-encoded the same
 *                   way along F before the down projection.  The output is bfloat16.  The MX format
 *                   is the one named for the reference MC2 matmul on the page
 *                   "MC2 通算融合架构总览", §1.
 */
#ifndef MOE_EXPERT_LAYER_H
#define MOE_EXPERT_LAYER_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,       /* null pointer, non-positive size, k > E, ...            */
    MOE_ERR_UNSUPPORTED = 2,            /* dtype or a size the kernels do not handle              */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_EXPERT_ID_OUT_OF_RANGE = 4, /* device-side: some id was outside [0, E)                */
    MOE_ERR_HIP = 5                     /* a HIP runtime call failed (message in moe_last_error)  */
} moe_status;

enum moe_dtype_code { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8_E4M3 = 2 };

/* moe_problem.flags.  By default the forward calls fold the permute step (a gather of token rows
 * into expert order, "NPU Training Operators - MC2", 执行路径 step 6) into the first grouped GEMM's
 * row loads when the large-tile kernels serve the sizes: those rows are read from x through the slot
 * list and x_perm is never written.  MOE_FLAG_SEPARATE_PERMUTE runs the permute kernel and the GEMM
 * on x_perm instead; the result is bitwise the same either way. */
#define MOE_FLAG_SEPARATE_PERMUTE 1u

/* moe_problem.flags, MX problems only: x is bfloat16 [T,H] and the library encodes it to OCP-MX
 * (E4M3 codes, one E8M0 scale per 32 elements along H, the rule of moe_mx_quantize) on its way into
 * the gather of 执行路径 step 6 ("NPU Training Operators - MC2"; the MX matmul of
 * "MC2 通算融合架构总览", §1): once per token into the workspace when the first grouped GEMM gathers
 * its rows from x itself, or straight into the permuted rows when the permute runs as its own step
 * (MOE_FLAG_SEPARATE_PERMUTE, or sizes the large tiles do not serve).  moe_workspace_size accounts
 * for the token-order buffer; moe_quantized_x_offsets says where the codes are left. */
#define MOE_FLAG_QUANTIZE_X 2u

/* The chunk height that "MC2 通算融合架构总览", §6 (切分策略) uses for its M-axis split: the
 * recommended moe_problem.head_m_size for a chunked call (0 still means unchunked). */
#define MOE_DEFAULT_HEAD_M_SIZE 512

/* Largest H and F the library accepts (MOE_ERR_UNSUPPORTED beyond): the grouped GEMMs address a
 * row tile's operands by 32-bit offsets from the tile's first row. */
#define MOE_MAX_HIDDEN (1 << 22)

typedef struct moe_problem {
    int64_t T;            /* tokens                                                              */
    int64_t H;            /* hidden size                                                         */
    int64_t F;            /* expert feed-forward size                                            */
    int64_t E;            /* experts                                                             */
    int64_t k;            /* experts per token (top-k), 1 <= k <= E                              */
    int32_t dtype;        /* enum moe_dtype_code                                                 */
    int32_t head_m_size;  /* 0: unchunked.  Otherwise the permuted rows are processed in chunks of
                             this many rows (a multiple of 256), in chunk order, and each chunk's
                             completion is counted in the workspace.  The M-axis split and its 512-row
                             default (MOE_DEFAULT_HEAD_M_SIZE, the value to pass for the pages' chunked
                             mode) are those of "MC2 通算融合架构总览", §6 切分策略; the result is
                             bitwise identical to the unchunked one.                              */
    uint32_t flags;       /* 0, or MOE_FLAG_SEPARATE_PERMUTE and / or MOE_FLAG_QUANTIZE_X        */
    uint32_t reserved;    /* must be 0                                                           */
} moe_problem;

/* ---------------------------------------------------------------------------------------------
 * Whole layer.
 * ------------------------------------------------------------------------------------------- */

/* Host only.  Workspace bytes needed by moe_expert_forward / moe_expert_forward_mx for `p`. */
moe_status moe_workspace_size(const moe_problem* p, size_t* bytes /* host */);

/* out[T,H] = sum_j probs[t,j] * FFN_{expert_ids[t,j]}(x[t]),
 *   FFN_e(v) = (silu(v Wg[e]) * (v Wu[e])) Wd[e],   silu(z) = z / (1 + exp(-z)).
 * dtype MOE_F32 or MOE_BF16 (x, weights and out in that dtype).
 *   x          [T,H]           w_gate, w_up [E,H,F]        w_down [E,F,H]
 *   expert_ids [T,k] int32     probs [T,k] float32         out [T,H]
 * Steps (all on `stream`): route, permute, fc1 + SwiGLU, fc2, unpermute.  The k slots of a token
 * are summed in j order with fp32 accumulation and one final rounding; no float atomics, so the
 * output is deterministic. */
moe_status moe_expert_forward(const moe_problem* p, const void* x, const void* w_gate,
                              const void* w_up, const void* w_down, const int32_t* expert_ids,
                              const float* probs, void* out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* moe_expert_forward (dtype MOE_BF16 only) that also keeps what the backward would recompute: the
 * gate and up values g = x Wg[e], u = x Wu[e] of every routed slot, as bfloat16 in
 * saved_gu [2, T*k, F] (g rows, then u rows; row p is the p-th slot in expert order, the row order of
 * moe_route's perm).  Pass saved_gu to moe_expert_backward with the same inputs and routing to skip
 * its recomputation; the gradients are then bitwise those of the recomputing call.  The output is
 * bitwise that of moe_expert_forward.  Workspace: moe_workspace_size. */
moe_status moe_expert_forward_train(const moe_problem* p, const void* x, const void* w_gate,
                                    const void* w_up, const void* w_down, const int32_t* expert_ids,
                                    const float* probs, void* out, void* saved_gu, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* The same layer on OCP-MX E4M3 inputs (dtype must be MOE_MXFP8_E4M3; H and F multiples of 128).
 * Element bytes and scale bytes as described above; out is bfloat16 [T,H].
 * With MOE_FLAG_QUANTIZE_X in p->flags, x points to bfloat16 activations [T,H] instead and x_scale
 * must be NULL: the library encodes x itself (see the flag).  The encoding is bit-exact, so the
 * output is bitwise that of a call on the host-encoded x. */
moe_status moe_expert_forward_mx(const moe_problem* p, const uint8_t* x, const uint8_t* x_scale,
                                 const uint8_t* w_gate, const uint8_t* wg_scale,
                                 const uint8_t* w_up, const uint8_t* wu_scale,
                                 const uint8_t* w_down, const uint8_t* wd_scale,
                                 const int32_t* expert_ids, const float* probs, void* out_bf16,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Backward of the layer.
 * ------------------------------------------------------------------------------------------- */

/* Host only.  Workspace bytes needed by moe_expert_backward for `p`. */
moe_status moe_backward_workspace_size(const moe_problem* p, size_t* bytes /* host */);

/* Gradients of L = sum_{t,h} dout[t,h] * out[t,h] for moe_expert_forward's layer with the same
 * inputs and routing.  The page "NPU Training Operators - MC2" wraps forward and backward of each
 * step of 执行路径 in its fused ops and lists the fc1 / fc2 gradients among its checks (验证项).
 * Per slot s = t*k + j with expert e = expert_ids[t,j], g = x[t] Wg[e], u = x[t] Wu[e],
 * sg = sigmoid(g), h = g sg u (silu(g) u):
 *   dprobs[t,j] = <dout[t], h Wd[e]>
 *   da          = probs[t,j] * dout[t] Wd[e]^T
 *   dg          = da u sg (1 + g (1 - sg)),   du = da g sg
 *   dx[t]       = sum_j (dg Wg[e]^T + du Wu[e]^T), the k slots added in j order
 *   dw_down[e]  = sum over the slots of expert e of h^T (probs[t,j] dout[t])
 *   dw_gate[e]  = sum over the slots of expert e of x[t]^T dg,   dw_up[e] likewise with du
 * dtype MOE_BF16 only; H and F multiples of 128; head_m_size 0; flags ignored.
 *   x [T,H], w_gate / w_up [E,H,F], w_down [E,F,H] bfloat16; expert_ids [T,k] int32;
 *   probs [T,k] float32; dout [T,H] bfloat16
 *   saved_gu: NULL, or the g and u that moe_expert_forward_train kept for the same inputs
 *   dx [T,H] bfloat16; dw_gate / dw_up [E,H,F], dw_down [E,F,H], dprobs [T,k] float32
 * Without saved_gu, g and u are recomputed from x.  g, u, dg, du and probs * h
 * are rounded to bfloat16, and so is each slot's dx row, except on problems with few 256-row tiles,
 * where dg Wg^T and du Wu^T run as separate tasks and stay fp32 until the per-token sum.  Every
 * gradient element is an fp32 sum in a fixed order (no float atomics): deterministic.  Experts that receive no slot get zero
 * weight gradients; slots with an out-of-range id are skipped (dprobs 0) and flag the status word. */
moe_status moe_expert_backward(const moe_problem* p, const void* x, const void* w_gate,
                               const void* w_up, const void* w_down, const int32_t* expert_ids,
                               const float* probs, const void* dout, const void* saved_gu, void* dx,
                               float* dw_gate, float* dw_up, float* dw_down, float* dprobs,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Sub-steps (the same kernels the whole-layer calls use).
 * ------------------------------------------------------------------------------------------- */

/* Host only.  Workspace bytes for moe_route. */
moe_status moe_route_workspace_size(int64_t T, int64_t k, int64_t E, size_t* bytes /* host */);

/* Routing ("NPU Training Operators - MC2", 执行路径 step 2 and the index maps of steps 6 and 10).
 * Slots are the flattened ids, s = t*k + j.
 *   counts[E]    slots per expert (histc with E bins over [0, E); out-of-range ids not counted)
 *   offsets[E+1] exclusive prefix sum of counts
 *   perm[M]      permuted row p holds slot perm[p]; rows are grouped by ascending expert and,
 *                inside an expert, by ascending slot (stable), M = T*k.  Entries past offsets[E]
 *                (only when ids were out of range) are -1.
 *   pos[M]       row of slot s (the inverse of perm), or -1 for an out-of-range id.
 * Integer only; bit-exact and deterministic. */
moe_status moe_route(const int32_t* expert_ids, int64_t T, int64_t k, int64_t E, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* pos, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* moe_route for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same kernels and results, with the
 * routing scratch (a status word and per-block expert histograms) in a static device array of
 * 256 B + 4 MiB that the library holds on each GPU it runs on until the process ends.  Nothing is
 * allocated and no workspace is passed; inputs and outputs are as for moe_route.
 * Limit: ceil(T*k / 2048) * (E + 1) <= 2^20 (e.g. any T*k < 2^31 for E = 8, T*k <= 2M slots for
 * E = 1023); larger problems return MOE_ERR_UNSUPPORTED with nothing enqueued.
 * Every call on one GPU uses that GPU's single scratch array: calls that overlap in time on one GPU
 * (on different streams or host threads) race and must be serialised by the caller.  The kernels
 * write every scratch word they read within the same call, so nothing needs clearing between calls.
 * Out-of-range ids are dropped as in moe_route; with no workspace status word, offsets[E] < T*k is
 * the sign that some were. */
moe_status moe_route_noalloc(const int32_t* expert_ids, int64_t T, int64_t k, int64_t E,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                             hipStream_t stream);

/* Permute ("NPU Training Operators - MC2", 执行路径 step 6): x_perm[pos[s]] = x[s / k] for every
 * slot with pos[s] >= 0.  Rows of p->H elements of p->dtype; for MOE_MXFP8_E4M3 the H/32 scale bytes
 * of each row move with it (x_scale -> x_perm_scale; both NULL otherwise).  x_perm has T*k rows.
 * A pure copy: bit-exact. */
moe_status moe_permute(const moe_problem* p, const void* x, const uint8_t* x_scale,
                       const int32_t* pos, void* x_perm, uint8_t* x_perm_scale, hipStream_t stream);

/* Unpermute ("NPU Training Operators - MC2", 执行路径 step 10):
 *   out[t] = sum_{j = 0..k-1, in order} probs[t,j] * y_perm[pos[t*k+j]]
 * fp32 accumulation (fused multiply-add, starting from 0), one rounding to the output dtype; slots
 * with pos < 0 are skipped.  y_perm [T*k, H] and out [T,H] are float32 for MOE_F32, bfloat16 for
 * MOE_BF16 and MOE_MXFP8_E4M3. */
moe_status moe_unpermute(const moe_problem* p, const void* y_perm, const int32_t* pos,
                         const float* probs, void* out, hipStream_t stream);

/* Host only.  Workspace bytes for moe_grouped_ffn / moe_grouped_ffn_mx with M rows in G groups. */
moe_status moe_grouped_ffn_workspace_size(const moe_problem* p, int64_t M, int64_t G,
                                          size_t* bytes /* host */);

/* Grouped expert FFN on rows that are already grouped, as one expert-parallel rank receives them
 * after the dispatch All-to-All ("NPU Training Operators - MC2", 执行路径 steps 5, 7-9): group g is
 * rows [group_offsets[g], group_offsets[g+1]) and uses expert group_expert[g] (both device arrays,
 * read only on the device, so the call never waits for the GPU).  Groups may be empty and several
 * groups may share an expert.  y_rows[r] = FFN_{expert of r}(rows[r]); rows / y_rows are [M,H] in
 * p->dtype (MOE_F32 or MOE_BF16).  p->T and p->k are ignored; p->E bounds group_expert. */
moe_status moe_grouped_ffn(const moe_problem* p, const void* rows, int64_t M,
                           const int32_t* group_offsets, const int32_t* group_expert, int64_t G,
                           const void* w_gate, const void* w_up, const void* w_down, void* y_rows,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same for OCP-MX rows (rows_scale [M, H/32]); y_rows is bfloat16 [M,H]. */
moe_status moe_grouped_ffn_mx(const moe_problem* p, const uint8_t* rows, const uint8_t* rows_scale,
                              int64_t M, const int32_t* group_offsets,
                              const int32_t* group_expert, int64_t G, const uint8_t* w_gate,
                              const uint8_t* wg_scale, const uint8_t* w_up,
                              const uint8_t* wu_scale, const uint8_t* w_down,
                              const uint8_t* wd_scale, void* y_rows, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Router in front of the layer: the gate's top-k.  logits [T, E] float32 (E <= 1024) ->
 * expert_ids [T, k] int32 and probs [T, k] float32 (1 <= k <= min(E, 64)), ready for
 * moe_expert_forward.  The gate is the first step of the step breakdown on the page "MC2 通算融合";
 * the router top-k distribution is one of the checks listed on the page "NPU Training Operators -
 * MC2" (验证项).  Per token: the k largest logits in descending order, equal logits taken in
 * ascending expert id; probs[t, j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected
 * (the softmax over all E renormalised over the k), float32 arithmetic.  Logits must not be NaN and
 * each token's largest logit must be finite (-inf logits are taken last, with probability 0).
 * Errors: MOE_ERR_INVALID_ARGUMENT for bad sizes or null pointers (nothing enqueued). */
moe_status moe_router_topk(const float* logits, int64_t T, int64_t E, int64_t k,
                           int32_t* expert_ids, float* probs, hipStream_t stream);

/* OCP-MX encoder used on h inside the MX layer, exposed on its own: v [rows, cols] float32
 * (cols a multiple of 32) -> codes [rows, cols] E4M3 bytes and scales [rows, cols/32] E8M0 bytes.
 * Shared exponent floor(log2 max|block|) - 8 clamped to [-127, 127] (-127 for an all-zero block);
 * elements v / 2^e rounded to nearest even on the E4M3 grid, saturated to +-448, sign kept.
 * The shared exponent is integer arithmetic on the float32 bits and the elements go through the
 * hardware E4M3 conversion after an exact power-of-two scaling and a clamp to +-448: bit-exact and
 * deterministic. */
moe_status moe_mx_quantize(const float* v, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream);

/* The encoder of the MX layer's fc1 epilogue (the SwiGLU output h -> E4M3 codes and E8M0 block
 * scales along F, "MC2 通算融合架构总览", §1 and §5), run by the same device code as inside the
 * grouped GEMM (the staging through LDS, the block maximum combined across lanes, the encoding and
 * the stores) but on caller-supplied float32 values in place of the SwiGLU output, so that the
 * epilogue can be checked exactly against a reference encoder.  v [rows, cols] float32 -> codes
 * [rows, cols] and scales [rows, cols/32], with moe_mx_quantize's rule.  large_tiles != 0: the
 * epilogue of the 256-row-tile kernel (cols a multiple of 128; the one serving H and F multiples of
 * 1024), else that of the 128-row-tile kernel (cols a multiple of 64).  rows * cols <= 2^28.
 * Errors: MOE_ERR_INVALID_ARGUMENT for bad sizes or null pointers (nothing enqueued). */
moe_status moe_mx_fc1_epilogue_encode(const float* v, int64_t rows, int64_t cols,
                                      int32_t large_tiles, uint8_t* codes, uint8_t* scales,
                                      hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Status, errors, diagnostics.
 * ------------------------------------------------------------------------------------------- */

/* Waits for `stream`, then reads the device status word that the last call using `workspace`
 * recorded (MOE_OK or MOE_ERR_EXPERT_ID_OUT_OF_RANGE) into *status (host). */
moe_status moe_query_device_status(const void* workspace, hipStream_t stream,
                                   int32_t* status /* host */);

/* Per-chunk completion counters of the last chunked call using `workspace` (head_m_size > 0):
 * after the call's work ends, counters (device, [num_chunks] int32, num_chunks = ceil(M /
 * head_m_size)) hold the number of down-projection tiles finished in each chunk; tiles_per_chunk
 * gives the expected totals.  Both are device pointers inside the workspace. */
moe_status moe_chunk_counters(const moe_problem* p, void* workspace, size_t workspace_bytes,
                              int64_t M, const int32_t** counters, const int32_t** tiles_per_chunk,
                              int64_t* num_chunks /* host */);

/* Host only.  For a forward with MOE_FLAG_QUANTIZE_X: where in the workspace the call leaves the
 * encoded x.  *permuted = 0: token order ([T, H] codes + [T, H/32] scales), when the first grouped
 * GEMM gathers its rows itself; *permuted = 1: the T*k permuted rows (the layout of moe_permute),
 * when the permute runs as its own step.  Valid after the call's work ends. */
moe_status moe_quantized_x_offsets(const moe_problem* p, size_t* codes_offset /* host */,
                                   size_t* scales_offset /* host */, int32_t* permuted /* host */);

/* Host only.  Byte offsets, inside the workspace of moe_grouped_ffn / moe_grouped_ffn_mx (M rows in G
 * groups) or of moe_expert_forward / _mx (M = T*k, G = E), of the intermediate SwiGLU output h
 * [M, F] (p->dtype elements; E4M3 bytes for MX) and, for MX, of its E8M0 scales [M, F/32].  After
 * the call's work ends they hold that call's h, for inspection. */
moe_status moe_intermediate_offsets(const moe_problem* p, int64_t M, int64_t G,
                                    size_t* h_offset /* host */, size_t* h_scale_offset /* host */);

const char* moe_status_string(moe_status s);
const char* moe_last_error(void);

/* Kernel timing for profiling.  While enabled, every kernel the library enqueues is bracketed by
 * two hipEvents recorded on the same stream.  moe_timing_collect waits for those events, adds
 * each kernel's elapsed time to a per-name total, and copies up to `capacity` entries into the host
 * arrays (name pointers stay valid for the life of the library).  Entries accumulate across calls
 * until moe_timing_reset. */
moe_status moe_timing_enable(int enable);
moe_status moe_timing_collect(const char** names /* host */, double* total_ms /* host */,
                              int64_t* launches /* host */, int capacity,
                              int* count /* host */);
moe_status moe_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EXPERT_LAYER_H */
