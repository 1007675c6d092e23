/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer hot path.
 *
 * The layer, as the pages state it ("Megatron-Bridge 深度剖析", section
 * "MoE 加速深度剖析 / Expert Parallel 基础", three-step diagram): a router
 * picks top-k experts per token with scores; tokens are regrouped by expert;
 * every expert runs its SwiGLU FFN over its tokens as ONE grouped GEMM
 * (section "计算融合 / Grouped GEMM"); results return to token order and are
 * combined.  An optional shared expert sees every token (section "Shared
 * Expert Overlap"), scaled by a per-token gate (TorchSpec pull request "Add
 * Megatron-Core MTP training for Qwen3.5 MoE", "What's in it").  Training
 * adds the grouped GEMM's dgrad and wgrad.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array pointer is a caller-owned DEVICE pointer (HBM), row-major,
 *    densely packed, 16-byte aligned.  The library never allocates, frees or
 *    keeps a pointer after it returns; scratch memory is the caller's
 *    workspace (`ws`, `ws_bytes`), sized by the matching *_workspace_size().
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 *    default stream).  No call synchronises the host: expert counts and
 *    offsets stay on the device and the kernels read them there.
 *  - `dt` selects the element type of activations and weights: MOE_F32 or
 *    MOE_BF16 (bf16 storage, fp32 accumulation).  Routing scores, routing
 *    weights, gates and weight gradients are always fp32.
 *  - Outputs must not alias inputs.  Calls are deterministic: the same
 *    inputs give bit-identical outputs (no floating-point atomics).
 *  - Errors: argument checks run on the host before anything is launched;
 *    a failed check returns a non-zero moe_status and launches nothing.
 *    A failed launch returns MOE_ERR_HIP.  Faults inside a kernel surface
 *    at the caller's next synchronisation.  Nothing is printed; no C++
 *    exception crosses this boundary.
 *  - Index arithmetic is 32-bit for row and slot indices: T*k must be below
 *    2^31.
 */
#ifndef MOE_MI355X_H_
#define MOE_MI355X_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* NULL where a pointer is required, bad enum   */
  MOE_ERR_SHAPE = 2,        /* a dimension out of the supported range       */
  MOE_ERR_DTYPE = 3,        /* unknown moe_dtype                            */
  MOE_ERR_ALIGNMENT = 4,    /* pointer not 16-byte aligned / d, F not x8    */
  MOE_ERR_WORKSPACE = 5,    /* ws NULL or smaller than *_workspace_size()   */
  MOE_ERR_UNSUPPORTED = 6,  /* valid request the library does not implement */
  MOE_ERR_HIP = 7           /* a HIP launch failed                          */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Score function of the router ("Megatron-Bridge 深度剖析", section
 * "Megatron-Core 架构速览": moe_router_score_function; the step-1 diagram of
 * "Expert Parallel 基础" shows top-6 sigmoid routing). */
typedef enum moe_score_fn { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

/* Tokens per histogram block of moe_route's block_counts and moe_permute. */
#define MOE_ROUTE_BLOCK_TOKENS 64

/* Version of this ABI (incremented on any signature change). */
MOE_API int32_t moe_abi_version(void);
/* Static, human-readable name of a status code. */
MOE_API const char* moe_status_string(moe_status s);

/* ------------------------------------------------------------------------
 * moe_route -- router logits, scores, top-k, weight normalisation, counts.
 *
 * Passage: "Megatron-Bridge 深度剖析", "Expert Parallel 基础", step 1
 * ("Router 决策": the router maps each token to its top-k experts with
 * scores).  For token t and expert e:
 *     z[t,e] = sum_i x[t,i] * w_router[e,i] + logit_bias[e]
 *     s[t,e] = softmax_e(z[t,:])  or  1 / (1 + exp(-z[t,e]))
 * The k experts with the largest fp32 scores are chosen, in descending
 * score order (equal scores: lower expert index first).  With `normalize`
 * the weights are s / (sum of the k chosen s), else the raw scores.  With
 * `normalize` and no selection_bias the experts are ranked by their fp32
 * logits z instead (softmax and sigmoid are increasing, so this is the score
 * order except where two scores lie within rounding of each other; equal
 * logits again rank the lower index first), and the scores are formed for
 * the k chosen experts only.
 * selection_bias (the expert-bias correction of the MoE-acceleration and
 * recipe config listings, "moe_router_enable_expert_bias", DeepSeek-style)
 * shifts only the choice: experts are ranked by the fp32 sum s + b[e],
 * the weights still come from the unbiased s.
 * With w_gate, gate[t] = 1 / (1 + exp(-x[t] . w_gate)) (shared-expert gate).
 *
 *   x          [T, d]  dt        tokens
 *   w_router   [E, d]  dt        router weight (Megatron's router.weight)
 *   logit_bias [E]     fp32      or NULL (added to the logits: moves the weights too)
 *   selection_bias [E] fp32      or NULL (ranking only; finite values)
 *   w_gate     [d]     dt        or NULL (then `gate` must be NULL too)
 *   topk_idx   [T, k]  int32     out
 *   topk_w     [T, k]  fp32      out
 *   expert_counts [E]  int32     out, or NULL: tokens routed to each expert
 *   block_counts [ceil(T / MOE_ROUTE_BLOCK_TOKENS), E] int32
 *                                out, or NULL: row b counts the choices of
 *                                tokens [64 b, 64 b + 64) per expert (the
 *                                histogram moe_permute can take in place of
 *                                its own counting pass)
 *   gate       [T]     fp32      out, or NULL
 * Limits: 1 <= k <= min(E, 32); 1 <= E <= 1024; d % 8 == 0; T >= 1;
 * 16*T*E < 2^31.  Workspace: moe_route_workspace_size(T, d, E, dt) bytes (the
 * fp32 logits, up to 16 K slabs, and for bf16 the K slabs of the gate's dot
 * product).  A NaN score is never chosen; a token with fewer than k
 * selectable scores gets index E (out of range) for the missing slots.  An
 * expert whose logit is -inf (masked, e.g. by a -inf logit_bias) has score
 * 0 and weight 0; it is chosen only after every expert with a finite
 * logit, lower index first.
 * --------------------------------------------------------------------- */
MOE_API size_t moe_route_workspace_size(int64_t T, int64_t d, int32_t E, moe_dtype dt);
MOE_API moe_status moe_route(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d,
                     int32_t E, int32_t k, moe_score_fn fn, int32_t normalize,
                     const void* x, const void* w_router,
                     const float* logit_bias, const float* selection_bias,
                     const void* w_gate, int32_t* topk_idx, float* topk_w,
                     int32_t* expert_counts, int32_t* block_counts, float* gate,
                     void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * moe_permute -- regroup token copies into per-expert contiguous segments.
 *
 * Passage: "Megatron-Bridge 深度剖析", "Expert Parallel 基础" step 2 (after
 * dispatch a GPU holds its tokens grouped by expert) and "Permute Fusion"
 * (the permute is a memory copy of the hidden states).  The N = T*k
 * (token, slot) pairs, taken token-major, are counting-sorted by expert
 * (stable: ascending token inside a segment):
 *     expert_offsets[e] = sum_{e' < e} count(e')          [E+1]
 *     slot_of[t,j]      = row holding token t's j-th choice
 *     row_token[r], row_w[r] = the token and routing weight of row r
 *     x_perm[r,:]       = x[row_token[r], :]
 *
 *   x          [T, d]  dt        in
 *   topk_idx   [T, k]  int32     in, values in [0, E)
 *   topk_w     [T, k]  fp32      in, or NULL (then row_w must be NULL)
 *   block_counts [ceil(T / MOE_ROUTE_BLOCK_TOKENS), E] int32
 *                                in, or NULL: moe_route's block_counts for
 *                                this topk_idx (skips the counting pass; not
 *                                modified); NULL: counted here
 *   expert_offsets [E+1] int32   out
 *   slot_of    [T, k]  int32     out
 *   row_token  [T*k]   int32     out
 *   row_w      [T*k]   fp32      out, or NULL
 *   x_perm     [T*k, d] dt       out, or NULL: no row copy is made (x may
 *                                then be NULL); a consumer that gathers by
 *                                row_token (moe_grouped_swiglu_fwd_gather)
 *                                reads x directly
 * An entry of topk_idx outside [0, E) is dropped: its slot_of is -1 and it
 * takes no row (rows past the last kept one are left unwritten).
 * Workspace: moe_permute_workspace_size(T, E, k) bytes.
 * Limits: 1 <= k <= 32; 1 <= E <= 1024; d*elt % 16 == 0.
 * --------------------------------------------------------------------- */
MOE_API size_t moe_permute_workspace_size(int64_t T, int32_t E, int32_t k);
MOE_API moe_status moe_permute(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d,
                       int32_t E, int32_t k, const void* x,
                       const int32_t* topk_idx, const float* topk_w,
                       const int32_t* block_counts,
                       int32_t* expert_offsets, int32_t* slot_of,
                       int32_t* row_token, float* row_w, void* x_perm,
                       void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * moe_permute_noalloc -- moe_permute without a caller workspace.
 *
 * For callers that cannot allocate device memory around the call (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, outputs and results as moe_permute, minus block_counts
 * (always counted here) and ws / ws_bytes:
 * the scratch (per-block expert histograms and per-expert totals) lives in a
 * static device array of 4 MiB inside the library, one per GPU, held until
 * the process ends.  Nothing is allocated or freed by the call.
 *   Limit: moe_permute_workspace_size(T, E, k) <= 4 MiB (ceil(T / 64) rows
 *   of E counts: T = 16384, E = 256 needs 0.25 MiB); larger
 *   shapes return MOE_ERR_WORKSPACE.  MOE_ERR_HIP if the array's device
 *   address cannot be obtained.
 *   Concurrency: every call on one GPU uses the same array; calls that
 *   overlap in time on one GPU (two streams, two threads) race and must be
 *   serialised by the caller.  No part of the array needs to start at zero:
 *   each call writes what it reads.
 * --------------------------------------------------------------------- */
MOE_API moe_status moe_permute_noalloc(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d,
                               int32_t E, int32_t k, const void* x,
                               const int32_t* topk_idx, const float* topk_w,
                               int32_t* expert_offsets, int32_t* slot_of,
                               int32_t* row_token, float* row_w, void* x_perm);

/* ------------------------------------------------------------------------
 * moe_grouped_swiglu_fwd -- every expert's SwiGLU FFN in one grouped GEMM.
 *
 * Passages: "Megatron-Bridge 深度剖析", "Grouped GEMM" (all experts' GEMMs
 * as one call over segments of different length), "权重映射策略"
 * (GatedMLPMapping: linear_fc1 = [gate_proj; up_proj], (2*ffn, hidden)),
 * "Motivation" (gate_proj, up_proj, down_proj per expert).  For expert e
 * with rows R_e = [expert_offsets[e], expert_offsets[e+1]):
 *     G = X[R_e] W1[e, 0:F]^T,  U = X[R_e] W1[e, F:2F]^T   (fp32 accumulate)
 *     A = silu(G) * U,          silu(z) = z / (1 + exp(-z))
 *     y_perm[R_e] = (A W2[e]^T) * row_scale[R_e]
 * For bf16, A is rounded to bf16 before the second GEMM.
 *
 *   x_perm     [N, d]      dt    in
 *   w1         [E, 2F, d]  dt    in (rows 0..F-1 gate, F..2F-1 up)
 *   w2         [E, d, F]   dt    in (down projection, (hidden, ffn))
 *   expert_offsets [E+1]   int32 in, device; 0 = off[0] <= ... <= off[E] = N
 *   row_scale  [N]         fp32  in, or NULL (= 1)
 *   y_perm     [N, d]      dt    out
 *   gu_save    [N, 2F]     dt    out, or NULL: G in cols 0..F-1, U in F..2F-1
 *                                (saved for the backward)
 * Workspace: moe_grouped_swiglu_fwd_workspace_size(N, F, dt) bytes.
 * Limits: E <= 1024, d % 8 == 0, F % 8 == 0, N >= 0, 4*F*d < 2^31 (one
 * expert's fc1 weights addressable with 32-bit byte offsets).  N = 0 (every
 * expert empty) computes nothing; x_perm, y_perm and the workspace may then
 * be NULL.
 * --------------------------------------------------------------------- */
MOE_API size_t moe_grouped_swiglu_fwd_workspace_size(int64_t N, int64_t F, moe_dtype dt);
MOE_API moe_status moe_grouped_swiglu_fwd(hipStream_t stream, moe_dtype dt, int64_t N,
                                  int64_t d, int64_t F, int32_t E,
                                  const void* x_perm, const void* w1,
                                  const void* w2, const int32_t* expert_offsets,
                                  const float* row_scale, void* y_perm,
                                  void* gu_save, void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * moe_grouped_swiglu_fwd_gather -- moe_grouped_swiglu_fwd with the permute
 * folded into the first GEMM's operand load.
 *
 * Passage: "Megatron-Bridge 深度剖析", "Permute Fusion" (the standalone
 * permute copy of the hidden states is replaced by reordering rows while
 * they are loaded).  Computes exactly moe_grouped_swiglu_fwd with
 *     x_perm[r, :] = x[row_token[r], :]
 * but never materialises x_perm: fc1 reads row r of each expert segment
 * from x[row_token[r]].
 *
 *   T          int64               rows of x, >= 1
 *   x          [T, d]      dt    in
 *   row_token  [N]         int32 in, device (moe_permute's row map); a value
 *                                outside [0, T) reads as a zero row
 *   the rest as in moe_grouped_swiglu_fwd (same workspace size)
 * Limits: those of moe_grouped_swiglu_fwd, and T*d*elt < 2^31 (x addressed
 * with 32-bit byte offsets).  Returns MOE_ERR_SHAPE beyond them.
 * --------------------------------------------------------------------- */
MOE_API moe_status moe_grouped_swiglu_fwd_gather(hipStream_t stream, moe_dtype dt, int64_t N,
                                         int64_t d, int64_t F, int32_t E, int64_t T,
                                         const void* x, const int32_t* row_token,
                                         const void* w1, const void* w2,
                                         const int32_t* expert_offsets,
                                         const float* row_scale, void* y_perm,
                                         void* gu_save, void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * moe_pack_weights -- expert weights in the tile-packed layout read by
 * moe_grouped_swiglu_fwd_packed.
 *
 * Passage: "Megatron-Bridge 深度剖析", "计算融合 / Grouped GEMM" (the experts'
 * weights are stored back to back and consumed by one grouped GEMM) and
 * "权重映射策略" (linear_fc1 = [gate_proj; up_proj]).  The values are those
 * of w; only their order in memory changes, so that each K tile of a weight
 * panel is one contiguous block (a sequential HBM stream):
 *     packed[e][t][kt][r][c] = w[e][row(t, r)][64 kt + c], zero past K or rows
 * with 256-row panels t and 64-wide K tiles kt.  gated = 0 (W2 [E, d, F]):
 * row(t, r) = 256 t + r.  gated = 1 (W1 [E, 2F, d], rows = 2F): panel t holds
 * the gate rows 128 t .. 128 t + 127 and then the matching up rows F + 128 t
 * .. F + 128 t + 127.
 *
 *   w          [E, rows, K] bf16   in
 *   w_packed   moe_pack_weights_size(E, rows, K, gated) bytes, out
 * Limits: bf16 only (MOE_ERR_DTYPE), K % 8 == 0, rows even when gated.
 * The layout is a function of (rows, K, gated) only; repack after the
 * weights change.
 * --------------------------------------------------------------------- */
MOE_API size_t moe_pack_weights_size(int32_t E, int64_t rows, int64_t K, int32_t gated);
MOE_API moe_status moe_pack_weights(hipStream_t stream, moe_dtype dt, int32_t E, int64_t rows,
                            int64_t K, int32_t gated, const void* w, void* w_packed);

/* ------------------------------------------------------------------------
 * moe_grouped_swiglu_fwd_packed -- moe_grouped_swiglu_fwd (row_token NULL,
 * x = x_perm [N, d]) or moe_grouped_swiglu_fwd_gather (row_token given, x
 * [T, d]) on tile-packed weights.
 *
 * Passages: those of the two calls it replaces.  Same results, bit for bit:
 * the kernels stage identical tiles, only the weight reads differ.
 *
 *   w1_packed  moe_pack_weights(E, 2F, d, gated = 1) of W1
 *   w2_packed  moe_pack_weights(E, d, F, gated = 0) of W2
 *   T          rows of x when row_token is given (ignored otherwise)
 *   the rest as in moe_grouped_swiglu_fwd / _gather (same workspace size)
 * Limits: bf16 only (MOE_ERR_DTYPE); those of the call it replaces; one
 * expert's packed weights below 2^31 bytes.
 * --------------------------------------------------------------------- */
MOE_API moe_status moe_grouped_swiglu_fwd_packed(hipStream_t stream, moe_dtype dt, int64_t N,
                                         int64_t d, int64_t F, int32_t E, int64_t T,
                                         const void* x, const int32_t* row_token,
                                         const void* w1_packed, const void* w2_packed,
                                         const int32_t* expert_offsets,
                                         const float* row_scale, void* y_perm,
                                         void* gu_save, void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * MXFP8 forward: the grouped SwiGLU with microscaled FP8 E4M3 operands.
 *
 * Passages: "Megatron-Bridge 深度剖析", section "FP8 训练" (E4M3 and its scale
 * factors; FP8 doubles the matrix rate and halves the traffic of the grouped
 * GEMM that BF16 leaves memory-bound) and the section on future directions
 * (MXFP8: finer-grained scale factors).  Format (OCP microscaling): E4M3
 * codes (largest finite 448), one E8M0 scale byte (2^(code - 127)) per 32
 * consecutive values along the reduction dimension,
 *     scale = 2^(floor(log2 max|v|) - 8),  code = RNE(clamp(v / scale, +-448));
 * an all-zero block gets scale byte 0.  Quantised: the token rows (along d),
 * W1 and W2 rows (along d and F), and A = silu(G) U per row along F (taken
 * from its fp32 value inside fc1's epilogue).  Accumulation is fp32 (the MFMA
 * adds each 64-value product at reduced internal precision, ~2^-14 relative).
 *
 * moe_quantize_mx: rows [R, K] bf16 -> codes [R, K] u8 and scales laid out
 *   [ceil(K/512)][R][16] u8: the scale of block b (values 32b .. 32b+31) of
 *   row r at [b / 16][r][b % 16], so a row's scales for 512 consecutive K
 *   values are 16 adjacent bytes; slots past K / 32 are 0.  K % 32 == 0.
 *   Scales occupy moe_quantize_mx_scales_size(R, K) bytes.
 * moe_pack_weights_mx: W [E, rows, K] bf16 -> codes in the tile-packed layout
 *   of moe_pack_weights with 128-wide K tiles, [e][panel][K tile][256 rows]
 *   [128], and scales [e][panel][K tile][256 rows][4]; gated = 1 for W1
 *   ([gate; up] panels of 128 + 128 rows), 0 for W2.  Sizes from
 *   moe_pack_weights_mx_size(E, rows, K, gated, scales = 0 / 1).
 * moe_grouped_swiglu_fwd_mx: the forward on those operands:
 *   xq, xs     moe_quantize_mx of x [T, d] (row_token given: fc1 gathers row
 *              r from x[row_token[r]]) or of x_perm [N, d] (row_token NULL)
 *   w1q, w1s   moe_pack_weights_mx(E, 2F, d, 1);  w2q, w2s: (E, d, F, 0)
 *   y_perm     [N, d] bf16 out, (A Q(W2)^T) * row_scale
 *   workspace  moe_grouped_swiglu_fwd_mx_workspace_size(N, F) bytes; after
 *              the call it holds A = silu(G) U quantised: codes [N, F] at
 *              offset 0 and scales in the moe_quantize_mx layout at offset
 *              round_up(N F, 256)
 * Limits: d % 32 == 0, F % 32 == 0, E <= 1024, one expert's packed codes and
 * the token rows below 2^31 bytes.  Inference only: no G, U save.
 * --------------------------------------------------------------------- */
MOE_API size_t moe_quantize_mx_scales_size(int64_t R, int64_t K);
MOE_API moe_status moe_quantize_mx(hipStream_t stream, int64_t R, int64_t K, const void* x,
                           void* codes, void* scales);
MOE_API size_t moe_pack_weights_mx_size(int32_t E, int64_t rows, int64_t K, int32_t gated,
                                int32_t scales);
MOE_API moe_status moe_pack_weights_mx(hipStream_t stream, int32_t E, int64_t rows, int64_t K,
                               int32_t gated, const void* w, void* w_codes, void* w_scales);
MOE_API size_t moe_grouped_swiglu_fwd_mx_workspace_size(int64_t N, int64_t F);
MOE_API moe_status moe_grouped_swiglu_fwd_mx(hipStream_t stream, int64_t N, int64_t d, int64_t F,
                                     int32_t E, int64_t T, const void* xq, const void* xs,
                                     const int32_t* row_token, const void* w1q, const void* w1s,
                                     const void* w2q, const void* w2s,
                                     const int32_t* expert_offsets, const float* row_scale,
                                     void* y_perm, void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * moe_grouped_swiglu_bwd -- grouped-GEMM dgrad and wgrad of the forward.
 *
 * Passage: "Megatron-Bridge 深度剖析", "通信隐藏与混合精度 / TP 通信重叠"
 * (the backward's dgrad and wgrad GEMMs) and "其他融合优化"
 * (gradient_accumulation_fusion: weight gradients accumulate into fp32
 * main grads).  Given dY = dL/dy_perm, for each expert e:
 *     dYs = dY * row_scale;       dA = dYs W2[e]
 *     dG  = dA * U * silu'(G);    dU = dA * silu(G);    dH = [dG | dU]
 *     dx_perm[R_e] = dH W1[e]
 *     dw2[e] (+)= dYs^T A;        dw1[e] (+)= dH^T X[R_e]
 * silu'(z) = s (1 + z (1 - s)), s = sigmoid(z).  An expert with no rows
 * gets dw = 0 (or is left unchanged when accumulating).
 *
 *   dy_perm    [N, d]      dt    in
 *   x_perm, w1, w2, expert_offsets, row_scale: as in the forward
 *   gu_save    [N, 2F]     dt    in (from the forward), or NULL: recompute
 *   accumulate int32             0: dw = grad;  1: dw += grad
 *   dx_perm    [N, d]      dt    out
 *   dw1        [E, 2F, d]  fp32  out
 *   dw2        [E, d, F]   fp32  out
 * Workspace: moe_grouped_swiglu_bwd_workspace_size(N, F, dt, recompute)
 * (needed also when N = 0: it holds the weight gradient's tile counters).
 * N = 0 (every expert empty) writes dw1, dw2 as zeros (or leaves them when
 * accumulating); dy_perm, x_perm and dx_perm may then be NULL.
 * Only MOE_BF16 is implemented (MOE_F32 returns MOE_ERR_UNSUPPORTED).
 * --------------------------------------------------------------------- */
MOE_API size_t moe_grouped_swiglu_bwd_workspace_size(int64_t N, int64_t F, moe_dtype dt,
                                             int32_t recompute);
MOE_API moe_status moe_grouped_swiglu_bwd(hipStream_t stream, moe_dtype dt, int64_t N,
                                  int64_t d, int64_t F, int32_t E,
                                  const void* dy_perm, const void* x_perm,
                                  const void* w1, const void* w2,
                                  const int32_t* expert_offsets,
                                  const void* gu_save, const float* row_scale,
                                  int32_t accumulate, void* dx_perm,
                                  float* dw1, float* dw2, void* ws,
                                  size_t ws_bytes);

/* ------------------------------------------------------------------------
 * moe_unpermute_combine -- back to token order, weighted k-way sum.
 *
 * Passage: "Megatron-Bridge 深度剖析", "Expert Parallel 基础" step 3 (the
 * results go back to the tokens' original layout) and "Shared Expert
 * Overlap" (the shared expert's output joins the routed result):
 *     y[t] = sum_j topk_w[t,j] * y_perm[slot_of[t,j]]
 *            (+ shared_gate[t] * y_shared[t], gate 1 when NULL)
 * summed in fp32 in slot order j = 0..k-1, rounded once to dt.  With
 * topk_w = NULL the rows are taken as already weighted (the forward can
 * apply the weight through row_scale, and the gate likewise).  slot_of < 0
 * entries are skipped.  A training forward keeps y_perm and y_shared
 * unweighted and passes topk_w and shared_gate here, so that
 * moe_combine_backward can form the weight and gate gradients.
 *
 *   y_perm   [N, d] dt   in        slot_of [T, k] int32  in
 *   topk_w   [T, k] fp32 in/NULL   y_shared [T, d] dt in/NULL
 *   shared_gate [T] fp32 in/NULL (requires y_shared)
 *   y        [T, d] dt   out
 * No workspace.  Limits: 1 <= k <= 32, d*elt % 16 == 0.
 * --------------------------------------------------------------------- */
MOE_API moe_status moe_unpermute_combine(hipStream_t stream, moe_dtype dt, int64_t T,
                                 int64_t d, int32_t k, int64_t N,
                                 const void* y_perm, const int32_t* slot_of,
                                 const float* topk_w, const void* y_shared,
                                 const float* shared_gate, void* y);

/* ------------------------------------------------------------------------
 * moe_combine_backward -- backward of the weighted combine.
 *
 * Passage: "Megatron-Bridge 深度剖析", "Expert Parallel 基础" step 3 and
 * "Shared Expert Overlap" (the forward being differentiated), "Activation
 * Recomputation" (the layer's backward).  For
 *     y[t] = sum_j w[t,j] Y[s(t,j)] + gate[t] Ysh[t],   s = slot_of,
 * with Y = y_perm and Ysh = y_shared unweighted:
 *     dy_perm[s(t,j)] = w[t,j] dy[t]
 *     d_topk_w[t,j]   = <dy[t], Y[s(t,j)]>        (0 for slot_of < 0)
 *     d_gate[t]       = <dy[t], Ysh[t]>
 * Dot products in fp32 (fixed order), dy_perm rounded once to dt.  Rows of
 * dy_perm that no (t, j) maps to are left unwritten.
 *
 *   dy       [T, d] dt    in       y_perm [N, d] dt  in (unweighted)
 *   slot_of  [T, k] int32 in       topk_w [T, k] fp32 in
 *   y_shared [T, d] dt    in/NULL (unweighted; then d_gate is required)
 *   dy_perm  [N, d] dt    out      d_topk_w [T, k] fp32 out
 *   d_gate   [T]    fp32  out/NULL
 * No workspace.  Limits: 1 <= k <= 32, d % 8 == 0.
 * --------------------------------------------------------------------- */
MOE_API moe_status moe_combine_backward(hipStream_t stream, moe_dtype dt, int64_t T,
                                int64_t d, int32_t k, int64_t N, const void* dy,
                                const void* y_perm, const int32_t* slot_of,
                                const float* topk_w, const void* y_shared,
                                void* dy_perm, float* d_topk_w, float* d_gate);

/* ------------------------------------------------------------------------
 * moe_route_backward -- permute backward + router backward (+ shared gate).
 *
 * Passage: "Megatron-Bridge 深度剖析", "Activation Recomputation" (the
 * backward recomputes the router softmax and the dispatch permute), with
 * the forward of moe_route / moe_permute.  For the selection topk_idx held
 * fixed, w = normalise(score(z)) (z = x W_r^T + b, score softmax or
 * sigmoid), c[t] = sum_j d_topk_w[t,j] w[t,j]:
 *     softmax, normalised:  dz[t,e_j] = w[t,j] (d_topk_w[t,j] - c[t])
 *     sigmoid, normalised:  dz[t,e_j] = (d_topk_w[t,j] - c[t]) / S[t] s (1 - s)
 *     sigmoid:              dz[t,e_j] = d_topk_w[t,j] s (1 - s)
 * (s = sigmoid(z[t,e_j]) recomputed in fp32, S[t] = sum_j s); dz = 0 off
 * the selection.  Softmax without normalisation (w[t,j] = p[t,e_j], p the
 * softmax over all E experts, recomputed in fp32) has a dense dz:
 *     softmax:              dz[t,e]   = p[t,e] (ds[t,e] - c[t])
 * with ds[t,e_j] = d_topk_w[t,j] and ds = 0 off the selection.
 * Shared gate g = sigmoid(x . w_gate): dgl = d_gate g (1-g).
 *     dx[t]        = sum_j dx_perm[slot_of[t,j]] + sum_e dz[t,e] W_r[e]
 *                    + dgl[t] w_gate + dx_add[t]          (rounded once)
 *     dw_router[e] (+)= sum_t dz[t,e] x[t]  (sparse dz: over expert e's rows
 *                       r, dz[r] x[row_token[r]])
 *     dw_gate      (+)= sum_t dgl[t] x[t]
 * All sums fp32 in a fixed order.  The dense case also needs T*E < 2^31 and
 * T*d < 2^31 (else MOE_ERR_SHAPE).
 *
 *   x [T, d], w_router [E, d], w_gate [d] or NULL: dt, as in the forward
 *   logit_bias [E] fp32 or NULL
 *   topk_idx, topk_w [T, k]: moe_route's outputs;  d_topk_w [T, k] fp32
 *   d_gate [T] fp32 (with w_gate, else NULL)
 *   expert_offsets [E+1], slot_of [T, k], row_token [T*k]: moe_permute's
 *   dx_perm [T*k, d] dt or NULL (the grouped backward's dx)
 *   dx_add  [T, d] dt or NULL (added to dx, e.g. the shared expert's dx)
 *   dx [T, d] dt out;  dw_router [E, d] fp32;  dw_gate [d] fp32 (with w_gate)
 *   accumulate int32: 0 dw = grad, 1 dw += grad (dx is always written)
 * Workspace: moe_route_backward_workspace_size(T, d, E, k, dt, fn,
 * normalize) bytes (0 for invalid sizes or dtype); the dense case holds the
 * fp32 logits, dz [T, E] and its dx term [T, d] there.
 * Limits: 1 <= k <= min(E, 32), E <= 1024, d % 8 == 0.
 * --------------------------------------------------------------------- */
MOE_API size_t moe_route_backward_workspace_size(int64_t T, int64_t d, int32_t E, int32_t k,
                                                 moe_dtype dt, moe_score_fn fn,
                                                 int32_t normalize);
MOE_API moe_status moe_route_backward(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d,
                              int32_t E, int32_t k, moe_score_fn fn, int32_t normalize,
                              const void* x, const void* w_router, const float* logit_bias,
                              const void* w_gate, const int32_t* topk_idx,
                              const float* topk_w, const float* d_topk_w, const float* d_gate,
                              const int32_t* expert_offsets, const int32_t* slot_of,
                              const int32_t* row_token, const void* dx_perm,
                              const void* dx_add, void* dx, float* dw_router, float* dw_gate,
                              int32_t accumulate, void* ws, size_t ws_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H_ */
