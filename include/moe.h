/*
 * moe.h - C ABI of libmoe.so, the MI355X (gfx950) sparse Mixture-of-Experts
 * layer: Route -> Dispatch (permute) -> Expert computation (one grouped FFN
 * over all experts) -> Combine (weighted un-permute), and the backward of each
 * stage. The four stages and the router's two outputs (routing weights and a
 * boolean token-expert map) are those of "Scalable Training of
 * Mixture-of-Experts Models with Megatron Core", section 2.1; the router
 * (gate linear, softmax or sigmoid score, top-k) is section 2.2 of that page;
 * top-k renormalisation is in "emerging-techniques-moe-training" (Quick Start,
 * Top-2 routing, Mixtral block).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is a DEVICE pointer into memory the caller owns
 *   (hipMalloc or a framework allocator), except where stated. The library
 *   allocates nothing and keeps no state between calls; all entry points are
 *   reentrant.
 * - Every call is asynchronous: it enqueues kernels on `stream` (a
 *   hipStream_t; NULL = the default stream) and returns. It never
 *   synchronises with the host, so expert token counts stay on the device.
 * - Tensors are dense, row-major, with the shapes given in brackets. Base
 *   pointers must be 16-byte aligned.
 * - dtype is MOE_DTYPE_BF16 (activations and weights in bfloat16, fp32
 *   accumulation) or MOE_DTYPE_F32. Routing quantities (logits, weights,
 *   routing-weight gradients) are always fp32; weight gradients are fp32.
 * - Arguments are validated on the host before anything is enqueued. A call
 *   that returns an error has enqueued nothing and left every output
 *   untouched. MOE_ERR_HIP reports a failed kernel launch; the message is in
 *   moe_last_error() (thread-local). No C++ exception crosses this ABI.
 * - Index inputs produced by one stage and consumed by the next (topk_idx,
 *   offsets, row_of, sorted_token) must be those the producing entry point
 *   wrote (or satisfy the same invariants). Kernels never read or write out of
 *   bounds for any index values, but results are unspecified for indices that
 *   break the invariants.
 * - Results are deterministic: identical inputs give bitwise identical
 *   outputs (no floating-point atomics).
 * - An empty batch (T = 0 tokens, so P = 0 pairs) is valid everywhere:
 *   pointers to arrays with T or P rows may then be NULL, per-expert outputs
 *   (counts, offsets, weight and bias gradients) are still written (zeros).
 *
 * Supported sizes (MOE_ERR_UNSUPPORTED otherwise): h % 64 == 0, F % 64 == 0,
 * 1 <= k <= E <= 256, T*k < 2^31.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad enum      */
    MOE_ERR_UNSUPPORTED = 2,  /* valid but outside the supported sizes      */
    MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
    MOE_ERR_HIP = 4           /* a HIP launch failed; see moe_last_error()  */
} moe_status;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 } moe_act;

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);
/* Static text for a moe_status value. */
const char *moe_status_string(int status);
/* Message of the last failing call on this thread ("" if none). */
const char *moe_last_error(void);

/* ------------------------------------------------------------------ Route
 * Router stage ("Scalable Training ... with Megatron Core", section 2.2:
 * gating l = W_r^T x, then a softmax or sigmoid score, then top-k; section
 * 5.1: the router stays in fp32).
 *
 *   x        [T,h] dtype       token hidden states
 *   w_gate   [E,h] dtype       router weight (row e = expert e)
 *   b_gate   [E]   fp32|NULL   router bias
 *   sel_bias [E]   fp32|NULL   aux-loss-free selection bias (sigmoid only;
 *                              enters the selection key, not the weights)
 * Outputs:
 *   logits      [T,E] fp32|NULL  gate logits
 *   topk_idx    [T,k] int32      selected experts, best first
 *   topk_w      [T,k] fp32       routing weights, summing to 1 per token
 *   routing_map [T,E] uint8|NULL 1 where expert e is selected for token t
 *   counts      [E]   int32      tokens per expert (overwritten)
 *
 * Logit of (t,e): fp32, summed in a fixed order: 64 partial sums by residue
 * i mod 64, each an fma chain over ascending i, then a halving tree
 * (s = 32..1: part[j] += part[j+s]), then + b_gate[e]. The key is the logit
 * (softmax; softmax is increasing in each logit) or sigma_c(l) + sel_bias[e]
 * (sigmoid; sigma_c rounds a fixed fp64 evaluation of 1/(1+e^-l), argument
 * clamped to [-80,80], to fp32). Top-k order: key descending, then expert
 * index ascending; -0 equals +0; a NaN key ranks as -inf. Weights: softmax
 * renormalised over the k selected (= softmax of the selected logits);
 * sigmoid: sigma(l_j) / sum of the selected sigma(l_i).
 *
 * Workspace (optional; NULL with 0 bytes is valid): device memory of
 * moe_route_workspace_size(T,E) bytes, 16-byte aligned. With it, bf16, at
 * least 32 experts, k <= 8 and no logits output, the route first computes all logits
 * with bf16 MFMA and proven error bounds, then the fixed-order logits only of
 * the experts that can still reach the top k; the outputs are identical, bit
 * for bit, to those of the fixed-order pass over all experts, for all finite
 * inputs (the bounds hold down to fp32's subnormal range, including matrix
 * products flushed to zero there; a token with a non-finite bound has all
 * of its experts recomputed in the fixed order).
 */
size_t moe_route_workspace_size(int64_t T, int E);
int moe_route(const void *x, int dtype, int64_t T, int64_t h, const void *w_gate,
              const float *b_gate, int E, int k, int score, const float *sel_bias,
              float *logits, int32_t *topk_idx, float *topk_w, uint8_t *routing_map,
              int32_t *counts, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------- Permute
 * Dispatch stage ("Scalable Training ... with Megatron Core", section 2.1
 * stage 2: tokens regrouped by expert before expert computation; no
 * all-to-all: every expert is local).
 *
 *   x        [T,h] dtype   token hidden states
 *   topk_idx [T,k] int32   from moe_route (or any per-token-distinct indices
 *                          in [0,E), e.g. replayed routing)
 * Outputs:
 *   offsets      [E+1] int32   start row of each expert's segment; offsets[E]
 *                              = T*k
 *   sorted_token [T*k] int32   token of each permuted row
 *   row_of       [T,k] int32   permuted row of pair (t, topk_idx[t,j])
 *   x_perm       [T*k,h] dtype|NULL  x[sorted_token[r]] in row r (NULL:
 *                              indices only)
 * Order inside a segment: ascending token index (stable).
 * Workspace: moe_permute_workspace_size(T,E,k) bytes of device memory.
 */
size_t moe_permute_workspace_size(int64_t T, int E, int k);
int moe_permute(const void *x, int dtype, int64_t T, int64_t h, int E, int k,
                const int32_t *topk_idx, int32_t *offsets, int32_t *sorted_token,
                int32_t *row_of, void *x_perm, void *workspace, size_t workspace_bytes,
                void *stream);

/* moe_permute without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops with a
 * fixed memory plan, harnesses that forbid hipMalloc): the same launches and
 * results, with the scratch in a static 1 MiB device array of the library
 * (one copy per GPU, held until the process ends; its address is looked up
 * once per device). Limit: ceil(T/256) * E <= 131072 (e.g. T = 131072 with
 * E = 256), otherwise MOE_ERR_UNSUPPORTED and nothing runs. Every scratch
 * entry a call reads it has first written in that call, so nothing needs
 * clearing between calls; calls that overlap on one GPU (other streams,
 * other threads) share the scratch and race, so the caller must order them.
 * Allocates nothing. */
int moe_permute_noalloc(const void *x, int dtype, int64_t T, int64_t h, int E, int k,
                        const int32_t *topk_idx, int32_t *offsets, int32_t *sorted_token,
                        int32_t *row_of, void *x_perm, void *stream);

/* ------------------------------------------------------------ Grouped FFN
 * Expert computation as one grouped GEMM over all experts ("Scalable
 * Training ... with Megatron Core", section 2.1 stage 3, TEGroupedMLP), each
 * expert a SwiGLU FFN without bias ("Mixture-of-Experts from Architecture to
 * Large-Scale Training", section 2.5: three weight matrices) or
 * Linear + GELU(erf) + Linear with biases ("emerging-techniques-moe-training",
 * Quick Start). Segment e is rows [offsets[e], offsets[e+1]) of x_perm and
 * uses expert e's weights; segment sizes are read on the device.
 *
 *   x_perm  [P,h] dtype       permuted tokens (P = T*k); or, when
 *                             gather_rows is not NULL, the unpermuted tokens
 *                             [x_rows,h], permuted row r being
 *                             x_perm[gather_rows[r]] (the sorted_token of
 *                             moe_permute: the dispatch copy is then skipped).
 *                             An index outside [0, x_rows) reads zeros.
 *                             Gathering needs x_rows * h * 4 < 2^31.
 *   gather_rows [P] int32|NULL, x_rows: see x_perm (x_rows ignored if NULL)
 *   offsets [E+1] int32       segment starts, offsets[E] = P
 *   w1      [E,n1*F,h] dtype  first projection; SwiGLU (n1 = 2): rows 0..F-1
 *                             gate, rows F..2F-1 up; GELU: n1 = 1
 *   b1      [E,n1*F] dtype|NULL, w2 [E,h,F] dtype, b2 [E,h] dtype|NULL
 *   x_sh    [T_sh,h] dtype|NULL  shared-expert input (the unpermuted x);
 *   w1_sh   [n1*F,h], w2_sh [h,F]  shared-expert weights (no bias)
 * Outputs:
 *   act  [P+T_sh,F] dtype     activation silu(g)*u or GELU(a) (input of the
 *                             second GEMM; rows P.. are the shared expert's)
 *   gu   [P+T_sh,n1*F] dtype|NULL  pre-activations kept for the backward
 *                             (SwiGLU: g then u; GELU: a, bias included)
 *   y    [P,h] dtype          expert outputs in permuted order
 *   y_sh [T_sh,h] dtype|NULL  shared-expert output
 * Arithmetic: fp32 accumulation on MFMA; act, gu and y are rounded to dtype.
 *
 * Workspace (optional; NULL with workspace_bytes 0 is valid): device memory
 * of moe_grouped_ffn_workspace_size(dtype) bytes (0 for fp32; for bf16 about
 * 256 KB per compute unit of the current device), 16-byte aligned, owned by
 * the caller and free to reuse once the call's work on the stream is done.
 * With it, a GEMM whose last round of tiles would leave most of the GPU idle
 * splits those tiles along h (resp. F) and sums the fp32 partial results in
 * a fixed order, so results stay deterministic for a given device and
 * workspace choice (with and without a workspace they may differ in
 * rounding). A smaller non-null workspace is used as far as it goes.
 */
size_t moe_grouped_ffn_workspace_size(int dtype);
int moe_grouped_ffn(const void *x_perm, const int32_t *gather_rows, int64_t x_rows, int dtype,
                    int64_t P, int64_t h, int64_t F, int E,
                    const int32_t *offsets, int act_kind, const void *w1, const void *b1,
                    const void *w2, const void *b2, const void *x_sh, int64_t T_sh,
                    const void *w1_sh, const void *w2_sh, void *act, void *gu, void *y,
                    void *y_sh, void *workspace, size_t workspace_bytes, void *stream);

/* Memory-efficient permutation ("Scalable Training ... with Megatron Core",
 * section 4.1.1): for experts without an output bias,
 *   sum_i p_i W2 phi(W1 x) = sum_i W2 (p_i phi(W1 x)),
 * so the routing weight can be applied to the activation before the second
 * projection. moe_grouped_ffn with the activation of permuted row r scaled by
 * row_w[r] (fp32 [P], e.g. from moe_permute_weights; shared-expert rows are
 * not scaled): act = p * silu(g) * u or p * GELU(a), and y = W2 act is then
 * the weighted expert output, to be combined by moe_unpermute with
 * topk_w = NULL. The expert output y is not needed by the backward
 * (moe_grouped_ffn_bwd_recompute derives the routing-weight gradient from the
 * pre-activations). There is no b2 argument: with an output bias the two
 * forms differ by (k-1) b2. gu keeps the unscaled pre-activations. */
int moe_grouped_ffn_weighted(const void *x_perm, const int32_t *gather_rows, int64_t x_rows,
                             int dtype, int64_t P, int64_t h, int64_t F, int E,
                             const int32_t *offsets, int act_kind, const void *w1, const void *b1,
                             const void *w2, const void *x_sh, int64_t T_sh, const void *w1_sh,
                             const void *w2_sh, const float *row_w, void *act, void *gu, void *y,
                             void *y_sh, void *workspace, size_t workspace_bytes, void *stream);

/* Routing weights in permuted-row order: row_w[row_of[t,j]] = topk_w[t,j]
 * (row_w [T*k] fp32, row_of [T,k] as moe_permute writes it), and the
 * backward gather grad_topk_w[t,j] = grad_row_w[row_of[t,j]]. */
int moe_permute_weights(const float *topk_w, int64_t T, int k, const int32_t *row_of,
                        float *row_w, void *stream);
int moe_permute_weights_bwd(const float *grad_row_w, int64_t T, int k, const int32_t *row_of,
                            float *grad_topk_w, void *stream);

/* -------------------------------------------------------------- Unpermute
 * Combine stage ("Scalable Training ... with Megatron Core", section 2.1
 * stage 4 and section 1.1's MoE(x) = sum over the top-k of p_i E_i(x)):
 *   out[t] = sum_{j<k, ascending} topk_w[t,j] * y[row_of[t,j]]  (+ y_sh[t])
 * accumulated in fp32, rounded once to dtype.
 *   y [P,h] dtype, row_of [T,k], topk_w [T,k] fp32 or NULL (weights 1: the
 *   rows of moe_grouped_ffn_weighted are already weighted), y_sh [T,h]
 *   dtype|NULL, out [T,h] dtype (output)
 */
int moe_unpermute(const void *y, int dtype, int64_t T, int64_t h, int k,
                  const int32_t *row_of, const float *topk_w, const void *y_sh, void *out,
                  void *stream);

/* ------------------------------------------------------------------ MXFP8
 * "Scalable Training ... with Megatron Core", section 5.3.3: activations and
 * weights quantised in 1 x 32 blocks with E8M0 scales (E4M3 elements); the
 * expert GEMMs run on CDNA4's scaled fp8 matrix instruction.
 *
 * moe_mx_quantize: src [rows,K] dtype (K % 32 == 0) to codes [rows,K] uint8
 * (E4M3) and scales [rows,K/32] uint8 (E8M0, 2^(s-127)). Per block of 32:
 * shared exponent floor(log2 max|v|) - 8, clamped to [-127,127] (-127 for an
 * all-zero block); elements v * 2^-exp rounded to nearest-even on the E4M3
 * grid, saturated at 448. Deterministic bit for bit. Weights are quantised
 * along their reduction axis: w1 [E,2F,h] as E*2F rows of h, w2 [E,h,F] as
 * E*h rows of F. */
int moe_mx_quantize(const void *src, int dtype, int64_t rows, int64_t K, uint8_t *codes,
                    uint8_t *scales, void *stream);

/* Grouped SwiGLU FFN in MXFP8 (no bias, no shared expert): tokens x_codes /
 * x_scales (rows quantised along h; permuted rows [P,h], or with gather_rows
 * the unpermuted [x_rows,h] as in moe_grouped_ffn), weights as quantised by
 * moe_mx_quantize. The first projection's epilogue quantises its fp32
 * activation silu(g)*u along F by moe_mx_quantize's rule, writing
 * act_codes [P,F] / act_scales [P,F/32] (and, when act is not NULL, the same
 * activation rounded to bf16 in act [P,F]); the second projection reads
 * those codes and writes y [P,h] bf16. fp32 accumulation. Needs h % 128 == 0,
 * F % 128 == 0; code, output and workspace pointers 16-byte aligned, scale
 * pointers 4-byte aligned. Workspace (optional, NULL allowed): device memory
 * of moe_grouped_ffn_mx_workspace_size(P,h,F,E) bytes (less is allowed); with
 * it, when the second projection's last round of tiles would leave more
 * than half of the compute units idle, those tiles are split along F into
 * pieces whose fp32 partial sums are added in piece order (deterministic:
 * the result does not depend on the grid, but differs from the unsplit sum
 * by the reassociation). */
size_t moe_grouped_ffn_mx_workspace_size(int64_t P, int64_t h, int64_t F, int E);
int moe_grouped_ffn_mx(const uint8_t *x_codes, const uint8_t *x_scales, const int32_t *gather_rows,
                       int64_t x_rows, int64_t P, int64_t h, int64_t F, int E,
                       const int32_t *offsets, int act_kind, const uint8_t *w1_codes,
                       const uint8_t *w1_scales, const uint8_t *w2_codes,
                       const uint8_t *w2_scales, void *act, uint8_t *act_codes,
                       uint8_t *act_scales, void *y, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Training in MXFP8 ("Scalable Training of Mixture-of-Experts Models with
 * Megatron Core": section 5.1 quantises the expert GEMMs and keeps the router
 * in FP32; section 5.3.3 MXFP8; section 5.4 aligns to 32 by padding the
 * routing map). Every expert GEMM takes both operands in MXFP8 blocked along
 * its own reduction axis (moe_mx_quantize's rule per block of 32).
 *
 * moe_mx_quantize_t: src [batch,R,C] dtype, each matrix quantised along R
 * (blocks of 32 consecutive rows of a column), stored transposed: codes
 * [batch,C,R], scales [batch,C,R/32]. For the input gradients: w1 [E,2F,h]
 * gives w1t [E,h,2F] (blocked along 2F), w2 [E,h,F] gives w2t [E,F,h]
 * (blocked along h). Needs R % 32 == 0, codes 16-byte aligned.
 *
 * moe_grouped_ffn_bwd_mx: the backward of moe_grouped_ffn_mx (SwiGLU),
 * recomputing the first projection (selective recomputation, in the pages'
 * optimisation stack) so that every quantised operand is formed from fp32
 * values rather than from bf16 copies:
 *   grad_out [T,h] bf16   dL/d(layer output)
 *   row_w [P] fp32        routing weight of each permuted row
 *                         (moe_permute_weights); dY row p = row_w[p] *
 *                         grad_out[sorted_token[p]] in fp32
 *   x [T,h] bf16, x_codes/x_scales: the tokens and the forward's codes of
 *                         them (along h); rows gathered by sorted_token [P]
 *   w1_codes/w1_scales    the forward's codes of w1 (moe_mx_quantize)
 *   w1t_*, w2t_*          moe_mx_quantize_t of w1 and w2
 * Computes gu = Q_h(x) Q_h(W1) (fp32 accumulation), act = silu(g) u, dgu =
 * the SwiGLU backward of Q_h(dY) Q_h(W2) at (g, u), and writes grad_x_perm
 * [P,h] bf16 = Q_2F(dgu) Q_2F(W1), grad_w1 [E,2F,h] = Q_tok(dgu)^T Q_tok(x)
 * and grad_w2 [E,h,F] = Q_tok(dY)^T Q_tok(act) in fp32, where Q_tok blocks
 * each expert's tokens from its first row in blocks of 32, the last one
 * completed with zero rows (an expert without tokens gets zero weight
 * gradients). fp32 accumulation, deterministic. The routing-weight gradient
 * comes from moe_unpermute_bwd on the forward's y. Needs h % 128 == 0,
 * F % 128 == 0, E <= 256, a workspace of
 * moe_grouped_ffn_bwd_mx_workspace_size(P,h,F,E) bytes (MOE_ERR_WORKSPACE
 * otherwise), tensor, code and workspace pointers 16-byte aligned, scale
 * pointers 4-byte aligned; T*h, P*h and 2*P*F below 2^31 and P + 127 E
 * below 2^23 (MOE_ERR_UNSUPPORTED otherwise). */
int moe_mx_quantize_t(const void *src, int dtype, int64_t batch, int64_t R, int64_t C,
                      uint8_t *codes, uint8_t *scales, void *stream);
size_t moe_grouped_ffn_bwd_mx_workspace_size(int64_t P, int64_t h, int64_t F, int E);
int moe_grouped_ffn_bwd_mx(const void *grad_out, const float *row_w, const void *x,
                           const uint8_t *x_codes, const uint8_t *x_scales,
                           const int32_t *sorted_token, int64_t T, int64_t P, int64_t h, int64_t F,
                           int E, const int32_t *offsets, int act_kind, const uint8_t *w1_codes,
                           const uint8_t *w1_scales, const uint8_t *w1t_codes,
                           const uint8_t *w1t_scales, const uint8_t *w2t_codes,
                           const uint8_t *w2t_scales, void *grad_x_perm, float *grad_w1,
                           float *grad_w2, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------- Routing variants
 * "emerging-techniques-moe-training".
 *
 * Capacity-factor token dropping (Capacity Factor Tuning; the DeepSpeed MoE
 * config's drop_tokens): expert e takes at most `capacity` of its pairs, the
 * first in ascending token order (the order of moe_permute's segments); the
 * other pairs are dropped: they reach no expert, add nothing to the output
 * and keep no row; the kept pairs keep their routing weights. The page's
 * capacity is int(tokens / experts * capacity_factor) (e.g. with the T*k
 * routing slots as tokens and a floor of min_capacity); the caller passes
 * the resulting integer. From moe_permute's topk_idx, offsets and row_of:
 *   offsets_kept      [E+1] int32  segment starts of the kept rows
 *   row_of_kept       [T,k] int32  kept row of each pair, -1 if dropped
 *   sorted_token_kept [T*k] int32  token of each kept row (rows past
 *                                  offsets_kept[E] are not written)
 *   x_perm_kept [T*k,h] dtype|NULL x rows in kept-row order (needs x)
 * The forward then runs moe_grouped_ffn on offsets_kept (with x_perm_kept,
 * or x and gather_rows = sorted_token_kept) and moe_unpermute with
 * row_of_kept (rows of -1 are skipped). In the backward, moe_unpermute_bwd,
 * moe_grouped_ffn_bwd and moe_permute_bwd take the kept arrays, while
 * moe_route_bwd keeps the full offsets and sorted_token: every selected
 * pair's logit gradient reaches the router (a dropped pair's routing-weight
 * gradient is 0, the kept weights still depend on its logit). */
int moe_capacity_drop(const int32_t *topk_idx, const int32_t *offsets, const int32_t *row_of,
                      const void *x, int dtype, int64_t T, int64_t h, int E, int k, int capacity,
                      int32_t *offsets_kept, int32_t *row_of_kept, int32_t *sorted_token_kept,
                      void *x_perm_kept, void *stream);

/* Expert-choice routing (Routing Mechanisms, Expert Choice Routing): with
 * the router's logits [T,E] fp32 (moe_route's logits output), expert e takes
 * the `capacity` tokens with the largest logits l[t,e] (ties: lower token
 * index; -0 = +0), 1 <= capacity <= T. Outputs:
 *   offsets      [E+1] int32       e * capacity
 *   sorted_token [E*capacity] int32 chosen tokens, expert-major, ascending
 *                                  within an expert
 *   row_w        [E*capacity] fp32 weight of each chosen pair: softmax over
 *                                  all E logits of the token, at e
 *   token_rows   [T,E] int32       rows of token t in ascending expert order
 *                                  (first token_nrows[t] entries written)
 *   token_nrows  [T] int32         number of experts that chose token t
 * The forward then runs moe_grouped_ffn_weighted(x, gather_rows =
 * sorted_token, P = E*capacity, row_w) and moe_combine_rows. Workspace:
 * moe_expert_choice_workspace_size(T,E) bytes, 16-byte aligned. */
size_t moe_expert_choice_workspace_size(int64_t T, int E);
int moe_expert_choice(const float *logits, int64_t T, int E, int capacity, int32_t *offsets,
                      int32_t *sorted_token, float *row_w, int32_t *token_rows,
                      int32_t *token_nrows, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Combine by per-token row lists: out[t] = sum over i < token_nrows[t]
 * (ascending) of y[token_rows[t*E + i]] (+ y_sh[t]), fp32, rounded once to
 * dtype. y [P,h] (already weighted), out [T,h]. */
int moe_combine_rows(const void *y, int dtype, int64_t T, int64_t h, int E, int64_t P,
                     const int32_t *token_rows, const int32_t *token_nrows, const void *y_sh,
                     void *out, void *stream);

/* =============================== backward ===============================
 * Gradients of L = sum(grad_out * out) (grad_out = dL/dout). Top-k indices
 * carry no gradient. Order of use: moe_unpermute_bwd, moe_grouped_ffn_bwd,
 * moe_route_bwd, moe_permute_bwd.
 */

/* Combine backward: grad_y[row_of[t,j]] = topk_w[t,j] * grad_out[t] (dtype)
 * and grad_topk_w[t,j] = <grad_out[t], y[row_of[t,j]]> (fp32). With
 * topk_w = NULL (the unweighted combine of weighted expert outputs):
 * grad_y[row_of[t,j]] = grad_out[t]; y and grad_topk_w are then not used and
 * may be NULL. */
int moe_unpermute_bwd(const void *grad_out, const void *y, int dtype, int64_t T, int64_t h,
                      int k, const int32_t *row_of, const float *topk_w, void *grad_y,
                      float *grad_topk_w, void *stream);

/* Grouped FFN backward. Per segment e with rows X_e of x_perm, the
 * activation act and the pre-activations gu the forward kept:
 *   dact = grad_y W2[e]
 *   SwiGLU (gu = [g u]): dg = dact * u * silu'(g), du = dact * silu(g),
 *                        dA = [dg du] [P,2F]
 *   GELU (gu = a = X W1[e]^T + b1[e]): dA = dact * gelu'(a) [P,F],
 *                        gelu'(a) = Phi(a) + a phi(a)
 *   grad_w2[e] = grad_y_e^T act_e          [h,F]    fp32
 *   grad_w1[e] = dA_e^T X_e                [n1F,h]  fp32 (zeros for an empty e)
 *   grad_x_perm = dA W1[e]                 [P,h]    dtype
 *   grad_b1[e] = column sums of dA_e       [n1F]    fp32 (NULL: not computed)
 *   grad_b2[e] = column sums of grad_y_e   [h]      fp32 (NULL: not computed)
 * grad_gu [P,n1F] dtype is caller-provided scratch that receives dA. bf16
 * SwiGLU runs on the matrix-core kernels; GELU (bf16 or fp32) and fp32
 * SwiGLU on a plainer fp32-FMA segmented GEMM (the small layers that use
 * them). Sums run in a fixed order (deterministic). */
int moe_grouped_ffn_bwd(const void *grad_y, const void *x_perm, const void *act,
                        const void *gu, int dtype, int64_t P, int64_t h, int64_t F, int E,
                        const int32_t *offsets, int act_kind, const void *w1, const void *w2,
                        void *grad_gu, void *grad_x_perm, float *grad_w1, float *grad_w2,
                        float *grad_b1, float *grad_b2, void *stream);

/* Grouped FFN backward with the activation recomputed ("Scalable Training ...
 * with Megatron Core", section 4.1.2, recomputing the activation function):
 * act is not read; act = p * silu(g) * u is rebuilt from gu in the workspace
 * (p = row_w[r], or 1 when row_w is NULL), with the forward epilogue's
 * expression. With row_w (memory-efficient permutation, see
 * moe_grouped_ffn_weighted; grad_y is then the unweighted
 * moe_unpermute_bwd result):
 *   dact = grad_y W2[e];  da = p dact;  (dg, du) from da as above
 *   grad_row_w[r] = <dact_r, silu(g_r) * u_r>   [P] fp32 (dL/dp; fixed-order
 *                                               sum, moe_permute_weights_bwd
 *                                               maps it to [T,k])
 *   grad_w2[e] = grad_y_e^T act_e, grad_w1, grad_x_perm as above.
 * row_w and grad_row_w are both NULL or both set. Workspace:
 * moe_grouped_ffn_bwd_recompute_workspace_size(P, F, row_w != NULL) bytes of
 * 16-byte aligned device memory. bf16 SwiGLU only. */
size_t moe_grouped_ffn_bwd_recompute_workspace_size(int64_t P, int64_t F, int weighted);
int moe_grouped_ffn_bwd_recompute(const void *grad_y, const void *x_perm, const void *gu,
                                  int dtype, int64_t P, int64_t h, int64_t F, int E,
                                  const int32_t *offsets, int act_kind, const void *w1,
                                  const void *w2, const float *row_w, void *grad_gu,
                                  void *grad_x_perm, float *grad_w1, float *grad_w2,
                                  float *grad_row_w, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Router backward. grad_logits_sel[t,j] = dL/dl for the selected expert
 * topk_idx[t,j] (unselected logits get 0):
 *   softmax:  w_j (g_j - sum_i w_i g_i)
 *   sigmoid:  s_j (1 - s_j) / S (g_j - sum_i w_i g_i), s = sigma(l), S = sum s
 * with g = grad_topk_w. Then, segment by segment of the permutation,
 *   grad_w_gate[e] = sum over rows r of e (ascending) of dl(r) x[sorted_token[r]]
 *   grad_b_gate[e] = sum of the same dl(r)
 * (grad_w_gate [E,h] fp32, grad_b_gate [E] fp32 or NULL). logits [T,E] fp32 is
 * read for sigmoid only (may be NULL for softmax). Workspace:
 * moe_route_bwd_workspace_size(T,h,E,k) bytes of device memory. */
size_t moe_route_bwd_workspace_size(int64_t T, int64_t h, int E, int k);
int moe_route_bwd(const void *x, int dtype, int64_t T, int64_t h, int E, int k, int score,
                  const float *logits, const int32_t *topk_idx, const float *topk_w,
                  const float *grad_topk_w, const int32_t *offsets,
                  const int32_t *sorted_token, float *grad_logits_sel, float *grad_w_gate,
                  float *grad_b_gate, void *workspace, size_t workspace_bytes, void *stream);

/* Dispatch backward plus the router's input gradient, one rounding:
 *   grad_x[t] = sum_j grad_x_perm[row_of[t,j]]
 *             + sum_j grad_logits_sel[t,j] * w_gate[topk_idx[t,j]]
 * (the second sum is skipped when grad_logits_sel is NULL). */
int moe_permute_bwd(const void *grad_x_perm, int dtype, int64_t T, int64_t h, int k,
                    const int32_t *row_of, const float *grad_logits_sel,
                    const int32_t *topk_idx, const void *w_gate, int E, void *grad_x,
                    void *stream);

/* ------------------------------------------------ auxiliary router losses
 *
 * "emerging-techniques-moe-training", section 3 (Load Balancing): the
 * load-balancing loss and the router z-loss, both on the router's logits l
 * [T,E] fp32 as moe_route writes them (gate bias included, selection bias
 * not), for either scoring function:
 *   aux = E * sum_e f_e P_e,  f_e = counts[e] / (T k),
 *                             P_e = mean_t softmax(l_t)_e (over all E)
 *   z   = mean_t logsumexp(l_t)^2
 * counts [E] int32 are the per-expert routing counts moe_route writes
 * (offsets[e+1] - offsets[e] serves as well). f_e is piecewise constant in l
 * and carries no gradient. Supported: k <= E <= 256. T = 0 gives
 * aux = z = 0. Sums over tokens run in a fixed order (deterministic). */
size_t moe_router_losses_workspace_size(int64_t T, int E);
/* losses [2] fp32 device: {aux, z}. probs_mean [E] fp32 (P_e) or NULL.
 * Workspace: moe_router_losses_workspace_size(T,E) bytes of device memory
 * (0 and NULL allowed when T = 0). */
int moe_router_losses(const float *logits, const int32_t *counts, int64_t T, int E, int k,
                      float *losses, float *probs_mean, void *workspace, size_t workspace_bytes,
                      void *stream);
/* grad_logits [T,E] fp32 = d(coef_aux * aux + coef_z * z)/dl (written, not
 * accumulated):
 *   coef_aux (E/T) p_tj (f_j - sum_e f_e p_te) + coef_z (2/T) lse_t p_tj,
 * p_t = softmax(l_t), lse_t = logsumexp(l_t). */
int moe_router_losses_bwd(const float *logits, const int32_t *counts, int64_t T, int E, int k,
                          float coef_aux, float coef_z, float *grad_logits, void *stream);

/* Router backward of a dense logit gradient D [T,E] fp32 (such as
 * moe_router_losses_bwd's), ACCUMULATED into the gradients that
 * moe_route_bwd and moe_permute_bwd wrote (call it after them):
 *   grad_w_gate [E,h] fp32 += D^T x       (NULL: skipped; needs x)
 *   grad_b_gate [E] fp32   += column sums of D   (NULL: skipped)
 *   grad_x [T,h] dtype     += D w_gate    (NULL: skipped; needs w_gate;
 *                             the sum is formed in fp32, then added and
 *                             rounded once to dtype)
 * x [T,h] and w_gate [E,h] are dtype. Sums run in a fixed order. Needs
 * h % 64 == 0, E <= 256, 16-byte aligned x, w_gate, grad_w_gate, grad_x and
 * workspace. With bf16 and E a multiple of 32 (and T * max(h, 2E) < 2^31)
 * the two products run on the matrix cores: D is split into bf16 parts
 * hi + lo (|D - hi - lo| <= 2^-16 |D| or so), every product of bf16 values is
 * exact in fp32 and the sums are fp32; there D w_gate is rounded to bf16
 * before the add, so grad_x takes two roundings. Workspace:
 * moe_router_dense_bwd_workspace_size(T,h,E) bytes of device memory
 * (required for grad_w_gate, and for grad_x on the matrix-core path). */
size_t moe_router_dense_bwd_workspace_size(int64_t T, int64_t h, int E);
int moe_router_dense_bwd(const void *x, const void *w_gate, int dtype, int64_t T, int64_t h,
                         int E, const float *grad_logits, float *grad_w_gate,
                         float *grad_b_gate, void *grad_x, void *workspace,
                         size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
