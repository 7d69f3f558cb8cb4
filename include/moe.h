/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer hot path.
 *
 * One Mixture-of-Experts layer, forward and backward, on one GPU, in the four
 * stages of "Scalable Training of Mixture-of-Experts Models with Megatron
 * Core" (section 2, Megatron-Core MoE Architecture):
 *   Route    -- router logits, probabilities, top-k experts, routing weights
 *   Dispatch -- tokens permuted by destination expert (expert-contiguous rows)
 *   Compute  -- all experts' SwiGLU FFNs as one grouped GEMM over ragged rows
 *   Combine  -- rows return to sequence order, weighted by the routing
 *               weights, plus an optional shared expert's output
 * and their backward passes.  The router stays in FP32 (section 5, Selective
 * precision).
 *
 * Conventions (every entry point):
 *   - Tensor arguments are DEVICE pointers to contiguous row-major arrays on
 *     the current HIP device; scalars are host values.  `stream` is a
 *     hipStream_t (NULL = the default stream).
 *   - Every call validates its arguments on the host first.  On failure it
 *     returns a negative moe_status, enqueues nothing and sets a thread-local
 *     message (moe_last_error).  On success it enqueues kernels on `stream`
 *     and returns MOE_OK without synchronising; outputs are valid once the
 *     stream reaches the call.  No call allocates device memory, copies device
 *     to host, or keeps a pointer after returning; the caller owns every
 *     buffer, including workspaces sized by the *_workspace_bytes functions.
 *   - Device-resident index data (offsets, dst_row, topk_idx) is range-checked
 *     inside the kernels: entries outside the valid range are skipped, never
 *     dereferenced.  Results for such inputs are unspecified.
 *   - Identical inputs give bit-identical outputs (no order-deciding atomics).
 *   - Sizes are 64-bit.  The kernels address with 64-bit offsets, except the
 *     grouped GEMMs (bf16, fp8, MXFP8), whose buffer resources take 32-bit
 *     byte offsets inside one group's slab: hence their per-expert limits
 *     (K * N, M * K, M * N below 2^31 or 2^32 bytes, as stated per call).
 *   - Zero-sized problems (T == 0, M == 0) are valid; a weight gradient of an
 *     empty group is written as zeros (or left unchanged when accumulating).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* a size is negative or inconsistent */
  MOE_ERR_DTYPE = -3,       /* unknown dtype or unsupported dtype combination */
  MOE_ERR_UNSUPPORTED = -4, /* valid request outside the library's limits */
  MOE_ERR_WORKSPACE = -5,   /* workspace missing or too small */
  MOE_ERR_HIP = -6          /* a HIP runtime call or launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;  /* fp8 codes are uint8_t arrays */
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score;
typedef enum {
  MOE_EPI_NONE = 0,
  MOE_EPI_SWIGLU = 1,     /* forward GEMM 1: also write H = silu(A) * B */
  MOE_EPI_SWIGLU_BWD = 2  /* dgrad of GEMM 2: turn dH into dAB in the epilogue */
} moe_epilogue;

/* Text for a status code; never NULL. */
const char* moe_status_string(int status);
/* Detail of the last failing call on this host thread ("" if none). */
const char* moe_last_error(void);
/* ABI version of this header: 2. */
int moe_abi_version(void);

/* ---------------------------------------------------------------- Route -- */

/* Router projection, forward (section 2, Route: token hidden states to expert
 * logits; section 5, Selective precision: the router stays in FP32).
 *   logits[t, e] = fp32( sum_i x[t, i] * w_r[i, e] ) + logit_bias[e]
 * fp32 multiply-adds on the vector ALUs (bf16 x widened exactly), each output
 * one sequential sum in a fixed order (deterministic); the bias is one fp32
 * addition after the sum.  The matrix cores are not used.
 *   x          [T, d]  x_dtype (MOE_F32 or MOE_BF16)
 *   w_r        [d, E]  fp32
 *   logit_bias [E]     fp32 or NULL: a per-expert constant added to the
 *                      logits before scoring (no gradient)
 *   logits     [T, E]  fp32 out: the selection key of moe_route_topk
 * Limits: 1 <= E <= 1024, d >= 1. */
int moe_router_logits(const void* x, int x_dtype, const float* w_r, const float* logit_bias,
                      int64_t T, int64_t d, int32_t E, float* logits, void* stream);

/* Router projection, backward: d_w_r = x^T d_logits ([d, E], fp32, overwritten)
 * and dx_router = d_logits w_r^T ([T, d], fp32, overwritten), fp32
 * multiply-adds on the vector ALUs as in the forward.  Either output may be
 * NULL to skip it. */
int moe_router_logits_bwd(const void* x, int x_dtype, const float* w_r, const float* d_logits,
                          int64_t T, int64_t d, int32_t E, float* d_w_r, float* dx_router,
                          void* stream);

/* The same two products as moe_router_logits_bwd when every row of d_logits
 * is zero outside the token's k chosen experts -- what moe_route_topk_bwd
 * gives for renormalised routing or sigmoid scores, and not for softmax
 * without renormalisation or with the auxiliary loss added (use
 * moe_router_logits_bwd for those).  Reads d_logits only at the chosen
 * entries: T k d multiply-adds per product instead of T E d, fp32 on the
 * vector ALUs, each output summed in a fixed order:
 *   dx_router[t] = sum_j d_logits[t, e_j] w_r[:, e_j]   (slots in order)
 *   d_w_r[:, e]  = sum over expert e's rows r (ascending) of
 *                  x[src_token[r]] d_logits[src_token[r], e]
 * topk_idx [T, k]; offsets [E+1] and src_token [T*k]: the DROPLESS dispatch
 * map of the route (before any capacity dropping, whose dropped pairs still
 * carry gradient to their keys).  Entries outside range are skipped.
 * Limits: E <= 256, k <= 64, d % 8 == 0, x 16-byte aligned. */
int moe_router_logits_bwd_topk(const void* x, int x_dtype, const float* w_r, const float* d_logits,
                               const int32_t* topk_idx, const int64_t* offsets,
                               const int32_t* src_token, int64_t T, int64_t d, int32_t E,
                               int32_t k, float* d_w_r, float* dx_router, void* stream);

/* Non-finite logits are a caller error (the routing of such a token is
 * unspecified).  This check flags them: *status (device int32) is set to 1
 * when any of x[0 .. n) is a NaN or an infinity, and is never cleared by the
 * library.  x must be 16-byte aligned.  The layer calls it on the logits
 * when the environment variable MOE_CHECK_FINITE is set. */
int moe_check_finite(const float* x, int64_t n, int32_t* status, void* stream);

/* Bytes of workspace moe_route_topk needs (device memory, any contents). */
size_t moe_route_topk_workspace_bytes(int64_t T, int32_t E, int32_t k);

/* Top-k selection, routing weights and the dispatch map (section 2, Route and
 * Dispatch).  Dropless: all T*k (token, slot) pairs get a permuted row.
 *   logits    [T, E] fp32 keys (bias already added).  Must be finite.
 *   selection: per token the k experts of largest key; equal keys go to the
 *              lower expert index; slots are listed by key descending, then
 *              index ascending.
 *   topk_idx  [T, k] int32 out
 *   topk_w    [T, k] fp32 out: score = MOE_SOFTMAX: softmax of the keys over
 *              the k chosen (renorm != 0) or over all E (renorm == 0);
 *              MOE_SIGMOID: sigmoid(key), divided by the sum over the chosen
 *              k when renorm != 0
 *   counts    [E]    int32 out: rows routed to each expert
 *   offsets   [E+1]  int64 out: exclusive prefix sum of counts (offsets[E] = T*k)
 *   dst_row   [T, k] int32 out: permuted row of (t, j); rows of expert e are
 *              offsets[e] .. offsets[e+1]-1 in ascending token order
 *   src_token [T*k]  int32 out: token of each permuted row (inverse of dst_row)
 *   workspace moe_route_topk_workspace_bytes(T, E, k) bytes
 * Limits: 1 <= k <= E <= 1024, T * k < 2^31. */
int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int score, int renorm,
                   int32_t* topk_idx, float* topk_w, int32_t* counts, int64_t* offsets,
                   int32_t* dst_row, int32_t* src_token, void* workspace, size_t workspace_bytes,
                   void* stream);

/* moe_route_topk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same results, with the workspace taken from a fixed 4 MiB array that
 * the library holds on each device until the process ends (no hipMalloc,
 * hipFree or allocating library call).  Arguments as moe_route_topk, without
 * the workspace.  Limit: ceil(T / 64) * E * 12 + 256 <= 4 MiB (e.g. T up to
 * 87,000 tokens at E = 256), else MOE_ERR_UNSUPPORTED.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.  The first
 * call on a device looks the array's address up (hipGetSymbolAddress). */
int moe_route_topk_noalloc(const float* logits, int64_t T, int32_t E, int32_t k, int score,
                           int renorm, int32_t* topk_idx, float* topk_w, int32_t* counts,
                           int64_t* offsets, int32_t* dst_row, int32_t* src_token, void* stream);

/* Debug check of a dispatch map (moe_route_topk, _replay, _expert_bias,
 * moe_apply_capacity, moe_pad_to_max): each violated invariant ORs one bit
 * into *status (device int32, never cleared by the library):
 *   1  offsets[0] != 0, decreasing offsets, a segment shorter than its
 *      count, or offsets[E] > n_rows
 *   2  a pair's row outside its expert's filled segment
 *      [offsets[e], offsets[e] + counts[e]) (row -1, a dropped pair, is allowed)
 *   4  src_token[row] is not the pair's token
 *   8  a segment's tokens not in ascending order
 *   16 a pair's expert outside [0, E)
 * n_rows: rows of the permuted buffers (T*k dropless, E*capacity padded).
 * Reads only, every index range-checked first, so a corrupt map is safe to
 * check.  The layer runs it after each route when the environment variable
 * MOE_DEBUG is set. */
int moe_check_dispatch(const int32_t* topk_idx, const int32_t* counts, const int64_t* offsets,
                       const int32_t* dst_row, const int32_t* src_token, int64_t T, int32_t E,
                       int32_t k, int64_t n_rows, int32_t* status, void* stream);

/* Top-k with a selection-only expert bias on sigmoid scores (the
 * auxiliary-loss-free biasing of section 7, Load Balancing): the key of
 * expert e is sigmoid_spec(logits[t, e]) + sel_bias[e] (one fp32 addition);
 * selection, slot order and the dispatch map as in moe_route_topk on those
 * keys; the routing weights are the UNBIASED scores sigmoid_spec(logits) of
 * the chosen experts, divided by their sum over the k when renorm != 0.
 * sigmoid_spec is a fixed sequence of correctly rounded fp32 operations, so
 * that any implementation can reproduce the keys bit for bit:
 *   x = min(max(-z, -87), 87);  n = rint(x * 1.44269504f)  (ties to even)
 *   r = (x - n * 0.693145751953125f) - n * 1.42860677e-06f
 *   p = 1/5040; p = p * r + c for c = 1/720, 1/120, 1/24, 1/6, 1/2, 1, 1
 *       (the fp32 values of 1/i!; a multiply, then an add: no fused multiply-add)
 *   sigmoid_spec(z) = 1 / (1 + p * 2^n)
 * sel_bias [E] fp32; other arguments as in moe_route_topk (workspace from
 * moe_route_topk_workspace_bytes). */
int moe_route_topk_expert_bias(const float* logits, const float* sel_bias, int64_t T, int32_t E,
                               int32_t k, int renorm, int32_t* topk_idx, float* topk_w,
                               int32_t* counts, int64_t* offsets, int32_t* dst_row,
                               int32_t* src_token, void* workspace, size_t workspace_bytes,
                               void* stream);

/* The expert-bias update that follows each step: with L = sum(counts) and
 * E experts, sel_bias[e] += rate * sign(L - E * counts[e]) (fp32; the sign
 * from exact integers): an expert above the mean load becomes less
 * attractive, one below it more.  counts [E] int32 (the routed loads, before
 * any dropping); sel_bias [E] fp32 in/out.  E <= 1024. */
int moe_expert_bias_update(const int32_t* counts, int32_t E, float rate, float* sel_bias,
                           void* stream);

/* Router replay: routing with the experts given (e.g. recorded from an
 * earlier pass, or a forced assignment such as the balanced routing of the
 * benchmark setting in section 8, Performance Evaluation), the routing weights
 * recomputed from the keys exactly as in moe_route_topk, and the same
 * dispatch map.  Arguments as moe_route_topk, plus:
 *   topk_idx_in [T, k] int32: expert of each (t, j), slots in the given order.
 *               A slot outside [0, E) or repeating an earlier slot of its
 *               token is replaced, in slot order, by the smallest expert the
 *               token does not use yet (so the dispatch map stays a
 *               bijection); topk_idx receives the experts used.
 *   status      int32 device word or NULL: set to 1 when a slot was replaced
 *               (never cleared by the library).
 *   workspace   moe_route_topk_workspace_bytes(T, E, k) bytes
 * Limits as moe_route_topk.  The backward is moe_route_topk_bwd. */
int moe_route_replay(const float* logits, const int32_t* topk_idx_in, int64_t T, int32_t E,
                     int32_t k, int score, int renorm, int32_t* topk_idx, float* topk_w,
                     int32_t* counts, int64_t* offsets, int32_t* dst_row, int32_t* src_token,
                     int32_t* status, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace moe_aux_loss needs to produce the loss value. */
size_t moe_aux_loss_workspace_bytes(int64_t T, int32_t E);

/* Auxiliary load-balancing loss (section 7, Load Balancing: auxiliary loss):
 *   loss = coeff * E * sum_e f_e * P_e,
 *   f_e = counts[e] / (T k)                  (fraction of routed pairs; no gradient)
 *   P_e = (1/T) sum_t p[t, e],  p[t, .] = softmax of the keys (MOE_SOFTMAX) or
 *         the sigmoid scores divided by their sum over the E experts (MOE_SIGMOID).
 *   logits [T, E] fp32 keys; counts [E] int32 (of moe_route_topk / _replay).
 *   loss     fp32 device scalar out, or NULL (no workspace needed then)
 *   d_logits [T, E] fp32 or NULL: dloss/dlogits is ADDED (call after
 *            moe_route_topk_bwd, which overwrites d_logits)
 * Deterministic (fixed-order sums).  Limits as moe_route_topk, T >= 1. */
int moe_aux_loss(const float* logits, const int32_t* counts, int64_t T, int32_t E, int32_t k,
                 int score, float coeff, float* loss, float* d_logits, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Capacity-limited dropping (section 7, Load Balancing: capacity-limited
 * dropping), applied to the dispatch map of moe_route_topk or
 * moe_route_replay: expert e keeps the first `capacity` of its (token, slot)
 * pairs in token order -- the first rows of its segment -- and drops the rest.
 *   counts_out [E]    int32: kept rows per expert (min(counts, capacity))
 *   offsets_out [E+1] int64: their exclusive prefix sum
 *   dst_row_out [T,k] int32: new row of each kept pair, -1 for a dropped one
 *   src_token_out     int32: token of each kept row; entries at and past
 *                     offsets_out[E] are not written
 * A dropped pair contributes nothing downstream (permute, combine and their
 * backward skip rows < 0; the grouped GEMMs see only the kept segments); the
 * routing weights are left as computed.  Outputs must not alias the inputs.
 * The usual capacity is ceil(capacity_factor * T * k / E). */
int moe_apply_capacity(const int32_t* topk_idx, const int32_t* counts, const int64_t* offsets,
                       const int32_t* dst_row, int64_t T, int32_t E, int32_t k, int64_t capacity,
                       int32_t* counts_out, int64_t* offsets_out, int32_t* dst_row_out,
                       int32_t* src_token_out, void* stream);

/* Pad-to-max (section 7, Load Balancing: variable expert counts turned into
 * static shapes): from a dropless dispatch map (moe_route_topk,
 * moe_route_replay, moe_route_topk_expert_bias), a layout in which every
 * expert owns `capacity` rows at e * capacity.  A pair whose rank in its
 * expert's token order is below the capacity keeps that rank as its row
 * offset; the others are dropped (the pairs capacity-limited dropping keeps).
 *   counts_out [E]      int32: min(counts, capacity)
 *   offsets_out [E+1]   int64: e * capacity (static)
 *   dst_row_out [T, k]  int32: padded row of each kept pair, -1 if dropped
 *   src_token_out [E * capacity] int32: token of each row, -1 on padding
 * Padding rows carry no pair: permute writes nothing there and combine never
 * reads them; moe_zero_unmapped_rows clears them in the buffers the grouped
 * GEMMs read (the permuted activations and dY), so that they stay zero
 * through every GEMM.  Outputs must not alias the inputs.  E * capacity <
 * 2^31. */
int moe_pad_to_max(const int32_t* topk_idx, const int32_t* counts, const int64_t* offsets,
                   const int32_t* dst_row, const int32_t* src_token, int64_t T, int32_t E,
                   int32_t k, int64_t capacity, int32_t* counts_out, int64_t* offsets_out,
                   int32_t* dst_row_out, int32_t* src_token_out, void* stream);

/* Writes zeros to every row r < M of buf [M, d] (`dtype`) with
 * src_token[r] < 0 -- the padding rows of a pad-to-max layout.  Rows of d
 * elements must be a multiple of 16 bytes. */
int moe_zero_unmapped_rows(void* buf, int dtype, const int32_t* src_token, int64_t M, int64_t d,
                           void* stream);

/* Gradient of the routing weights with respect to the keys (the selection
 * itself carries none).  With g = sum_j w_j dw_j over a token's chosen slots:
 *   softmax, renorm   : d_logits[e_j] = w_j (dw_j - g), 0 elsewhere
 *   softmax, no renorm: d_logits[e]   = p_e (G_e - g) for all e, where p is the
 *                       softmax over all E and G_e = dw_j if e = e_j else 0
 *   sigmoid, renorm   : d_logits[e_j] = (dw_j - g) / S * s_j (1 - s_j), S = sum s_j
 *   sigmoid, no renorm: d_logits[e_j] = dw_j s_j (1 - s_j)
 * logits [T, E], topk_idx/topk_w/d_topk_w [T, k] as produced above;
 * d_logits [T, E] fp32 out (every entry written). */
int moe_route_topk_bwd(const float* logits, const int32_t* topk_idx, const float* topk_w,
                       const float* d_topk_w, int64_t T, int32_t E, int32_t k, int score,
                       int renorm, float* d_logits, void* stream);

/* ------------------------------------------------------------- Dispatch -- */

/* Permute tokens into expert-contiguous rows (section 2, Dispatch):
 *   x_perm[dst_row[t, j]] = x[t]     for all t < T, j < k
 * x [T, d] and x_perm [n_rows, d] of `dtype`; each token row is read once.
 * n_rows: rows of the permuted buffer, T*k for the dropless layout (also
 * after capacity dropping), E*capacity for pad-to-max; dst_row entries < 0
 * (dropped pairs) or >= n_rows are skipped, here and in the three calls
 * below that take n_rows.
 * Limits: d % 8 == 0 (bf16) or d % 4 == 0 (fp32). */
int moe_permute(const void* x, int dtype, const int32_t* dst_row, int64_t T, int64_t d, int32_t k,
                int64_t n_rows, void* x_perm, void* stream);

/* Adjoint of moe_permute plus optional addends (fp32 accumulation, one
 * rounding to `dtype`):
 *   dx[t] = sum_j dx_perm[dst_row[t, j]] + addend[t] + addend_f32[t]
 * dx_perm [n_rows, d], dx [T, d], addend [T, d] of `dtype` or NULL,
 * addend_f32 [T, d] fp32 or NULL. */
int moe_permute_bwd(const void* dx_perm, int dtype, const int32_t* dst_row, int64_t T, int64_t d,
                    int32_t k, int64_t n_rows, const void* addend, const float* addend_f32,
                    void* dx, void* stream);

/* -------------------------------------------------------------- Compute -- */

/* Grouped GEMM over G groups of contiguous rows (section 2, Expert
 * Computation: the local experts' GEMMs run together).  Group g owns rows
 * offsets[g] .. offsets[g+1]-1 of the M rows; offsets is DEVICE int64 [G+1],
 * non-decreasing, offsets[0] = 0, offsets[G] = M (rows outside every group
 * are left untouched).  A, B and outputs share `dtype` (MOE_BF16: bf16 MFMA
 * with fp32 accumulation; MOE_F32: fp32 FMA).
 *
 * Forward:  C[rows g] = A[rows g] . B[g]     A [M, K], B [G, K, N], C [M, N]
 *   epilogue MOE_EPI_NONE  : write C.
 *   epilogue MOE_EPI_SWIGLU: N = 2f, columns [0, f) are the gate a and [f, 2f)
 *     the up projection b; write C (may be NULL to skip) and
 *     H [M, f] = silu(a) * b, silu(a) = a / (1 + exp(-a)), from the fp32 sums.
 * Limits (bf16): K % 64 == 0, N % 128 == 0 (SWIGLU: f % 64 == 0), K * N < 2^31
 *        (one expert's weights under 4 GiB); (fp32): none beyond sizes >= 1.
 *        G <= 1024. */
int moe_grouped_gemm_fwd(const void* A, const void* B, const int64_t* offsets, int32_t G, int64_t M,
                         int64_t K, int64_t N, int dtype, int epilogue, void* C, void* H,
                         void* stream);

/* Data gradient: dA[rows g] = dC[rows g] . B[g]^T    dC [M, N], B [G, K, N], dA [M, K].
 *   epilogue MOE_EPI_SWIGLU_BWD: the product is dH [M, K] of a SwiGLU whose
 *     pre-activations are ab [M, 2K] (a = ab[:, :K], b = ab[:, K:]); write
 *     dA = dAB [M, 2K] with dAB[:, :K] = dH * b * s * (1 + a (1 - s)),
 *     dAB[:, K:] = dH * silu(a), s = sigmoid(a).  `ab` is NULL otherwise.
 * Limits (bf16): N % 64 == 0, K % 128 == 0, K * N < 2^31.  (fp32): none.
 * G <= 1024. */
int moe_grouped_gemm_dgrad(const void* dC, const void* B, const int64_t* offsets, int32_t G,
                           int64_t M, int64_t K, int64_t N, int dtype, int epilogue,
                           const void* ab, void* dA, void* stream);

/* Weight gradient: dB[g] = A[rows g]^T . dC[rows g]   A [M, K], dC [M, N], dB [G, K, N].
 * The contraction runs over each group's rows (ragged).  dB_dtype is `dtype`
 * or MOE_F32.  accumulate != 0 adds into dB instead of overwriting it.
 * Limits (bf16): K % 128 == 0, N % 128 == 0, M * K < 2^31, M * N < 2^31.
 * (fp32): none.  G <= 1024. */
int moe_grouped_gemm_wgrad(const void* A, const void* dC, const int64_t* offsets, int32_t G,
                           int64_t M, int64_t K, int64_t N, int dtype, int dB_dtype,
                           int accumulate, void* dB, void* stream);

/* SwiGLU on its own: h [M, f] = silu(ab[:, :f]) * ab[:, f:], ab [M, 2f]. */
int moe_swiglu(const void* ab, int dtype, int64_t M, int64_t f, void* h, void* stream);

/* SwiGLU backward on its own: dab [M, 2f] from dh [M, f] and ab [M, 2f]
 * (formulas as in MOE_EPI_SWIGLU_BWD). */
int moe_swiglu_bwd(const void* dh, const void* ab, int dtype, int64_t M, int64_t f, void* dab,
                   void* stream);

/* ------------------------------------------------------- FP8 (E4M3) -- */
/* Blockwise FP8 ("Scalable Training of Mixture-of-Experts Models with Megatron
 * Core", section 5, Platform-specific recipes): 1 x 128 tiles for activations
 * and gradients, 128 x 128 blocks for weights, fp32 scales.  Codes are OCP
 * E4M3 (bias 7, no infinities, largest finite 448).  Per block:
 *   amax = max |v|,  scale = amax / 448,  inv = 448 / amax   (one IEEE fp32
 *   division each; scale = inv = 1 when amax = 0),
 *   code = nearest E4M3 value of fp32(v * inv), ties to the even code,
 *   saturated to +-448;  value = decode(code) * scale.
 * The weight gradients contract over tokens, so their operands use 128-token
 * x 1 tiles, each group's rows zero-padded to a multiple of 128.  Layouts are
 * those the fp8 grouped GEMM reads (every operand k-contiguous, every scale a
 * contiguous vector over a 128-row tile).  All inputs are bf16.
 * Limits: K and N multiples of 128 wherever they are blocked. */

/* 1 x 128 tiles along rows: q [M, K] codes, scale_t [K/128, M] (block-major). */
int moe_quant_fp8_rows(const void* x, int64_t M, int64_t K, uint8_t* q, float* scale_t,
                       void* stream);

/* 128 x 128 blocks of w [G, K, N]: ONE code array q [G, K, N] in w's own
 * layout, which both GEMMs read (a block's scale serves either orientation),
 * and the block scale s[g][kb][nb] expanded along each GEMM's output columns:
 *   s_fwd [G, K/128, N] = s[g][kb][n / 128]   (forward)
 *   s_dgrad [G, N/128, K] = s[g][k / 128][nb]  (dgrad)
 * w 16-byte and q 8-byte aligned. */
int moe_quant_fp8_weights(const void* w, int32_t G, int64_t K, int64_t N, uint8_t* q,
                          float* s_fwd, float* s_dgrad, void* stream);

/* Host helper: rows a padded layout of M rows in G groups can need,
 * M + G * (align - 1) rounded up to align (the row length `ldm` of the
 * token-tile operands); 0 for M < 0, G < 1, align < 1 or M > 2^60. */
int64_t moe_padded_rows_bound(int64_t M, int32_t G, int32_t align);

/* padded [G+1] (device): padded[0] = 0, padded[g+1] = padded[g] +
 * round_up(offsets[g+1] - offsets[g], align).  1 <= G <= 1024. */
int moe_padded_offsets(const int64_t* offsets, int32_t G, int64_t M, int32_t align,
                       int64_t* padded, void* stream);

/* 128-token x 1 tiles of x [M, K]: group g's rows offsets[g].. land at padded
 * rows padded[g].. (zero codes past the group's end); written transposed,
 * q_t [K, ldm] (row c holds column c's codes), scale [ldm/128, K].
 * ldm = moe_padded_rows_bound(M, G, 128) or larger, a multiple of 128. */
int moe_quant_fp8_token_tiles(const void* x, const int64_t* offsets, const int64_t* padded,
                              int32_t G, int64_t M, int64_t K, int64_t ldm, uint8_t* q_t,
                              float* scale, void* stream);

/* fp8 grouped GEMMs, fp32 accumulation, each 128-wide k block promoted with
 * its two scales; outputs bf16 (dB: bf16 or fp32).  Groups as in the bf16
 * calls.  Epilogues as in the bf16 calls.
 *   forward: C[rows g] = deq(A)[rows g] . deq(B_g)   A [M, K] + scale_t [K/128, M]
 *            from moe_quant_fp8_rows; B = q [G, K, N] from moe_quant_fp8_weights
 *            with s_fwd (the weights' own layout, read transposed)
 *   dgrad:   dA[rows g] = deq(dC)[rows g] . deq(B_g)^T   dC [M, N] + scale_t
 *            [N/128, M]; B = the same q [G, K, N] with s_dgrad
 *   wgrad:   dB[g] = deq(A)^T . deq(dC) over group g's padded rows; A_t [K, ldm],
 *            dC_t [N, ldm] and scales from moe_quant_fp8_token_tiles
 * Limits: K % 128 == 0, N % 128 == 0 (forward SWIGLU: N / 2 % 64 == 0),
 * K * N < 2^32 (one expert's weight codes under 4 GiB). */
int moe_grouped_gemm_fp8_fwd(const uint8_t* A, const float* a_scale_t, const uint8_t* B,
                             const float* b_scale_fwd, const int64_t* offsets, int32_t G,
                             int64_t M, int64_t K, int64_t N, int epilogue, void* C, void* H,
                             void* stream);
int moe_grouped_gemm_fp8_dgrad(const uint8_t* dC, const float* dc_scale_t, const uint8_t* B_dgrad,
                               const float* b_scale_dgrad, const int64_t* offsets, int32_t G,
                               int64_t M, int64_t K, int64_t N, int epilogue, const void* ab,
                               void* dA, void* stream);
int moe_grouped_gemm_fp8_wgrad(const uint8_t* A_t, const float* a_scale, const uint8_t* dC_t,
                               const float* dc_scale, const int64_t* padded, int32_t G,
                               int64_t ldm, int64_t K, int64_t N, int dB_dtype, int accumulate,
                               void* dB, void* stream);

/* ----------------------------------------------------------------- MXFP8 -- */
/* The microscaling FP8 recipe (section 5, Platform-specific recipes), in the
 * OCP Microscaling Formats encoding: every operand of every expert GEMM is
 * quantized in blocks of 32 consecutive elements along its contraction axis,
 * each block sharing one E8M0 scale byte that the gfx950 matrix cores apply
 * themselves (v_mfma_scale_f32_32x32x64_f8f6f4).  Per block:
 *   X = floor(log2(amax)) - 8, clamped to [-127, 127]  (X = -127 if amax = 0)
 *   byte = X + 127
 *   code = E4M3 nearest value of v * 2^-X, ties to the even code, saturated
 *          to +-448 (v * 2^-X < 512, so values in (448, 512) * 2^X clamp)
 *   value = decode(code) * 2^X
 * Codes are OCP E4M3 as in the fp8 calls; every input is bf16.  Scale arrays
 * hold one byte per block, a row's blocks contiguous.
 * Limits: every blocked size (K, N, ldm) a multiple of 128; code arrays
 * 8-byte aligned, scale arrays 4-byte aligned, bf16 inputs 16-byte aligned. */

/* 1 x 32 blocks along rows: x [M, K] -> q [M, K], scale [M, K/32]. */
int moe_quant_mxfp8_rows(const void* x, int64_t M, int64_t K, uint8_t* q, uint8_t* scale,
                         void* stream);

/* The permutation fused into the row quantizer (section 2, Dispatch): row r
 * of q / scale is the quantization of x[src_token[r]] for r < offsets[G], so
 * the permuted bf16 rows are never written.  x [T, K]; src_token [M] int32
 * (moe_route_topk / moe_apply_capacity); offsets [G+1]; q [M, K] and scale
 * [M, K/32] out, rows at and past offsets[G] not written.  A src_token entry
 * outside [0, T) reads as a zero row. */
int moe_permute_quant_mxfp8(const void* x, int64_t T, int64_t K, const int32_t* src_token,
                            const int64_t* offsets, int32_t G, int64_t M, uint8_t* q,
                            uint8_t* scale, void* stream);

/* The same dispatch driven from the token side (section 2, Dispatch): each
 * token of x [T, K] is read and quantized once, and its codes and scale bytes
 * are written to every row dst_row[t k + j] (dst_row [T, k] int32, the map of
 * moe_route_topk / moe_apply_capacity) that lies in [0, min(M, offsets[G])).
 * A slot whose row is outside that range (a dropped slot, -1) is skipped, and
 * rows named by no slot are not written: on a map where every row below
 * offsets[G] has exactly one slot (dropless, or capacity-limited) the result
 * equals moe_permute_quant_mxfp8's byte for byte, while reading x once
 * instead of k times.  A map with padding rows (moe_pad_to_max) needs
 * moe_permute_quant_mxfp8, which writes them as zero rows.  q [M, K] and
 * scale [M, K/32] out. */
int moe_scatter_quant_mxfp8(const void* x, int64_t T, int64_t K, const int32_t* dst_row,
                            int32_t k, const int64_t* offsets, int32_t G, int64_t M, uint8_t* q,
                            uint8_t* scale, void* stream);

/* Both GEMM operand layouts of w [G, K, N], each blocked along the axis its
 * GEMM contracts:
 *   q_fwd [G, N, K] (transposed) with s_fwd [G, N, K/32]  (blocks along K)
 *   q_dgrad [G, K, N]            with s_dgrad [G, K, N/32] (blocks along N) */
int moe_quant_mxfp8_weights(const void* w, int32_t G, int64_t K, int64_t N, uint8_t* q_fwd,
                            uint8_t* s_fwd, uint8_t* q_dgrad, uint8_t* s_dgrad, void* stream);

/* 32-token x 1 blocks for the weight gradients, which contract over tokens:
 * group g's rows offsets[g].. land at padded rows padded[g]..
 * (moe_padded_offsets with align 128; zero codes past the group's end),
 * written transposed: q_t [K, ldm] (row c holds column c's codes) and
 * scale_t [K, ldm/32].  Row r of the groups is x[r] (src_row NULL, x_rows =
 * M) or x[src_row[r]] (the permutation fused in; entries outside
 * [0, x_rows) read as zero rows).  ldm = moe_padded_rows_bound(M, G, 128) or
 * larger, a multiple of 128; padded blocks past padded[G] are not written. */
int moe_quant_mxfp8_token_tiles(const void* x, int64_t x_rows, const int32_t* src_row,
                                const int64_t* offsets, const int64_t* padded, int32_t G,
                                int64_t M, int64_t K, int64_t ldm, uint8_t* q_t, uint8_t* scale_t,
                                void* stream);

/* MXFP8 grouped GEMMs: the products of the dequantized operands, summed in
 * fp32; outputs and epilogues as in the bf16 calls.
 *   forward: C[rows g] = deq(A)[rows g] . deq(B_g)
 *            A, a_scale from moe_quant_mxfp8_rows / moe_permute_quant_mxfp8
 *            ([M, K], [M, K/32]); B (q_fwd, s_fwd) of moe_quant_mxfp8_weights
 *   dgrad:   dA[rows g] = deq(dC)[rows g] . deq(B_g)^T
 *            dC [M, N] with dc_scale [M, N/32]; B (q_dgrad, s_dgrad)
 *   wgrad:   dB[g] = deq(A)^T . deq(dC) over group g's padded rows; A_t
 *            [K, ldm], dC_t [N, ldm] and their scales from
 *            moe_quant_mxfp8_token_tiles
 * Limits: K % 128 == 0, N % 128 == 0 (forward SWIGLU: N / 2 % 64 == 0),
 * K * N < 2^32 (one expert's weight codes under 4 GiB). */
int moe_grouped_gemm_mxfp8_fwd(const uint8_t* A, const uint8_t* a_scale, const uint8_t* B_fwd,
                               const uint8_t* b_scale_fwd, const int64_t* offsets, int32_t G,
                               int64_t M, int64_t K, int64_t N, int epilogue, void* C, void* H,
                               void* stream);
int moe_grouped_gemm_mxfp8_dgrad(const uint8_t* dC, const uint8_t* dc_scale,
                                 const uint8_t* B_dgrad, const uint8_t* b_scale_dgrad,
                                 const int64_t* offsets, int32_t G, int64_t M, int64_t K, int64_t N,
                                 int epilogue, const void* ab, void* dA, void* stream);
int moe_grouped_gemm_mxfp8_wgrad(const uint8_t* A_t, const uint8_t* a_scale_t,
                                 const uint8_t* dC_t, const uint8_t* dc_scale_t,
                                 const int64_t* padded, int32_t G, int64_t ldm, int64_t K,
                                 int64_t N, int dB_dtype, int accumulate, void* dB, void* stream);

/* ------------------------------- Routing weight applied inside the expert -- */
/* The memory-saving arrangement of the permutation (section 4, Memory): the
 * routing weight of each permuted row scales H before W2,
 *   y'[r] = (w_perm[r] * silu(a[r]) * b[r]) . W2[e],
 * so the combine is an unweighted sum (moe_unpermute_combine with topk_w NULL)
 * and its backward is a plain gather of dout (moe_permute of dout), with no
 * need to keep Y.  The routing-weight gradient is <dH'[r], h[r]> over the ffn
 * axis, dH' = dout[t] . W2[e]^T. */

/* w_perm[dst_row[t, j]] = topk_w[t, j]: the routing weight of every permuted
 * row.  topk_w, dst_row [T, k]; w_perm [T*k] fp32. */
int moe_permute_weights(const float* topk_w, const int32_t* dst_row, int64_t T, int32_t k,
                        float* w_perm, void* stream);

/* Forward GEMM 1 with the SwiGLU epilogue and the routing weight applied:
 * as moe_grouped_gemm_fwd with MOE_EPI_SWIGLU, except
 *   H [M, N/2] = row_scale[row] * silu(a) * b   (AB [M, N] unscaled, or NULL).
 * row_scale [M] fp32 (moe_permute_weights).  bf16 only; K % 64 == 0,
 * (N/2) % 64 == 0. */
int moe_grouped_gemm_gated_fwd(const void* A, const void* B, const int64_t* offsets, int32_t G,
                               int64_t M, int64_t K, int64_t N, int dtype, const float* row_scale,
                               void* AB, void* H, void* stream);

/* Data gradient of GEMM 2 with the SwiGLU backward and the routing weight
 * applied: dH' = dC[rows g] . B[g]^T ([M, K], not stored), then
 *   dAB [M, 2K] = SwiGLU'(row_scale[row] * dH')  (as MOE_EPI_SWIGLU_BWD, from ab)
 *   gate_partials[row, c] = sum over columns 64c .. 64c+63 of dH' * h,
 *     h = silu(a) * b from ab; gate_partials [M, K/64] fp32.
 * bf16 only; N % 64 == 0, K % 128 == 0. */
int moe_grouped_gemm_gated_dgrad(const void* dC, const void* B, const int64_t* offsets, int32_t G,
                                 int64_t M, int64_t K, int64_t N, int dtype, const void* ab,
                                 const float* row_scale, void* dAB, float* gate_partials,
                                 void* stream);

/* Routing-weight gradient from the partials, summed in column order:
 *   d_topk_w[t, j] = sum_{c < P} gate_partials[dst_row[t, j], c].
 * gate_partials [T*k, P] fp32, dst_row [T, k], d_topk_w [T, k] fp32 out. */
int moe_gate_grad(const float* gate_partials, int64_t P, const int32_t* dst_row, int64_t T,
                  int32_t k, float* d_topk_w, void* stream);

/* -------------------------------------------------------------- Combine -- */

/* Unpermute and combine (section 2, Combine: rows return to sequence order,
 * weighted by the routing weights, plus an optional shared expert's output):
 *   out[t] = sum_j topk_w[t, j] * y_perm[dst_row[t, j]] + shared_y[t]
 * fp32 accumulation in slot order, one rounding to `dtype`.
 * y_perm [n_rows, d], shared_y [T, d] or NULL, out [T, d], all `dtype`;
 * topk_w [T, k] fp32, or NULL for an unweighted sum (the routing weights
 * already applied inside the experts, moe_grouped_gemm_gated_fwd). */
int moe_unpermute_combine(const void* y_perm, int dtype, const float* topk_w,
                          const int32_t* dst_row, const void* shared_y, int64_t T, int64_t d,
                          int32_t k, int64_t n_rows, void* out, void* stream);

/* Backward of moe_unpermute_combine:
 *   dy_perm[dst_row[t, j]] = topk_w[t, j] * dout[t]
 *   d_topk_w[t, j]         = < dout[t], y_perm[dst_row[t, j]] >   (fp32)
 * (the shared expert's output gradient is dout itself). */
int moe_unpermute_combine_bwd(const void* dout, const void* y_perm, int dtype, const float* topk_w,
                              const int32_t* dst_row, int64_t T, int64_t d, int32_t k,
                              int64_t n_rows, void* dy_perm, float* d_topk_w, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
