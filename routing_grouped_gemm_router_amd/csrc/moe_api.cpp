// C-ABI entry points of the MoE hot path (declared in include/moe.h):
// host-side validation, then kernel launches on the caller's stream.
// Validation never touches the HIP runtime, so every error path can be
// exercised without a GPU.
#include "moe.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b < lim for non-negative a and b, without forming the product (which
// could overflow for sizes a caller got wrong)
bool prod_below(int64_t a, int64_t b, int64_t lim) {
  return a >= 0 && b >= 0 && (b == 0 || a <= (lim - 1) / b);
}

bool valid_dtype(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

int check_row_vectors(int dtype, int64_t d, const char* what) {
  const int64_t q = dtype == MOE_BF16 ? 8 : 4;
  REQUIRE(d % q == 0, MOE_ERR_UNSUPPORTED, "%s: row length %lld must be a multiple of %lld", what,
          static_cast<long long>(d), static_cast<long long>(q));
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "invalid shape";
    case MOE_ERR_DTYPE: return "invalid dtype";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

int moe_abi_version(void) { return 2; }

int moe_router_logits(const void* x, int x_dtype, const float* w_r, const float* logit_bias,
                      int64_t T, int64_t d, int32_t E, float* logits, void* stream) {
  REQUIRE(valid_dtype(x_dtype), MOE_ERR_DTYPE, "moe_router_logits: bad x dtype %d", x_dtype);
  REQUIRE(T >= 0 && d >= 1, MOE_ERR_SHAPE, "moe_router_logits: T=%lld d=%lld",
          static_cast<long long>(T), static_cast<long long>(d));
  REQUIRE(E >= 1 && E <= 1024, MOE_ERR_UNSUPPORTED, "moe_router_logits: E=%d outside [1, 1024]", E);
  if (T == 0) return ok();
  REQUIRE(x && w_r && logits, MOE_ERR_NULL, "moe_router_logits: x, w_r and logits are required");
  return hip_status(moe::launch_router_fwd(x, x_dtype, w_r, logit_bias, T, d, E, logits,
                                           as_stream(stream)),
                    "moe_router_logits");
}

int moe_router_logits_bwd(const void* x, int x_dtype, const float* w_r, const float* d_logits,
                          int64_t T, int64_t d, int32_t E, float* d_w_r, float* dx_router,
                          void* stream) {
  REQUIRE(valid_dtype(x_dtype), MOE_ERR_DTYPE, "moe_router_logits_bwd: bad x dtype %d", x_dtype);
  REQUIRE(T >= 0 && d >= 1, MOE_ERR_SHAPE, "moe_router_logits_bwd: T=%lld d=%lld",
          static_cast<long long>(T), static_cast<long long>(d));
  REQUIRE(E >= 1 && E <= 1024, MOE_ERR_UNSUPPORTED, "moe_router_logits_bwd: E=%d outside [1, 1024]",
          E);
  if (!d_w_r && !dx_router) return ok();
  REQUIRE(T == 0 || d_logits, MOE_ERR_NULL, "moe_router_logits_bwd: d_logits is required");
  REQUIRE(!d_w_r || T == 0 || x, MOE_ERR_NULL, "moe_router_logits_bwd: x is required for d_w_r");
  REQUIRE(!dx_router || T == 0 || w_r, MOE_ERR_NULL,
          "moe_router_logits_bwd: w_r is required for dx_router");
  return hip_status(moe::launch_router_bwd(x, x_dtype, w_r, d_logits, T, d, E, d_w_r, dx_router,
                                           as_stream(stream)),
                    "moe_router_logits_bwd");
}

int moe_router_logits_bwd_topk(const void* x, int x_dtype, const float* w_r, const float* d_logits,
                               const int32_t* topk_idx, const int64_t* offsets,
                               const int32_t* src_token, int64_t T, int64_t d, int32_t E,
                               int32_t k, float* d_w_r, float* dx_router, void* stream) {
  const char* fn = "moe_router_logits_bwd_topk";
  REQUIRE(valid_dtype(x_dtype), MOE_ERR_DTYPE, "%s: bad x dtype %d", fn, x_dtype);
  REQUIRE(T >= 0 && d >= 1 && E >= 1 && k >= 1 && k <= E, MOE_ERR_SHAPE,
          "%s: T=%lld d=%lld E=%d k=%d", fn, static_cast<long long>(T), static_cast<long long>(d), E,
          k);
  REQUIRE(E <= 256, MOE_ERR_UNSUPPORTED, "%s: E=%d above 256 (use moe_router_logits_bwd)", fn, E);
  REQUIRE(k <= 64, MOE_ERR_UNSUPPORTED, "%s: k=%d above 64 (use moe_router_logits_bwd)", fn, k);
  REQUIRE(prod_below(T, k, int64_t(1) << 31) && d < (int64_t(1) << 40), MOE_ERR_UNSUPPORTED,
          "%s: T*k must be below 2^31", fn);
  REQUIRE(d % 8 == 0, MOE_ERR_UNSUPPORTED, "%s: d=%lld must be a multiple of 8", fn,
          static_cast<long long>(d));
  if (!d_w_r && !dx_router) return ok();
  REQUIRE(T == 0 || (d_logits && topk_idx), MOE_ERR_NULL, "%s: d_logits and topk_idx are required",
          fn);
  REQUIRE(!d_w_r || T == 0 || (x && offsets && src_token), MOE_ERR_NULL,
          "%s: x, offsets and src_token are required for d_w_r", fn);
  REQUIRE(!dx_router || T == 0 || w_r, MOE_ERR_NULL, "%s: w_r is required for dx_router", fn);
  REQUIRE(!d_w_r || T == 0 || aligned16(x), MOE_ERR_UNSUPPORTED, "%s: x must be 16-byte aligned",
          fn);
  return hip_status(moe::launch_router_bwd_topk(x, x_dtype, w_r, d_logits, topk_idx, offsets,
                                                src_token, T, d, E, k, d_w_r, dx_router,
                                                as_stream(stream)),
                    fn);
}

size_t moe_route_topk_workspace_bytes(int64_t T, int32_t E, int32_t k) {
  (void)k;
  if (T < 0 || E < 1) return 0;
  return moe::route_topk_workspace(T, E);
}

static int check_route_shape(const char* fn, int64_t T, int32_t E, int32_t k, int score) {
  REQUIRE(T >= 0, MOE_ERR_SHAPE, "%s: T=%lld", fn, static_cast<long long>(T));
  REQUIRE(E >= 1 && E <= 1024, MOE_ERR_UNSUPPORTED, "%s: E=%d outside [1, 1024]", fn, E);
  REQUIRE(k >= 1 && k <= E, MOE_ERR_SHAPE, "%s: k=%d outside [1, E=%d]", fn, k, E);
  REQUIRE(k <= 64, MOE_ERR_UNSUPPORTED, "%s: k=%d above 64", fn, k);
  REQUIRE(prod_below(T, k, int64_t(1) << 31), MOE_ERR_UNSUPPORTED, "%s: T*k must be below 2^31", fn);
  REQUIRE(score == MOE_SOFTMAX || score == MOE_SIGMOID, MOE_ERR_SHAPE, "%s: bad score %d", fn,
          score);
  return MOE_OK;
}

int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int score, int renorm,
                   int32_t* topk_idx, float* topk_w, int32_t* counts, int64_t* offsets,
                   int32_t* dst_row, int32_t* src_token, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int st = check_route_shape("moe_route_topk", T, E, k, score);
  if (st != MOE_OK) return st;
  REQUIRE(counts && offsets, MOE_ERR_NULL, "moe_route_topk: counts and offsets are required");
  REQUIRE(T == 0 || (logits && topk_idx && topk_w && dst_row && src_token), MOE_ERR_NULL,
          "moe_route_topk: logits, topk_idx, topk_w, dst_row and src_token are required");
  const size_t need = moe::route_topk_workspace(T, E);
  REQUIRE(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "moe_route_topk: workspace needs %zu bytes, got %zu", need, workspace_bytes);
  REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 7u) == 0, MOE_ERR_UNSUPPORTED,
          "moe_route_topk: workspace must be 8-byte aligned");
  return hip_status(moe::launch_route_topk(logits, T, E, k, score, renorm != 0, nullptr, topk_idx,
                                           topk_w, counts, offsets, dst_row, src_token, workspace,
                                           as_stream(stream)),
                    "moe_route_topk");
}

int moe_route_topk_expert_bias(const float* logits, const float* sel_bias, int64_t T, int32_t E,
                               int32_t k, int renorm, int32_t* topk_idx, float* topk_w,
                               int32_t* counts, int64_t* offsets, int32_t* dst_row,
                               int32_t* src_token, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const char* fn = "moe_route_topk_expert_bias";
  int st = check_route_shape(fn, T, E, k, MOE_SIGMOID);
  if (st != MOE_OK) return st;
  REQUIRE(counts && offsets, MOE_ERR_NULL, "%s: counts and offsets are required", fn);
  REQUIRE(T == 0 || (logits && sel_bias && topk_idx && topk_w && dst_row && src_token),
          MOE_ERR_NULL, "%s: logits, sel_bias, topk_idx, topk_w, dst_row and src_token are required",
          fn);
  const size_t need = moe::route_topk_workspace(T, E);
  REQUIRE(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "%s: workspace needs %zu bytes, got %zu", fn, need, workspace_bytes);
  REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 7u) == 0, MOE_ERR_UNSUPPORTED,
          "%s: workspace must be 8-byte aligned", fn);
  return hip_status(moe::launch_route_topk(logits, T, E, k, MOE_SIGMOID, renorm != 0, sel_bias,
                                           topk_idx, topk_w, counts, offsets, dst_row, src_token,
                                           workspace, as_stream(stream)),
                    fn);
}

int moe_pad_to_max(const int32_t* topk_idx, const int32_t* counts, const int64_t* offsets,
                   const int32_t* dst_row, const int32_t* src_token, int64_t T, int32_t E,
                   int32_t k, int64_t capacity, int32_t* counts_out, int64_t* offsets_out,
                   int32_t* dst_row_out, int32_t* src_token_out, void* stream) {
  const char* fn = "moe_pad_to_max";
  REQUIRE(T >= 0 && E >= 1 && k >= 1 && k <= E && capacity >= 1, MOE_ERR_SHAPE,
          "%s: T=%lld E=%d k=%d capacity=%lld", fn, static_cast<long long>(T), E, k,
          static_cast<long long>(capacity));
  REQUIRE(E <= 1024, MOE_ERR_UNSUPPORTED, "%s: E=%d above 1024", fn, E);
  REQUIRE(prod_below(E, capacity, int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
          "%s: E * capacity must be below 2^31", fn);
  REQUIRE(counts && offsets && counts_out && offsets_out && src_token_out, MOE_ERR_NULL,
          "%s: counts, offsets and the outputs are required", fn);
  REQUIRE(T == 0 || (topk_idx && dst_row && src_token && dst_row_out), MOE_ERR_NULL,
          "%s: topk_idx, dst_row, src_token and dst_row_out are required", fn);
  return hip_status(moe::launch_pad_to_max(topk_idx, counts, offsets, dst_row, src_token, T, E, k,
                                           capacity, counts_out, offsets_out, dst_row_out,
                                           src_token_out, as_stream(stream)),
                    fn);
}

int moe_zero_unmapped_rows(void* buf, int dtype, const int32_t* src_token, int64_t M, int64_t d,
                           void* stream) {
  const char* fn = "moe_zero_unmapped_rows";
  REQUIRE(M >= 0 && d >= 1, MOE_ERR_SHAPE, "%s: M=%lld d=%lld", fn, static_cast<long long>(M),
          static_cast<long long>(d));
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, MOE_ERR_DTYPE, "%s: dtype %d", fn, dtype);
  REQUIRE(d < (int64_t(1) << 40), MOE_ERR_UNSUPPORTED, "%s: row length %lld", fn,
          static_cast<long long>(d));
  const int64_t row_bytes = d * (dtype == MOE_F32 ? 4 : 2);
  REQUIRE(row_bytes % 16 == 0, MOE_ERR_UNSUPPORTED, "%s: rows must be multiples of 16 bytes", fn);
  if (M == 0) return ok();
  REQUIRE(buf && src_token, MOE_ERR_NULL, "%s: buf and src_token are required", fn);
  REQUIRE(aligned16(buf), MOE_ERR_UNSUPPORTED, "%s: buf must be 16-byte aligned", fn);
  return hip_status(moe::launch_zero_unmapped_rows(buf, row_bytes, src_token, M, as_stream(stream)),
                    fn);
}

int moe_expert_bias_update(const int32_t* counts, int32_t E, float rate, float* sel_bias,
                           void* stream) {
  const char* fn = "moe_expert_bias_update";
  REQUIRE(E >= 1, MOE_ERR_SHAPE, "%s: E=%d", fn, E);
  REQUIRE(E <= 1024, MOE_ERR_UNSUPPORTED, "%s: E=%d above 1024", fn, E);
  REQUIRE(counts && sel_bias, MOE_ERR_NULL, "%s: counts and sel_bias are required", fn);
  return hip_status(moe::launch_expert_bias_update(counts, E, rate, sel_bias, as_stream(stream)),
                    fn);
}

int moe_route_topk_noalloc(const float* logits, int64_t T, int32_t E, int32_t k, int score,
                           int renorm, int32_t* topk_idx, float* topk_w, int32_t* counts,
                           int64_t* offsets, int32_t* dst_row, int32_t* src_token, void* stream) {
  const char* fn = "moe_route_topk_noalloc";
  int st = check_route_shape(fn, T, E, k, score);
  if (st != MOE_OK) return st;
  REQUIRE(counts && offsets, MOE_ERR_NULL, "%s: counts and offsets are required", fn);
  REQUIRE(T == 0 || (logits && topk_idx && topk_w && dst_row && src_token), MOE_ERR_NULL,
          "%s: logits, topk_idx, topk_w, dst_row and src_token are required", fn);
  const size_t need = moe::route_topk_workspace(T, E);
  REQUIRE(need <= moe::route_noalloc_scratch_bytes(), MOE_ERR_UNSUPPORTED,
          "%s: needs %zu bytes of scratch, above the fixed %zu (ceil(T/64) * E * 12 + 256)", fn,
          need, moe::route_noalloc_scratch_bytes());
  void* scratch = nullptr;
  hipError_t e = moe::route_scratch_ptr(&scratch);
  if (e != hipSuccess) return hip_status(e, fn);
  return hip_status(moe::launch_route_topk(logits, T, E, k, score, renorm != 0, nullptr, topk_idx,
                                           topk_w, counts, offsets, dst_row, src_token, scratch,
                                           as_stream(stream)),
                    fn);
}

int moe_check_finite(const float* x, int64_t n, int32_t* status, void* stream) {
  const char* fn = "moe_check_finite";
  REQUIRE(n >= 0, MOE_ERR_SHAPE, "%s: n=%lld", fn, static_cast<long long>(n));
  if (n == 0) return ok();
  REQUIRE(x && status, MOE_ERR_NULL, "%s: x and status are required", fn);
  REQUIRE(aligned16(x), MOE_ERR_UNSUPPORTED, "%s: x must be 16-byte aligned", fn);
  return hip_status(moe::launch_check_finite(x, n, status, as_stream(stream)), fn);
}

int moe_check_dispatch(const int32_t* topk_idx, const int32_t* counts, const int64_t* offsets,
                       const int32_t* dst_row, const int32_t* src_token, int64_t T, int32_t E,
                       int32_t k, int64_t n_rows, int32_t* status, void* stream) {
  const char* fn = "moe_check_dispatch";
  REQUIRE(T >= 0 && E >= 1 && k >= 1 && n_rows >= 0, MOE_ERR_SHAPE, "%s: T=%lld E=%d k=%d", fn,
          static_cast<long long>(T), E, k);
  REQUIRE(E <= 1024 && prod_below(T, k, int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
          "%s: E=%d, T*k must be below 2^31", fn, E);
  REQUIRE(counts && offsets && status, MOE_ERR_NULL, "%s: counts, offsets and status are required",
          fn);
  REQUIRE(T == 0 || (topk_idx && dst_row && (n_rows == 0 || src_token)), MOE_ERR_NULL,
          "%s: topk_idx, dst_row and src_token are required", fn);
  return hip_status(moe::launch_check_dispatch(topk_idx, counts, offsets, dst_row, src_token, T, E,
                                               k, n_rows, status, as_stream(stream)),
                    fn);
}

int moe_route_replay(const float* logits, const int32_t* topk_idx_in, int64_t T, int32_t E,
                     int32_t k, int score, int renorm, int32_t* topk_idx, float* topk_w,
                     int32_t* counts, int64_t* offsets, int32_t* dst_row, int32_t* src_token,
                     int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_route_shape("moe_route_replay", T, E, k, score);
  if (st != MOE_OK) return st;
  REQUIRE(counts && offsets, MOE_ERR_NULL, "moe_route_replay: counts and offsets are required");
  REQUIRE(T == 0 || (logits && topk_idx_in && topk_idx && topk_w && dst_row && src_token),
          MOE_ERR_NULL,
          "moe_route_replay: logits, topk_idx_in, topk_idx, topk_w, dst_row and src_token are "
          "required");
  const size_t need = moe::route_topk_workspace(T, E);
  REQUIRE(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "moe_route_replay: workspace needs %zu bytes, got %zu", need, workspace_bytes);
  REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 7u) == 0, MOE_ERR_UNSUPPORTED,
          "moe_route_replay: workspace must be 8-byte aligned");
  return hip_status(moe::launch_route_replay(logits, topk_idx_in, T, E, k, score, renorm != 0,
                                             topk_idx, topk_w, counts, offsets, dst_row,
                                             src_token, status, workspace, as_stream(stream)),
                    "moe_route_replay");
}

int moe_apply_capacity(const int32_t* topk_idx, const int32_t* counts, const int64_t* offsets,
                       const int32_t* dst_row, int64_t T, int32_t E, int32_t k, int64_t capacity,
                       int32_t* counts_out, int64_t* offsets_out, int32_t* dst_row_out,
                       int32_t* src_token_out, void* stream) {
  const char* fn = "moe_apply_capacity";
  REQUIRE(T >= 0 && E >= 1 && k >= 1 && k <= E && prod_below(T, k, int64_t(1) << 31), MOE_ERR_SHAPE,
          "%s: T=%lld E=%d k=%d", fn, static_cast<long long>(T), E, k);
  REQUIRE(E <= 1024, MOE_ERR_UNSUPPORTED, "%s: E=%d above 1024", fn, E);
  REQUIRE(capacity >= 0, MOE_ERR_SHAPE, "%s: capacity=%lld", fn, static_cast<long long>(capacity));
  REQUIRE(counts && offsets && counts_out && offsets_out, MOE_ERR_NULL,
          "%s: counts and offsets (in and out) are required", fn);
  REQUIRE(T == 0 || (topk_idx && dst_row && dst_row_out && src_token_out), MOE_ERR_NULL,
          "%s: topk_idx, dst_row, dst_row_out and src_token_out are required", fn);
  REQUIRE(dst_row_out != dst_row && offsets_out != offsets, MOE_ERR_SHAPE,
          "%s: outputs must not alias the inputs", fn);
  return hip_status(moe::launch_apply_capacity(topk_idx, counts, offsets, dst_row, T, E, k,
                                               capacity, counts_out, offsets_out, dst_row_out,
                                               src_token_out, as_stream(stream)),
                    fn);
}

size_t moe_aux_loss_workspace_bytes(int64_t T, int32_t E) {
  if (T < 0 || E < 1) return 0;
  return moe::aux_loss_workspace(T, E);
}

int moe_aux_loss(const float* logits, const int32_t* counts, int64_t T, int32_t E, int32_t k,
                 int score, float coeff, float* loss, float* d_logits, void* workspace,
                 size_t workspace_bytes, void* stream) {
  const char* fn = "moe_aux_loss";
  int st = check_route_shape(fn, T, E, k, score);
  if (st != MOE_OK) return st;
  REQUIRE(T >= 1, MOE_ERR_SHAPE, "%s: T must be at least 1", fn);
  REQUIRE(logits && counts && (loss || d_logits), MOE_ERR_NULL,
          "%s: logits, counts and at least one of loss / d_logits are required", fn);
  const size_t need = moe::aux_loss_workspace(T, E);
  REQUIRE(!loss || (workspace && workspace_bytes >= need), MOE_ERR_WORKSPACE,
          "%s: workspace needs %zu bytes, got %zu", fn, need, workspace_bytes);
  REQUIRE(!loss || (reinterpret_cast<uintptr_t>(workspace) & 3u) == 0, MOE_ERR_UNSUPPORTED,
          "%s: workspace must be 4-byte aligned", fn);
  return hip_status(moe::launch_aux_loss(logits, counts, T, E, k, score, coeff, loss, d_logits,
                                         workspace, as_stream(stream)),
                    fn);
}

int moe_route_topk_bwd(const float* logits, const int32_t* topk_idx, const float* topk_w,
                       const float* d_topk_w, int64_t T, int32_t E, int32_t k, int score,
                       int renorm, float* d_logits, void* stream) {
  int st = check_route_shape("moe_route_topk_bwd", T, E, k, score);
  if (st != MOE_OK) return st;
  if (T == 0) return ok();
  REQUIRE(logits && topk_idx && topk_w && d_topk_w && d_logits, MOE_ERR_NULL,
          "moe_route_topk_bwd: all pointers are required");
  return hip_status(moe::launch_route_topk_bwd(logits, topk_idx, topk_w, d_topk_w, T, E, k, score,
                                               renorm != 0, d_logits, as_stream(stream)),
                    "moe_route_topk_bwd");
}

int moe_permute(const void* x, int dtype, const int32_t* dst_row, int64_t T, int64_t d, int32_t k,
                int64_t n_rows, void* x_perm, void* stream) {
  REQUIRE(valid_dtype(dtype), MOE_ERR_DTYPE, "moe_permute: bad dtype %d", dtype);
  REQUIRE(T >= 0 && d >= 1 && k >= 1 && n_rows >= 0, MOE_ERR_SHAPE,
          "moe_permute: T=%lld d=%lld k=%d n_rows=%lld", static_cast<long long>(T),
          static_cast<long long>(d), k, static_cast<long long>(n_rows));
  int st = check_row_vectors(dtype, d, "moe_permute");
  if (st != MOE_OK) return st;
  if (T == 0) return ok();
  REQUIRE(x && dst_row && x_perm, MOE_ERR_NULL, "moe_permute: x, dst_row and x_perm are required");
  REQUIRE(aligned16(x) && aligned16(x_perm), MOE_ERR_UNSUPPORTED,
          "moe_permute: x and x_perm must be 16-byte aligned");
  return hip_status(
      moe::launch_permute(x, dtype, dst_row, T, d, k, n_rows, x_perm, as_stream(stream)),
      "moe_permute");
}

int moe_permute_bwd(const void* dx_perm, int dtype, const int32_t* dst_row, int64_t T, int64_t d,
                    int32_t k, int64_t n_rows, const void* addend, const float* addend_f32,
                    void* dx, void* stream) {
  REQUIRE(valid_dtype(dtype), MOE_ERR_DTYPE, "moe_permute_bwd: bad dtype %d", dtype);
  REQUIRE(T >= 0 && d >= 1 && k >= 1 && n_rows >= 0, MOE_ERR_SHAPE,
          "moe_permute_bwd: T=%lld d=%lld k=%d n_rows=%lld", static_cast<long long>(T),
          static_cast<long long>(d), k, static_cast<long long>(n_rows));
  int st = check_row_vectors(dtype, d, "moe_permute_bwd");
  if (st != MOE_OK) return st;
  if (T == 0) return ok();
  REQUIRE(dx_perm && dst_row && dx, MOE_ERR_NULL,
          "moe_permute_bwd: dx_perm, dst_row and dx are required");
  REQUIRE(aligned16(dx_perm) && aligned16(dx) && aligned16(addend) && aligned16(addend_f32),
          MOE_ERR_UNSUPPORTED, "moe_permute_bwd: tensors must be 16-byte aligned");
  return hip_status(moe::launch_permute_bwd(dx_perm, dtype, dst_row, T, d, k, n_rows, addend,
                                            addend_f32, dx, as_stream(stream)),
                    "moe_permute_bwd");
}

// a * b < lim for non-negative a, b, without forming the product
static int check_gemm(const char* fn, const void* p0, const void* p1, const int64_t* off, int32_t G,
                      int64_t M, int64_t K, int64_t N, int dtype) {
  REQUIRE(valid_dtype(dtype), MOE_ERR_DTYPE, "%s: bad dtype %d", fn, dtype);
  REQUIRE(G >= 1 && M >= 0 && K >= 1 && N >= 1, MOE_ERR_SHAPE, "%s: G=%d M=%lld K=%lld N=%lld", fn,
          G, static_cast<long long>(M), static_cast<long long>(K), static_cast<long long>(N));
  REQUIRE(G <= 1024, MOE_ERR_UNSUPPORTED, "%s: G=%d above 1024", fn, G);
  REQUIRE(M / 64 + G < (int64_t(1) << 31) / 64, MOE_ERR_UNSUPPORTED, "%s: M too large", fn);
  // the bf16 kernels address one expert's weights with 32-bit byte offsets
  REQUIRE(dtype != MOE_BF16 || prod_below(K, N, int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
          "%s: K*N must be below 2^31 (one expert's bf16 weights under 4 GiB)", fn);
  if (M == 0) return MOE_OK;  // nothing to read or write
  REQUIRE(p0 && p1 && off, MOE_ERR_NULL, "%s: operands and offsets are required", fn);
  REQUIRE(aligned16(p0) && aligned16(p1), MOE_ERR_UNSUPPORTED, "%s: operands must be 16-byte aligned",
          fn);
  return MOE_OK;
}

int moe_grouped_gemm_fwd(const void* A, const void* B, const int64_t* offsets, int32_t G, int64_t M,
                         int64_t K, int64_t N, int dtype, int epilogue, void* C, void* H,
                         void* stream) {
  const char* fn = "moe_grouped_gemm_fwd";
  int st = check_gemm(fn, A, B, offsets, G, M, K, N, dtype);
  if (st != MOE_OK) return st;
  REQUIRE(epilogue == MOE_EPI_NONE || epilogue == MOE_EPI_SWIGLU, MOE_ERR_SHAPE,
          "%s: epilogue %d not available in the forward", fn, epilogue);
  if (epilogue == MOE_EPI_SWIGLU) {
    REQUIRE(N % 2 == 0, MOE_ERR_SHAPE, "%s: SWIGLU needs an even N", fn);
    REQUIRE(M == 0 || H, MOE_ERR_NULL, "%s: SWIGLU needs H", fn);
  } else {
    REQUIRE(M == 0 || C, MOE_ERR_NULL, "%s: C is required", fn);
  }
  if (dtype == MOE_BF16) {
    REQUIRE(K % 64 == 0, MOE_ERR_UNSUPPORTED, "%s: bf16 needs K %% 64 == 0 (K=%lld)", fn,
            static_cast<long long>(K));
    REQUIRE(epilogue == MOE_EPI_SWIGLU ? (N / 2) % 64 == 0 : N % 128 == 0, MOE_ERR_UNSUPPORTED,
            "%s: bf16 needs N %% 128 == 0 (SWIGLU: f %% 64 == 0), N=%lld", fn,
            static_cast<long long>(N));
  }
  if (M == 0) return ok();
  hipError_t e = dtype == MOE_BF16
                     ? moe::launch_gg_bf16_fwd(A, B, offsets, G, M, K, N, epilogue, C, H,
                                               as_stream(stream))
                     : moe::launch_gg_f32_fwd(static_cast<const float*>(A),
                                              static_cast<const float*>(B), offsets, G, M, K, N,
                                              epilogue, static_cast<float*>(C),
                                              static_cast<float*>(H), as_stream(stream));
  return hip_status(e, fn);
}

int moe_grouped_gemm_dgrad(const void* dC, const void* B, const int64_t* offsets, int32_t G,
                           int64_t M, int64_t K, int64_t N, int dtype, int epilogue,
                           const void* ab, void* dA, void* stream) {
  const char* fn = "moe_grouped_gemm_dgrad";
  int st = check_gemm(fn, dC, B, offsets, G, M, K, N, dtype);
  if (st != MOE_OK) return st;
  REQUIRE(epilogue == MOE_EPI_NONE || epilogue == MOE_EPI_SWIGLU_BWD, MOE_ERR_SHAPE,
          "%s: epilogue %d not available in dgrad", fn, epilogue);
  REQUIRE(M == 0 || dA, MOE_ERR_NULL, "%s: dA is required", fn);
  REQUIRE(M == 0 || epilogue != MOE_EPI_SWIGLU_BWD || ab, MOE_ERR_NULL,
          "%s: SWIGLU_BWD needs ab", fn);
  if (dtype == MOE_BF16) {
    REQUIRE(N % 64 == 0 && K % 128 == 0, MOE_ERR_UNSUPPORTED,
            "%s: bf16 needs N %% 64 == 0 and K %% 128 == 0 (K=%lld N=%lld)", fn,
            static_cast<long long>(K), static_cast<long long>(N));
  }
  if (M == 0) return ok();
  hipError_t e = dtype == MOE_BF16
                     ? moe::launch_gg_bf16_dgrad(dC, B, offsets, G, M, K, N, epilogue, ab, dA,
                                                 as_stream(stream))
                     : moe::launch_gg_f32_dgrad(static_cast<const float*>(dC),
                                                static_cast<const float*>(B), offsets, G, M, K, N,
                                                epilogue, static_cast<const float*>(ab),
                                                static_cast<float*>(dA), as_stream(stream));
  return hip_status(e, fn);
}

int moe_grouped_gemm_wgrad(const void* A, const void* dC, const int64_t* offsets, int32_t G,
                           int64_t M, int64_t K, int64_t N, int dtype, int dB_dtype,
                           int accumulate, void* dB, void* stream) {
  const char* fn = "moe_grouped_gemm_wgrad";
  REQUIRE(G >= 1 && M >= 0 && K >= 1 && N >= 1, MOE_ERR_SHAPE, "%s: G=%d M=%lld K=%lld N=%lld", fn,
          G, static_cast<long long>(M), static_cast<long long>(K), static_cast<long long>(N));
  REQUIRE(valid_dtype(dtype), MOE_ERR_DTYPE, "%s: bad dtype %d", fn, dtype);
  REQUIRE(dB_dtype == dtype || dB_dtype == MOE_F32, MOE_ERR_DTYPE,
          "%s: dB dtype must be the input dtype or fp32", fn);
  REQUIRE(G <= 1024, MOE_ERR_UNSUPPORTED, "%s: G=%d above 1024", fn, G);
  REQUIRE(offsets && dB, MOE_ERR_NULL, "%s: offsets and dB are required", fn);
  REQUIRE(M == 0 || (A && dC), MOE_ERR_NULL, "%s: A and dC are required", fn);
  if (dtype == MOE_BF16) {
    REQUIRE(K % 128 == 0 && N % 128 == 0, MOE_ERR_UNSUPPORTED,
            "%s: bf16 needs K %% 128 == 0 and N %% 128 == 0 (K=%lld N=%lld)", fn,
            static_cast<long long>(K), static_cast<long long>(N));
    // a group's rows of A and dC are addressed with 32-bit byte offsets
    REQUIRE(prod_below(M, K, int64_t(1) << 31) && prod_below(M, N, int64_t(1) << 31),
            MOE_ERR_UNSUPPORTED, "%s: M*K and M*N must be below 2^31 for bf16", fn);
    REQUIRE(aligned16(A) && aligned16(dC), MOE_ERR_UNSUPPORTED, "%s: operands must be 16-byte aligned",
            fn);
  }
  hipError_t e = dtype == MOE_BF16
                     ? moe::launch_gg_bf16_wgrad(A, dC, offsets, G, M, K, N, dB_dtype == MOE_F32,
                                                 accumulate != 0, dB, as_stream(stream))
                     : moe::launch_gg_f32_wgrad(static_cast<const float*>(A),
                                                static_cast<const float*>(dC), offsets, G, M, K, N,
                                                accumulate != 0, static_cast<float*>(dB),
                                                as_stream(stream));
  return hip_status(e, fn);
}

int moe_swiglu(const void* ab, int dtype, int64_t M, int64_t f, void* h, void* stream) {
  REQUIRE(valid_dtype(dtype), MOE_ERR_DTYPE, "moe_swiglu: bad dtype %d", dtype);
  REQUIRE(M >= 0 && f >= 1, MOE_ERR_SHAPE, "moe_swiglu: M=%lld f=%lld", static_cast<long long>(M),
          static_cast<long long>(f));
  int st = check_row_vectors(dtype, f, "moe_swiglu");
  if (st != MOE_OK) return st;
  if (M == 0) return ok();
  REQUIRE(ab && h, MOE_ERR_NULL, "moe_swiglu: ab and h are required");
  REQUIRE(aligned16(ab) && aligned16(h), MOE_ERR_UNSUPPORTED, "moe_swiglu: 16-byte alignment needed");
  return hip_status(moe::launch_swiglu(ab, dtype, M, f, h, as_stream(stream)), "moe_swiglu");
}

int moe_swiglu_bwd(const void* dh, const void* ab, int dtype, int64_t M, int64_t f, void* dab,
                   void* stream) {
  REQUIRE(valid_dtype(dtype), MOE_ERR_DTYPE, "moe_swiglu_bwd: bad dtype %d", dtype);
  REQUIRE(M >= 0 && f >= 1, MOE_ERR_SHAPE, "moe_swiglu_bwd: M=%lld f=%lld",
          static_cast<long long>(M), static_cast<long long>(f));
  int st = check_row_vectors(dtype, f, "moe_swiglu_bwd");
  if (st != MOE_OK) return st;
  if (M == 0) return ok();
  REQUIRE(dh && ab && dab, MOE_ERR_NULL, "moe_swiglu_bwd: dh, ab and dab are required");
  REQUIRE(aligned16(dh) && aligned16(ab) && aligned16(dab), MOE_ERR_UNSUPPORTED,
          "moe_swiglu_bwd: 16-byte alignment needed");
  return hip_status(moe::launch_swiglu_bwd(dh, ab, dtype, M, f, dab, as_stream(stream)),
                    "moe_swiglu_bwd");
}

int moe_unpermute_combine(const void* y_perm, int dtype, const float* topk_w,
                          const int32_t* dst_row, const void* shared_y, int64_t T, int64_t d,
                          int32_t k, int64_t n_rows, void* out, void* stream) {
  REQUIRE(valid_dtype(dtype), MOE_ERR_DTYPE, "moe_unpermute_combine: bad dtype %d", dtype);
  REQUIRE(T >= 0 && d >= 1 && k >= 1 && n_rows >= 0, MOE_ERR_SHAPE,
          "moe_unpermute_combine: T=%lld d=%lld k=%d n_rows=%lld", static_cast<long long>(T),
          static_cast<long long>(d), k, static_cast<long long>(n_rows));
  int st = check_row_vectors(dtype, d, "moe_unpermute_combine");
  if (st != MOE_OK) return st;
  if (T == 0) return ok();
  REQUIRE(y_perm && dst_row && out, MOE_ERR_NULL,
          "moe_unpermute_combine: y_perm, dst_row and out are required");
  REQUIRE(aligned16(y_perm) && aligned16(out) && aligned16(shared_y), MOE_ERR_UNSUPPORTED,
          "moe_unpermute_combine: 16-byte alignment needed");
  return hip_status(moe::launch_combine(y_perm, dtype, topk_w, dst_row, shared_y, T, d, k, n_rows,
                                        out, as_stream(stream)),
                    "moe_unpermute_combine");
}

int moe_permute_weights(const float* topk_w, const int32_t* dst_row, int64_t T, int32_t k,
                        float* w_perm, void* stream) {
  REQUIRE(T >= 0 && k >= 1 && prod_below(T, k, int64_t(1) << 31), MOE_ERR_SHAPE,
          "moe_permute_weights: T=%lld k=%d", static_cast<long long>(T), k);
  if (T == 0) return ok();
  REQUIRE(topk_w && dst_row && w_perm, MOE_ERR_NULL, "moe_permute_weights: all pointers are required");
  return hip_status(moe::launch_permute_weights(topk_w, dst_row, T, k, w_perm, as_stream(stream)),
                    "moe_permute_weights");
}

int moe_gate_grad(const float* gate_partials, int64_t P, const int32_t* dst_row, int64_t T,
                  int32_t k, float* d_topk_w, void* stream) {
  REQUIRE(T >= 0 && k >= 1 && P >= 1 && prod_below(T, k, int64_t(1) << 31), MOE_ERR_SHAPE,
          "moe_gate_grad: T=%lld k=%d P=%lld", static_cast<long long>(T), k,
          static_cast<long long>(P));
  if (T == 0) return ok();
  REQUIRE(gate_partials && dst_row && d_topk_w, MOE_ERR_NULL,
          "moe_gate_grad: all pointers are required");
  return hip_status(moe::launch_gate_grad(gate_partials, P, dst_row, T, k, d_topk_w,
                                          as_stream(stream)),
                    "moe_gate_grad");
}

int moe_unpermute_combine_bwd(const void* dout, const void* y_perm, int dtype, const float* topk_w,
                              const int32_t* dst_row, int64_t T, int64_t d, int32_t k,
                              int64_t n_rows, void* dy_perm, float* d_topk_w, void* stream) {
  REQUIRE(valid_dtype(dtype), MOE_ERR_DTYPE, "moe_unpermute_combine_bwd: bad dtype %d", dtype);
  REQUIRE(T >= 0 && d >= 1 && k >= 1 && n_rows >= 0, MOE_ERR_SHAPE,
          "moe_unpermute_combine_bwd: T=%lld d=%lld k=%d n_rows=%lld", static_cast<long long>(T),
          static_cast<long long>(d), k, static_cast<long long>(n_rows));
  REQUIRE(k <= 64, MOE_ERR_UNSUPPORTED, "moe_unpermute_combine_bwd: k=%d above 64", k);
  REQUIRE(prod_below(T, k, int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
          "moe_unpermute_combine_bwd: T*k must be below 2^31");
  int st = check_row_vectors(dtype, d, "moe_unpermute_combine_bwd");
  if (st != MOE_OK) return st;
  if (T == 0) return ok();
  REQUIRE(dout && y_perm && topk_w && dst_row && dy_perm && d_topk_w, MOE_ERR_NULL,
          "moe_unpermute_combine_bwd: all pointers are required");
  REQUIRE(aligned16(dout) && aligned16(y_perm) && aligned16(dy_perm), MOE_ERR_UNSUPPORTED,
          "moe_unpermute_combine_bwd: 16-byte alignment needed");
  return hip_status(moe::launch_combine_bwd(dout, y_perm, dtype, topk_w, dst_row, T, d, k, n_rows,
                                            dy_perm, d_topk_w, as_stream(stream)),
                    "moe_unpermute_combine_bwd");
}


int moe_grouped_gemm_gated_fwd(const void* A, const void* B, const int64_t* offsets, int32_t G,
                               int64_t M, int64_t K, int64_t N, int dtype, const float* row_scale,
                               void* AB, void* H, void* stream) {
  const char* fn = "moe_grouped_gemm_gated_fwd";
  int st = check_gemm(fn, A, B, offsets, G, M, K, N, dtype);
  if (st != MOE_OK) return st;
  REQUIRE(dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "%s: bf16 only", fn);
  REQUIRE(K % 64 == 0 && N % 2 == 0 && (N / 2) % 64 == 0, MOE_ERR_UNSUPPORTED,
          "%s: needs K %% 64 == 0 and f %% 64 == 0 (K=%lld, N=%lld)", fn,
          static_cast<long long>(K), static_cast<long long>(N));
  if (M == 0) return ok();
  REQUIRE(row_scale && H, MOE_ERR_NULL, "%s: row_scale and H are required", fn);
  REQUIRE(aligned16(H) && (AB == nullptr || aligned16(AB)), MOE_ERR_UNSUPPORTED,
          "%s: outputs must be 16-byte aligned", fn);
  return hip_status(moe::launch_gg_bf16_gated_fwd(A, B, offsets, G, M, K, N, row_scale, AB, H,
                                                  as_stream(stream)),
                    fn);
}

int moe_grouped_gemm_gated_dgrad(const void* dC, const void* B, const int64_t* offsets, int32_t G,
                                 int64_t M, int64_t K, int64_t N, int dtype, const void* ab,
                                 const float* row_scale, void* dAB, float* gate_partials,
                                 void* stream) {
  const char* fn = "moe_grouped_gemm_gated_dgrad";
  int st = check_gemm(fn, dC, B, offsets, G, M, K, N, dtype);
  if (st != MOE_OK) return st;
  REQUIRE(dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "%s: bf16 only", fn);
  REQUIRE(N % 64 == 0 && K % 128 == 0, MOE_ERR_UNSUPPORTED,
          "%s: needs N %% 64 == 0 and K %% 128 == 0 (K=%lld, N=%lld)", fn,
          static_cast<long long>(K), static_cast<long long>(N));
  if (M == 0) return ok();
  REQUIRE(ab && row_scale && dAB && gate_partials, MOE_ERR_NULL,
          "%s: ab, row_scale, dAB and gate_partials are required", fn);
  REQUIRE(aligned16(ab) && aligned16(dAB), MOE_ERR_UNSUPPORTED, "%s: ab and dAB must be 16-byte aligned",
          fn);
  return hip_status(moe::launch_gg_bf16_gated_dgrad(dC, B, offsets, G, M, K, N, ab, row_scale,
                                                    dAB, gate_partials, as_stream(stream)),
                    fn);
}

int moe_quant_fp8_rows(const void* x, int64_t M, int64_t K, uint8_t* q, float* scale_t,
                       void* stream) {
  const char* fn = "moe_quant_fp8_rows";
  REQUIRE(M >= 0 && K >= 1, MOE_ERR_SHAPE, "%s: M=%lld K=%lld", fn, static_cast<long long>(M),
          static_cast<long long>(K));
  REQUIRE(K % 128 == 0, MOE_ERR_UNSUPPORTED, "%s: K %% 128 != 0", fn);
  if (M == 0) return ok();
  REQUIRE(x && q && scale_t, MOE_ERR_NULL, "%s: x, q and scale_t are required", fn);
  REQUIRE(aligned16(x) && (reinterpret_cast<uintptr_t>(q) & 7u) == 0, MOE_ERR_UNSUPPORTED,
          "%s: x must be 16-byte and q 8-byte aligned", fn);
  return hip_status(moe::launch_quant_rows(x, M, K, q, scale_t, as_stream(stream)), fn);
}

int moe_quant_fp8_weights(const void* w, int32_t G, int64_t K, int64_t N, uint8_t* q,
                          float* s_fwd, float* s_dgrad, void* stream) {
  const char* fn = "moe_quant_fp8_weights";
  REQUIRE(G >= 1 && K >= 1 && N >= 1, MOE_ERR_SHAPE, "%s: G=%d K=%lld N=%lld", fn, G,
          static_cast<long long>(K), static_cast<long long>(N));
  REQUIRE(K % 128 == 0 && N % 128 == 0, MOE_ERR_UNSUPPORTED, "%s: K and N must be multiples of 128",
          fn);
  REQUIRE(w && q && s_fwd && s_dgrad, MOE_ERR_NULL, "%s: all pointers are required", fn);
  REQUIRE(aligned16(w) && (reinterpret_cast<uintptr_t>(q) & 7u) == 0, MOE_ERR_UNSUPPORTED,
          "%s: w must be 16-byte and q 8-byte aligned", fn);
  return hip_status(moe::launch_quant_weights(w, G, K, N, q, s_fwd, s_dgrad, as_stream(stream)),
                    fn);
}

int64_t moe_padded_rows_bound(int64_t M, int32_t G, int32_t align) {
  if (M < 0 || G < 1 || align < 1 || M > (int64_t(1) << 60)) return 0;
  const int64_t n = M + static_cast<int64_t>(G) * (align - 1);
  return (n + align - 1) / align * align;
}

int moe_padded_offsets(const int64_t* offsets, int32_t G, int64_t M, int32_t align,
                       int64_t* padded, void* stream) {
  const char* fn = "moe_padded_offsets";
  REQUIRE(G >= 1 && M >= 0 && align >= 1, MOE_ERR_SHAPE, "%s: G=%d M=%lld align=%d", fn, G,
          static_cast<long long>(M), align);
  REQUIRE(G <= 1024, MOE_ERR_UNSUPPORTED, "%s: G=%d above 1024", fn, G);
  REQUIRE(offsets && padded, MOE_ERR_NULL, "%s: offsets and padded are required", fn);
  return hip_status(moe::launch_padded_offsets(offsets, G, M, align, padded, as_stream(stream)), fn);
}

int moe_quant_fp8_token_tiles(const void* x, const int64_t* offsets, const int64_t* padded,
                              int32_t G, int64_t M, int64_t K, int64_t ldm, uint8_t* q_t,
                              float* scale, void* stream) {
  const char* fn = "moe_quant_fp8_token_tiles";
  REQUIRE(G >= 1 && M >= 0 && K >= 1 && ldm >= 0, MOE_ERR_SHAPE, "%s: G=%d M=%lld K=%lld ldm=%lld",
          fn, G, static_cast<long long>(M), static_cast<long long>(K), static_cast<long long>(ldm));
  REQUIRE(G <= 1024, MOE_ERR_UNSUPPORTED, "%s: G=%d above 1024", fn, G);
  REQUIRE(K % 128 == 0 && ldm % 128 == 0, MOE_ERR_UNSUPPORTED, "%s: K and ldm must be multiples of 128",
          fn);
  REQUIRE(ldm >= moe_padded_rows_bound(M, G, 128), MOE_ERR_SHAPE,
          "%s: ldm=%lld below the padded bound %lld", fn, static_cast<long long>(ldm),
          static_cast<long long>(moe_padded_rows_bound(M, G, 128)));
  REQUIRE(offsets && padded && q_t && scale && (M == 0 || x), MOE_ERR_NULL,
          "%s: pointers are required", fn);
  REQUIRE(aligned16(x) && (reinterpret_cast<uintptr_t>(q_t) & 7u) == 0, MOE_ERR_UNSUPPORTED,
          "%s: alignment", fn);
  return hip_status(moe::launch_quant_token_tiles(x, offsets, padded, G, M, K, ldm, q_t, scale,
                                                  as_stream(stream)),
                    fn);
}

static int check_gemm_fp8(const char* fn, const void* a, const void* sa, const void* b,
                          const void* sb, const int64_t* off, int32_t G, int64_t M, int64_t K,
                          int64_t N) {
  REQUIRE(G >= 1 && M >= 0 && K >= 1 && N >= 1, MOE_ERR_SHAPE, "%s: G=%d M=%lld K=%lld N=%lld", fn,
          G, static_cast<long long>(M), static_cast<long long>(K), static_cast<long long>(N));
  REQUIRE(G <= 1024, MOE_ERR_UNSUPPORTED, "%s: G=%d above 1024", fn, G);
  REQUIRE(K % 128 == 0 && N % 128 == 0, MOE_ERR_UNSUPPORTED, "%s: K and N must be multiples of 128",
          fn);
  REQUIRE(M / 64 + G < (int64_t(1) << 31) / 64, MOE_ERR_UNSUPPORTED, "%s: M too large", fn);
  // one expert's weight codes are addressed with 32-bit byte offsets
  REQUIRE(prod_below(K, N, int64_t(1) << 32), MOE_ERR_UNSUPPORTED,
          "%s: K*N must be below 2^32 (one expert's weight codes under 4 GiB)", fn);
  if (M == 0) return MOE_OK;
  REQUIRE(a && sa && b && sb && off, MOE_ERR_NULL, "%s: operands, scales and offsets are required",
          fn);
  REQUIRE(aligned16(a) && aligned16(b), MOE_ERR_UNSUPPORTED, "%s: operands must be 16-byte aligned",
          fn);
  return MOE_OK;
}

int moe_grouped_gemm_fp8_fwd(const uint8_t* A, const float* a_scale_t, const uint8_t* B_fwd,
                             const float* b_scale_fwd, const int64_t* offsets, int32_t G,
                             int64_t M, int64_t K, int64_t N, int epilogue, void* C, void* H,
                             void* stream) {
  const char* fn = "moe_grouped_gemm_fp8_fwd";
  int st = check_gemm_fp8(fn, A, a_scale_t, B_fwd, b_scale_fwd, offsets, G, M, K, N);
  if (st != MOE_OK) return st;
  REQUIRE(epilogue == MOE_EPI_NONE || epilogue == MOE_EPI_SWIGLU, MOE_ERR_SHAPE,
          "%s: epilogue %d not available in the forward", fn, epilogue);
  if (epilogue == MOE_EPI_SWIGLU)
    REQUIRE((N / 2) % 64 == 0, MOE_ERR_UNSUPPORTED, "%s: SWIGLU needs N / 2 %% 64 == 0", fn);
  if (M == 0) return ok();
  REQUIRE(epilogue == MOE_EPI_SWIGLU ? H != nullptr : C != nullptr, MOE_ERR_NULL,
          "%s: output missing", fn);
  return hip_status(moe::launch_gg_fp8_fwd(A, a_scale_t, B_fwd, b_scale_fwd, offsets, G, M, K, N,
                                           epilogue, C, H, as_stream(stream)),
                    fn);
}

int moe_grouped_gemm_fp8_dgrad(const uint8_t* dC, const float* dc_scale_t, const uint8_t* B_dgrad,
                               const float* b_scale_dgrad, const int64_t* offsets, int32_t G,
                               int64_t M, int64_t K, int64_t N, int epilogue, const void* ab,
                               void* dA, void* stream) {
  const char* fn = "moe_grouped_gemm_fp8_dgrad";
  int st = check_gemm_fp8(fn, dC, dc_scale_t, B_dgrad, b_scale_dgrad, offsets, G, M, K, N);
  if (st != MOE_OK) return st;
  REQUIRE(epilogue == MOE_EPI_NONE || epilogue == MOE_EPI_SWIGLU_BWD, MOE_ERR_SHAPE,
          "%s: epilogue %d not available in dgrad", fn, epilogue);
  if (M == 0) return ok();
  REQUIRE(dA && (epilogue != MOE_EPI_SWIGLU_BWD || ab), MOE_ERR_NULL, "%s: output missing", fn);
  return hip_status(moe::launch_gg_fp8_dgrad(dC, dc_scale_t, B_dgrad, b_scale_dgrad, offsets, G, M,
                                             K, N, epilogue, ab, dA, as_stream(stream)),
                    fn);
}

int moe_grouped_gemm_fp8_wgrad(const uint8_t* A_t, const float* a_scale, const uint8_t* dC_t,
                               const float* dc_scale, const int64_t* padded, int32_t G,
                               int64_t ldm, int64_t K, int64_t N, int dB_dtype, int accumulate,
                               void* dB, void* stream) {
  const char* fn = "moe_grouped_gemm_fp8_wgrad";
  REQUIRE(G >= 1 && ldm >= 0 && K >= 1 && N >= 1, MOE_ERR_SHAPE, "%s: G=%d ldm=%lld K=%lld N=%lld",
          fn, G, static_cast<long long>(ldm), static_cast<long long>(K), static_cast<long long>(N));
  REQUIRE(G <= 1024, MOE_ERR_UNSUPPORTED, "%s: G=%d above 1024", fn, G);
  REQUIRE(K % 128 == 0 && N % 128 == 0 && ldm % 128 == 0, MOE_ERR_UNSUPPORTED,
          "%s: K, N and ldm must be multiples of 128", fn);
  REQUIRE(dB_dtype == MOE_BF16 || dB_dtype == MOE_F32, MOE_ERR_DTYPE, "%s: dB must be bf16 or fp32",
          fn);
  REQUIRE(padded && dB && a_scale && dc_scale && (ldm == 0 || (A_t && dC_t)), MOE_ERR_NULL,
          "%s: pointers are required", fn);
  REQUIRE(aligned16(A_t) && aligned16(dC_t), MOE_ERR_UNSUPPORTED, "%s: alignment", fn);
  return hip_status(moe::launch_gg_fp8_wgrad(A_t, a_scale, dC_t, dc_scale, padded, G, ldm, K, N,
                                             dB_dtype == MOE_F32, accumulate != 0, dB,
                                             as_stream(stream)),
                    fn);
}

static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
static bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

int moe_quant_mxfp8_rows(const void* x, int64_t M, int64_t K, uint8_t* q, uint8_t* scale,
                         void* stream) {
  const char* fn = "moe_quant_mxfp8_rows";
  REQUIRE(M >= 0 && K >= 1, MOE_ERR_SHAPE, "%s: M=%lld K=%lld", fn, static_cast<long long>(M),
          static_cast<long long>(K));
  REQUIRE(K % 128 == 0, MOE_ERR_UNSUPPORTED, "%s: K %% 128 != 0", fn);
  if (M == 0) return ok();
  REQUIRE(x && q && scale, MOE_ERR_NULL, "%s: x, q and scale are required", fn);
  REQUIRE(aligned16(x) && aligned8(q) && aligned4(scale), MOE_ERR_UNSUPPORTED, "%s: alignment", fn);
  return hip_status(moe::launch_quant_mx_rows(x, M, nullptr, nullptr, M, K, q, scale,
                                              as_stream(stream)),
                    fn);
}

int moe_permute_quant_mxfp8(const void* x, int64_t T, int64_t K, const int32_t* src_token,
                            const int64_t* offsets, int32_t G, int64_t M, uint8_t* q,
                            uint8_t* scale, void* stream) {
  const char* fn = "moe_permute_quant_mxfp8";
  REQUIRE(T >= 0 && K >= 1 && G >= 1 && M >= 0, MOE_ERR_SHAPE, "%s: T=%lld K=%lld G=%d M=%lld", fn,
          static_cast<long long>(T), static_cast<long long>(K), G, static_cast<long long>(M));
  REQUIRE(K % 128 == 0, MOE_ERR_UNSUPPORTED, "%s: K %% 128 != 0", fn);
  if (M == 0) return ok();
  REQUIRE(src_token && offsets && q && scale && (T == 0 || x), MOE_ERR_NULL,
          "%s: pointers are required", fn);
  REQUIRE(aligned16(x) && aligned8(q) && aligned4(scale), MOE_ERR_UNSUPPORTED, "%s: alignment", fn);
  return hip_status(moe::launch_quant_mx_rows(x, T, src_token, offsets + G, M, K, q, scale,
                                              as_stream(stream)),
                    fn);
}

int moe_scatter_quant_mxfp8(const void* x, int64_t T, int64_t K, const int32_t* dst_row,
                            int32_t k, const int64_t* offsets, int32_t G, int64_t M, uint8_t* q,
                            uint8_t* scale, void* stream) {
  const char* fn = "moe_scatter_quant_mxfp8";
  REQUIRE(T >= 0 && K >= 1 && k >= 1 && G >= 1 && M >= 0, MOE_ERR_SHAPE,
          "%s: T=%lld K=%lld k=%d G=%d M=%lld", fn, static_cast<long long>(T),
          static_cast<long long>(K), k, G, static_cast<long long>(M));
  REQUIRE(K % 128 == 0, MOE_ERR_UNSUPPORTED, "%s: K %% 128 != 0", fn);
  if (T == 0 || M == 0) return ok();
  REQUIRE(x && dst_row && offsets && q && scale, MOE_ERR_NULL, "%s: pointers are required", fn);
  REQUIRE(aligned16(x) && aligned8(q) && aligned4(scale), MOE_ERR_UNSUPPORTED, "%s: alignment", fn);
  return hip_status(moe::launch_quant_mx_scatter(x, T, K, dst_row, k, offsets + G, M, q, scale,
                                                 as_stream(stream)),
                    fn);
}

int moe_quant_mxfp8_weights(const void* w, int32_t G, int64_t K, int64_t N, uint8_t* q_fwd,
                            uint8_t* s_fwd, uint8_t* q_dgrad, uint8_t* s_dgrad, void* stream) {
  const char* fn = "moe_quant_mxfp8_weights";
  REQUIRE(G >= 1 && K >= 1 && N >= 1, MOE_ERR_SHAPE, "%s: G=%d K=%lld N=%lld", fn, G,
          static_cast<long long>(K), static_cast<long long>(N));
  REQUIRE(K % 128 == 0 && N % 128 == 0, MOE_ERR_UNSUPPORTED, "%s: K and N must be multiples of 128",
          fn);
  REQUIRE(w && q_fwd && s_fwd && q_dgrad && s_dgrad, MOE_ERR_NULL, "%s: all pointers are required",
          fn);
  REQUIRE(aligned16(w) && aligned8(q_fwd) && aligned8(q_dgrad) && aligned4(s_fwd) &&
              aligned4(s_dgrad),
          MOE_ERR_UNSUPPORTED, "%s: alignment", fn);
  return hip_status(moe::launch_quant_mx_weights(w, G, K, N, q_fwd, s_fwd, q_dgrad, s_dgrad,
                                                 as_stream(stream)),
                    fn);
}

int moe_quant_mxfp8_token_tiles(const void* x, int64_t x_rows, const int32_t* src_row,
                                const int64_t* offsets, const int64_t* padded, int32_t G,
                                int64_t M, int64_t K, int64_t ldm, uint8_t* q_t, uint8_t* scale_t,
                                void* stream) {
  const char* fn = "moe_quant_mxfp8_token_tiles";
  REQUIRE(G >= 1 && M >= 0 && K >= 1 && ldm >= 0 && x_rows >= 0, MOE_ERR_SHAPE,
          "%s: G=%d M=%lld K=%lld ldm=%lld x_rows=%lld", fn, G, static_cast<long long>(M),
          static_cast<long long>(K), static_cast<long long>(ldm), static_cast<long long>(x_rows));
  REQUIRE(G <= 1024, MOE_ERR_UNSUPPORTED, "%s: G=%d above 1024", fn, G);
  REQUIRE(K % 128 == 0 && ldm % 128 == 0, MOE_ERR_UNSUPPORTED,
          "%s: K and ldm must be multiples of 128", fn);
  REQUIRE(ldm >= moe_padded_rows_bound(M, G, 128), MOE_ERR_SHAPE,
          "%s: ldm=%lld below the padded bound %lld", fn, static_cast<long long>(ldm),
          static_cast<long long>(moe_padded_rows_bound(M, G, 128)));
  REQUIRE(src_row || x_rows == M, MOE_ERR_SHAPE, "%s: without src_row, x_rows must equal M", fn);
  REQUIRE(offsets && padded && q_t && scale_t && (x_rows == 0 || x), MOE_ERR_NULL,
          "%s: pointers are required", fn);
  REQUIRE(aligned16(x) && aligned8(q_t) && aligned4(scale_t), MOE_ERR_UNSUPPORTED, "%s: alignment",
          fn);
  return hip_status(moe::launch_quant_mx_token_tiles(x, x_rows, src_row, offsets, padded, G, M, K,
                                                     ldm, q_t, scale_t, as_stream(stream)),
                    fn);
}

static int check_gemm_mx(const char* fn, const void* a, const void* sa, const void* b,
                         const void* sb, const int64_t* off, int32_t G, int64_t M, int64_t K,
                         int64_t N) {
  int st = check_gemm_fp8(fn, a, sa, b, sb, off, G, M, K, N);
  if (st != MOE_OK || M == 0) return st;
  REQUIRE(aligned4(sa) && aligned4(sb), MOE_ERR_UNSUPPORTED, "%s: scales must be 4-byte aligned",
          fn);
  return MOE_OK;
}

int moe_grouped_gemm_mxfp8_fwd(const uint8_t* A, const uint8_t* a_scale, const uint8_t* B_fwd,
                               const uint8_t* b_scale_fwd, const int64_t* offsets, int32_t G,
                               int64_t M, int64_t K, int64_t N, int epilogue, void* C, void* H,
                               void* stream) {
  const char* fn = "moe_grouped_gemm_mxfp8_fwd";
  int st = check_gemm_mx(fn, A, a_scale, B_fwd, b_scale_fwd, offsets, G, M, K, N);
  if (st != MOE_OK) return st;
  REQUIRE(epilogue == MOE_EPI_NONE || epilogue == MOE_EPI_SWIGLU, MOE_ERR_SHAPE,
          "%s: epilogue %d not available in the forward", fn, epilogue);
  if (epilogue == MOE_EPI_SWIGLU)
    REQUIRE((N / 2) % 64 == 0, MOE_ERR_UNSUPPORTED, "%s: SWIGLU needs N / 2 %% 64 == 0", fn);
  if (M == 0) return ok();
  REQUIRE(epilogue == MOE_EPI_SWIGLU ? H != nullptr : C != nullptr, MOE_ERR_NULL,
          "%s: output missing", fn);
  return hip_status(moe::launch_gg_mx_fwd(A, a_scale, B_fwd, b_scale_fwd, offsets, G, M, K, N,
                                          epilogue, C, H, as_stream(stream)),
                    fn);
}

int moe_grouped_gemm_mxfp8_dgrad(const uint8_t* dC, const uint8_t* dc_scale,
                                 const uint8_t* B_dgrad, const uint8_t* b_scale_dgrad,
                                 const int64_t* offsets, int32_t G, int64_t M, int64_t K, int64_t N,
                                 int epilogue, const void* ab, void* dA, void* stream) {
  const char* fn = "moe_grouped_gemm_mxfp8_dgrad";
  int st = check_gemm_mx(fn, dC, dc_scale, B_dgrad, b_scale_dgrad, offsets, G, M, K, N);
  if (st != MOE_OK) return st;
  REQUIRE(epilogue == MOE_EPI_NONE || epilogue == MOE_EPI_SWIGLU_BWD, MOE_ERR_SHAPE,
          "%s: epilogue %d not available in dgrad", fn, epilogue);
  if (M == 0) return ok();
  REQUIRE(dA && (epilogue != MOE_EPI_SWIGLU_BWD || ab), MOE_ERR_NULL, "%s: output missing", fn);
  return hip_status(moe::launch_gg_mx_dgrad(dC, dc_scale, B_dgrad, b_scale_dgrad, offsets, G, M, K,
                                            N, epilogue, ab, dA, as_stream(stream)),
                    fn);
}

int moe_grouped_gemm_mxfp8_wgrad(const uint8_t* A_t, const uint8_t* a_scale_t,
                                 const uint8_t* dC_t, const uint8_t* dc_scale_t,
                                 const int64_t* padded, int32_t G, int64_t ldm, int64_t K,
                                 int64_t N, int dB_dtype, int accumulate, void* dB, void* stream) {
  const char* fn = "moe_grouped_gemm_mxfp8_wgrad";
  REQUIRE(G >= 1 && ldm >= 0 && K >= 1 && N >= 1, MOE_ERR_SHAPE, "%s: G=%d ldm=%lld K=%lld N=%lld",
          fn, G, static_cast<long long>(ldm), static_cast<long long>(K), static_cast<long long>(N));
  REQUIRE(G <= 1024, MOE_ERR_UNSUPPORTED, "%s: G=%d above 1024", fn, G);
  REQUIRE(K % 128 == 0 && N % 128 == 0 && ldm % 128 == 0, MOE_ERR_UNSUPPORTED,
          "%s: K, N and ldm must be multiples of 128", fn);
  REQUIRE(dB_dtype == MOE_BF16 || dB_dtype == MOE_F32, MOE_ERR_DTYPE, "%s: dB must be bf16 or fp32",
          fn);
  REQUIRE(padded && dB && a_scale_t && dc_scale_t && (ldm == 0 || (A_t && dC_t)), MOE_ERR_NULL,
          "%s: pointers are required", fn);
  REQUIRE(aligned16(A_t) && aligned16(dC_t) && aligned4(a_scale_t) && aligned4(dc_scale_t),
          MOE_ERR_UNSUPPORTED, "%s: alignment", fn);
  return hip_status(moe::launch_gg_mx_wgrad(A_t, a_scale_t, dC_t, dc_scale_t, padded, G, ldm, K, N,
                                            dB_dtype == MOE_F32, accumulate != 0, dB,
                                            as_stream(stream)),
                    fn);
}

}  // extern "C"
