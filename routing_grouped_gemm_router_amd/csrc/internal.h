// Launchers of the HIP kernels, called by the C-ABI layer after validation.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace moe {

enum { GRP_NONE = 0, GRP_M = 1, GRP_K = 2 };
enum { EPI_NONE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2, EPI_BIAS = 3 };

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);

// route.hip
size_t route_topk_workspace(int64_t T, int E);
// the allocation-free route's per-device scratch: its size, and its device
// address on the current device (looked up once per device)
size_t route_noalloc_scratch_bytes();
hipError_t route_scratch_ptr(void** out);
hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int score, int renorm,
                             const float* sel_bias, int32_t* topk_idx, float* topk_w,
                             int32_t* counts, int64_t* offsets, int32_t* dst_row,
                             int32_t* src_token, void* ws, hipStream_t stream);
hipError_t launch_pad_to_max(const int32_t* topk_idx, const int32_t* counts,
                             const int64_t* offsets, const int32_t* dst_row,
                             const int32_t* src_token, int64_t T, int E, int k, int64_t C,
                             int32_t* counts_out, int64_t* offsets_out, int32_t* dst_row_out,
                             int32_t* src_token_out, hipStream_t stream);
hipError_t launch_zero_unmapped_rows(void* buf, int64_t row_bytes, const int32_t* src_token,
                                     int64_t M, hipStream_t s);
hipError_t launch_expert_bias_update(const int32_t* counts, int E, float rate, float* bias,
                                     hipStream_t stream);
hipError_t launch_check_finite(const float* p, int64_t n, int32_t* status, hipStream_t stream);
hipError_t launch_check_dispatch(const int32_t* topk_idx, const int32_t* counts,
                                 const int64_t* offsets, const int32_t* dst_row,
                                 const int32_t* src_token, int64_t T, int E, int k, int64_t n_rows,
                                 int32_t* status, hipStream_t stream);
hipError_t launch_route_replay(const float* logits, const int32_t* idx_in, int64_t T, int E, int k,
                               int score, int renorm, int32_t* topk_idx, float* topk_w,
                               int32_t* counts, int64_t* offsets, int32_t* dst_row,
                               int32_t* src_token, int32_t* status, void* ws, hipStream_t stream);
hipError_t launch_apply_capacity(const int32_t* topk_idx, const int32_t* counts,
                                 const int64_t* offsets, const int32_t* dst_row, int64_t T, int E,
                                 int k, int64_t C, int32_t* counts_out, int64_t* offsets_out,
                                 int32_t* dst_out, int32_t* src_out, hipStream_t stream);
size_t aux_loss_workspace(int64_t T, int E);
hipError_t launch_aux_loss(const float* logits, const int32_t* counts, int64_t T, int E, int k,
                           int score, float coeff, float* loss, float* d_logits, void* ws,
                           hipStream_t stream);
hipError_t launch_route_topk_bwd(const float* logits, const int32_t* topk_idx, const float* topk_w,
                                 const float* d_topk_w, int64_t T, int E, int k, int score,
                                 int renorm, float* d_logits, hipStream_t s);

// permute.hip
// nrows: rows of the permuted buffer (T * k dropless, E * capacity padded);
// dst_row entries outside [0, nrows) are skipped
hipError_t launch_permute(const void* x, int dtype, const int32_t* dst_row, int64_t T, int64_t d,
                          int k, int64_t nrows, void* xp, hipStream_t s);
hipError_t launch_permute_bwd(const void* dxp, int dtype, const int32_t* dst_row, int64_t T,
                              int64_t d, int k, int64_t nrows, const void* addend,
                              const float* addend_f32, void* dx, hipStream_t s);
hipError_t launch_combine(const void* y, int dtype, const float* topk_w, const int32_t* dst_row,
                          const void* shared, int64_t T, int64_t d, int k, int64_t nrows,
                          void* out, hipStream_t s);
hipError_t launch_combine_bwd(const void* dout, const void* y, int dtype, const float* topk_w,
                              const int32_t* dst_row, int64_t T, int64_t d, int k, int64_t nrows,
                              void* dy, float* d_w, hipStream_t s);
hipError_t launch_swiglu(const void* ab, int dtype, int64_t M, int64_t f, void* h, hipStream_t s);
hipError_t launch_swiglu_bwd(const void* dh, const void* ab, int dtype, int64_t M, int64_t f,
                             void* dab, hipStream_t s);

// gemm_f32.hip
hipError_t launch_router_fwd(const void* x, int x_dtype, const float* w_r, const float* bias,
                             int64_t T, int64_t d, int E, float* logits, hipStream_t s);
hipError_t launch_router_bwd(const void* x, int x_dtype, const float* w_r, const float* dz,
                             int64_t T, int64_t d, int E, float* dw_r, float* dx_r, hipStream_t s);
hipError_t launch_router_bwd_topk(const void* x, int x_dtype, const float* w_r, const float* dz,
                                  const int32_t* topk_idx, const int64_t* offsets,
                                  const int32_t* src_token, int64_t T, int64_t d, int E, int k,
                                  float* dw_r, float* dx_r, hipStream_t s);
hipError_t launch_gg_f32_fwd(const float* A, const float* B, const int64_t* off, int G, int64_t M,
                             int64_t K, int64_t N, int epi, float* C, float* H, hipStream_t s);
hipError_t launch_gg_f32_dgrad(const float* dC, const float* B, const int64_t* off, int G,
                               int64_t M, int64_t K, int64_t N, int epi, const float* ab,
                               float* dA, hipStream_t s);
hipError_t launch_gg_f32_wgrad(const float* A, const float* dC, const int64_t* off, int G,
                               int64_t M, int64_t K, int64_t N, int accumulate, float* dB,
                               hipStream_t s);

// gemm_bf16.hip
hipError_t launch_gg_bf16_fwd(const void* A, const void* B, const int64_t* off, int G, int64_t M,
                              int64_t K, int64_t N, int epi, void* C, void* H, hipStream_t s);
hipError_t launch_gg_bf16_dgrad(const void* dC, const void* B, const int64_t* off, int G,
                                int64_t M, int64_t K, int64_t N, int epi, const void* ab, void* dA,
                                hipStream_t s);
hipError_t launch_gg_bf16_wgrad(const void* A, const void* dC, const int64_t* off, int G,
                                int64_t M, int64_t K, int64_t N, int db_f32, int accumulate,
                                void* dB, hipStream_t s);

// grouped_gemm.hip, fp8 E4M3 operands (all k-contiguous) with fp32 row scales
hipError_t launch_gg_bf16_gated_fwd(const void* A, const void* B, const int64_t* off, int G,
                                    int64_t M, int64_t K, int64_t N, const float* row_scale,
                                    void* AB, void* H, hipStream_t s);
hipError_t launch_gg_bf16_gated_dgrad(const void* dC, const void* B, const int64_t* off, int G,
                                      int64_t M, int64_t K, int64_t N, const void* ab,
                                      const float* row_scale, void* dAB, float* gate_part,
                                      hipStream_t s);
hipError_t launch_permute_weights(const float* topk_w, const int32_t* dst_row, int64_t T, int k,
                                  float* w_perm, hipStream_t s);
hipError_t launch_gate_grad(const float* gate_part, int64_t P, const int32_t* dst_row, int64_t T,
                            int k, float* d_topk_w, hipStream_t s);
hipError_t launch_gg_fp8_fwd(const uint8_t* A, const float* sa, const uint8_t* Bt, const float* sb,
                             const int64_t* off, int G, int64_t M, int64_t K, int64_t N, int epi,
                             void* C, void* H, hipStream_t s);
hipError_t launch_gg_fp8_dgrad(const uint8_t* dC, const float* sa, const uint8_t* B,
                               const float* sb, const int64_t* off, int G, int64_t M, int64_t K,
                               int64_t N, int epi, const void* ab, void* dA, hipStream_t s);
hipError_t launch_gg_fp8_wgrad(const uint8_t* At, const float* sa, const uint8_t* dCt,
                               const float* sb, const int64_t* poff, int G, int64_t ldm, int64_t K,
                               int64_t N, int db_f32, int accumulate, void* dB, hipStream_t s);
hipError_t launch_gg_mx_fwd(const uint8_t* A, const uint8_t* ea, const uint8_t* Bt,
                            const uint8_t* eb, const int64_t* off, int G, int64_t M, int64_t K,
                            int64_t N, int epi, void* C, void* H, hipStream_t s);
hipError_t launch_gg_mx_dgrad(const uint8_t* dC, const uint8_t* ea, const uint8_t* B,
                              const uint8_t* eb, const int64_t* off, int G, int64_t M, int64_t K,
                              int64_t N, int epi, const void* ab, void* dA, hipStream_t s);
hipError_t launch_gg_mx_wgrad(const uint8_t* At, const uint8_t* ea, const uint8_t* dCt,
                              const uint8_t* eb, const int64_t* poff, int G, int64_t ldm, int64_t K,
                              int64_t N, int db_f32, int accumulate, void* dB, hipStream_t s);

// quant.hip
hipError_t launch_quant_rows(const void* x, int64_t M, int64_t K, uint8_t* q, float* sT,
                             hipStream_t s);
hipError_t launch_quant_weights(const void* w, int G, int64_t K, int64_t N, uint8_t* q, float* sf,
                                float* sd, hipStream_t s);
hipError_t launch_padded_offsets(const int64_t* off, int G, int64_t M, int64_t align,
                                 int64_t* poff, hipStream_t s);
hipError_t launch_quant_mx_rows(const void* x, int64_t x_rows, const int32_t* src,
                                const int64_t* rows_end, int64_t M, int64_t K, uint8_t* q,
                                uint8_t* e, hipStream_t s);
hipError_t launch_quant_mx_scatter(const void* x, int64_t T, int64_t K, const int32_t* dst_row,
                                   int k, const int64_t* rows_end, int64_t M, uint8_t* q,
                                   uint8_t* e, hipStream_t s);
hipError_t launch_quant_mx_weights(const void* w, int G, int64_t K, int64_t N, uint8_t* qf,
                                   uint8_t* ef, uint8_t* qd, uint8_t* ed, hipStream_t s);
hipError_t launch_quant_mx_token_tiles(const void* x, int64_t x_rows, const int32_t* src,
                                       const int64_t* off, const int64_t* poff, int G, int64_t M,
                                       int64_t K, int64_t ldm, uint8_t* qT, uint8_t* eT,
                                       hipStream_t st);
hipError_t launch_quant_token_tiles(const void* x, const int64_t* off, const int64_t* poff, int G,
                                    int64_t M, int64_t K, int64_t ldm, uint8_t* qT, float* s,
                                    hipStream_t st);

}  // namespace moe
