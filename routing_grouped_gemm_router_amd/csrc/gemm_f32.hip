// fp32 vector-ALU GEMM family: the router projection and its backward (the
// router stays in FP32 -- "Scalable Training of Mixture-of-Experts Models with
// Megatron Core", section 5, Selective precision) and the fp32 grouped expert
// GEMMs (section 2, Expert Computation).
//
//   C[m, n] (+)= sum_k Aop(m, k) * Bop(k, n)
//   Aop(m, k) = A[m * lda + k]            (A_MC = false: k contiguous)
//             = A[k * lda + m]            (A_MC = true:  m contiguous)
//   Bop(k, n) = B[k * ldb + n]            (B_KC = false: n contiguous)
//             = B[n * ldb + k]            (B_KC = true:  k contiguous)
// Grouping: GRP_NONE one problem; GRP_M groups of rows [off[g], off[g+1]) with
// B advanced by g * strideB; GRP_K groups of the contraction range with C
// advanced by g * strideC.
//
// Tile 64 x 64 x 16, 256 threads, 4 x 4 outputs per thread, operands staged
// through LDS as [k][m] and [k][n] so every thread's inner product reads two
// 16-byte LDS vectors per k.  Every access is bounds-checked, so any M, N, K.
#include "common.h"
#include "internal.h"

namespace moe {

constexpr int FBM = 64, FBN = 64, FBK = 16, FPAD = 4;

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  fill_zero_kernel<<<dim3(static_cast<unsigned>(b)), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

template <typename TA, bool A_MC, bool B_KC, int GRP, int EPI, typename TC>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const TA* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ B, int64_t ldb,
                                                       int64_t strideB, TC* __restrict__ C,
                                                       int64_t ldc, int64_t strideC,
                                                       const int64_t* __restrict__ off, int G,
                                                       int64_t M, int64_t N, int64_t K,
                                                       const float* __restrict__ bias,
                                                       const TC* __restrict__ ab, TC* __restrict__ H,
                                                       int accumulate) {
  __shared__ float As[FBK][FBM + FPAD];
  __shared__ float Bs[FBK][FBN + FPAD];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;

  // ---- which rows / contraction range / group this block owns
  int64_t m_lo = static_cast<int64_t>(blockIdx.y) * FBM, m_hi = M;
  int64_t k_lo = 0, k_hi = K;
  int g = 0;
  if (GRP == GRP_M) {
    // blockIdx.y enumerates (group, row tile) pairs in order
    int64_t tile = blockIdx.y;
    bool found = false;
    for (g = 0; g < G; ++g) {
      int64_t lo = off[g], hi = off[g + 1];
      lo = lo < 0 ? 0 : (lo > M ? M : lo);
      hi = hi < lo ? lo : (hi > M ? M : hi);
      const int64_t nt = (hi - lo + FBM - 1) / FBM;
      if (tile < nt) {
        m_lo = lo + tile * FBM;
        m_hi = hi;
        found = true;
        break;
      }
      tile -= nt;
    }
    if (!found) return;
    B += static_cast<int64_t>(g) * strideB;
  } else if (GRP == GRP_K) {
    g = blockIdx.z;
    int64_t lo = off[g], hi = off[g + 1];
    lo = lo < 0 ? 0 : (lo > K ? K : lo);
    hi = hi < lo ? lo : (hi > K ? K : hi);
    k_lo = lo;
    k_hi = hi;
    C += static_cast<int64_t>(g) * strideC;
  }
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * (EPI == EPI_SWIGLU ? FBN / 2 : FBN);
  const int64_t fh = N / 2;  // SWIGLU: width of each half

  // tile column c -> global output column of Bop
  auto colmap = [&](int c) -> int64_t {
    if (EPI == EPI_SWIGLU) {
      const int q = c & 3;
      return (q < 2 ? 0 : fh) + n0 + (c >> 2) * 2 + (q & 1);
    }
    return n0 + c;
  };
  const int64_t n_lim = EPI == EPI_SWIGLU ? fh : N;

  float acc[4][4] = {};
  for (int64_t k0 = k_lo; k0 < k_hi; k0 += FBK) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = tid + v * 256;
      int mm, kk;
      if (A_MC) { kk = e >> 6; mm = e & 63; } else { kk = e & 15; mm = e >> 4; }
      const int64_t m = m_lo + mm, k = k0 + kk;
      float val = 0.f;
      if (m < m_hi && k < k_hi)
        val = Elem<TA>::ld(A_MC ? A + k * lda + m : A + m * lda + k);
      As[kk][mm] = val;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = tid + v * 256;
      int nn, kk;
      if (B_KC) { kk = e & 15; nn = e >> 4; } else { kk = e >> 6; nn = e & 63; }
      const int64_t k = k0 + kk;
      const int64_t logical = EPI == EPI_SWIGLU ? n0 + (nn >> 2) * 2 + (nn & 1) : n0 + nn;
      const int64_t n = colmap(nn);
      float val = 0.f;
      if (logical < n_lim && k < k_hi) val = B_KC ? B[n * ldb + k] : B[k * ldb + n];
      Bs[kk][nn] = val;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m_lo + ty * 4 + i;
    if (m >= m_hi || (GRP != GRP_M && m >= M)) continue;
    if (EPI == EPI_SWIGLU) {
      // columns j = 0, 1 are gates, j = 2, 3 the matching up projections
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t c = n0 + tx * 2 + j;
        if (c >= fh) continue;
        const float a = acc[i][j], b = acc[i][j + 2];
        if (C) {
          Elem<TC>::st(C + m * ldc + c, a);
          Elem<TC>::st(C + m * ldc + fh + c, b);
        }
        Elem<TC>::st(H + m * fh + c, a / (1.0f + expf(-a)) * b);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + tx * 4 + j;
        if (n >= N) continue;
        float v = acc[i][j];
        if (EPI == EPI_BIAS && bias) v = v + bias[n];
        if (EPI == EPI_SWIGLU_BWD) {
          // v is dH[m, n]; ab / output rows are 2N wide
          const float a = Elem<TC>::ld(ab + m * 2 * N + n);
          const float b = Elem<TC>::ld(ab + m * 2 * N + N + n);
          const float s = 1.0f / (1.0f + expf(-a));
          Elem<TC>::st(C + m * 2 * N + n, v * b * s * (1.0f + a * (1.0f - s)));
          Elem<TC>::st(C + m * 2 * N + N + n, v * a * s);
          continue;
        }
        TC* p = C + m * ldc + n;
        if (accumulate) v += Elem<TC>::ld(p);
        Elem<TC>::st(p, v);
      }
    }
  }
}

template <typename TA, bool A_MC, bool B_KC, int GRP, int EPI, typename TC>
static hipError_t run_f32(const TA* A, int64_t lda, const float* B, int64_t ldb, int64_t strideB,
                          TC* C, int64_t ldc, int64_t strideC, const int64_t* off, int G,
                          int64_t M, int64_t N, int64_t K, const float* bias, const TC* ab, TC* H,
                          int accumulate, hipStream_t s) {
  const int64_t ncols = EPI == EPI_SWIGLU ? N / 2 : N;
  const int64_t bn = EPI == EPI_SWIGLU ? FBN / 2 : FBN;
  dim3 grid(static_cast<unsigned>((ncols + bn - 1) / bn), 1, 1);
  if (GRP == GRP_M)
    grid.y = static_cast<unsigned>(M / FBM + G);
  else
    grid.y = static_cast<unsigned>((M + FBM - 1) / FBM);
  if (GRP == GRP_K) grid.z = G;
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  gemm_f32_kernel<TA, A_MC, B_KC, GRP, EPI, TC><<<grid, 256, 0, s>>>(
      A, lda, B, ldb, strideB, C, ldc, strideC, off, G, M, N, K, bias, ab, H, accumulate);
  return hipGetLastError();
}

hipError_t launch_router_fwd(const void* x, int x_dtype, const float* w_r, const float* bias,
                             int64_t T, int64_t d, int E, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (x_dtype == 0)
    return run_f32<float, false, false, GRP_NONE, EPI_BIAS, float>(
        static_cast<const float*>(x), d, w_r, E, 0, logits, E, 0, nullptr, 1, T, E, d, bias,
        nullptr, nullptr, 0, s);
  return run_f32<bf16_t, false, false, GRP_NONE, EPI_BIAS, float>(
      static_cast<const bf16_t*>(x), d, w_r, E, 0, logits, E, 0, nullptr, 1, T, E, d, bias,
      nullptr, nullptr, 0, s);
}

hipError_t launch_router_bwd(const void* x, int x_dtype, const float* w_r, const float* dz,
                             int64_t T, int64_t d, int E, float* dw_r, float* dx_r,
                             hipStream_t s) {
  hipError_t err = hipSuccess;
  if (dw_r) {
    // dW_r [d, E] = x^T [d, T] . dz [T, E]
    if (T == 0) {
      err = launch_fill_zero(dw_r, d * E, s);
    } else if (x_dtype == 0) {
      err = run_f32<float, true, false, GRP_NONE, EPI_NONE, float>(
          static_cast<const float*>(x), d, dz, E, 0, dw_r, E, 0, nullptr, 1, d, E, T, nullptr,
          nullptr, nullptr, 0, s);
    } else {
      err = run_f32<bf16_t, true, false, GRP_NONE, EPI_NONE, float>(
          static_cast<const bf16_t*>(x), d, dz, E, 0, dw_r, E, 0, nullptr, 1, d, E, T, nullptr,
          nullptr, nullptr, 0, s);
    }
    if (err != hipSuccess) return err;
  }
  if (dx_r && T > 0) {
    // dx_r [T, d] = dz [T, E] . W_r^T  (Bop(k=e, n=i) = W_r[i * E + e])
    err = run_f32<float, false, true, GRP_NONE, EPI_NONE, float>(
        dz, E, w_r, E, 0, dx_r, d, 0, nullptr, 1, T, d, E, nullptr, nullptr, nullptr, 0, s);
  }
  return err;
}

hipError_t launch_gg_f32_fwd(const float* A, const float* B, const int64_t* off, int G, int64_t M,
                             int64_t K, int64_t N, int epi, float* C, float* H, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (epi == EPI_SWIGLU)
    return run_f32<float, false, false, GRP_M, EPI_SWIGLU, float>(A, K, B, N, K * N, C, N, 0, off,
                                                                  G, M, N, K, nullptr, nullptr, H,
                                                                  0, s);
  return run_f32<float, false, false, GRP_M, EPI_NONE, float>(A, K, B, N, K * N, C, N, 0, off, G,
                                                              M, N, K, nullptr, nullptr, nullptr,
                                                              0, s);
}

hipError_t launch_gg_f32_dgrad(const float* dC, const float* B, const int64_t* off, int G,
                               int64_t M, int64_t K, int64_t N, int epi, const float* ab,
                               float* dA, hipStream_t s) {
  // dA [M, K] = dC [M, N] . B_g^T : Bop(k = n_c, n = k_out) = B_g[k_out * N + n_c]
  if (M == 0) return hipSuccess;
  if (epi == EPI_SWIGLU_BWD)
    return run_f32<float, false, true, GRP_M, EPI_SWIGLU_BWD, float>(
        dC, N, B, N, K * N, dA, K, 0, off, G, M, K, N, nullptr, ab, nullptr, 0, s);
  return run_f32<float, false, true, GRP_M, EPI_NONE, float>(dC, N, B, N, K * N, dA, K, 0, off, G,
                                                             M, K, N, nullptr, nullptr, nullptr, 0,
                                                             s);
}

hipError_t launch_gg_f32_wgrad(const float* A, const float* dC, const int64_t* off, int G,
                               int64_t M, int64_t K, int64_t N, int accumulate, float* dB,
                               hipStream_t s) {
  // dB_g [K, N] = A_g^T . dC_g : Aop(m = k_out, k = row) = A[row * K + k_out]
  return run_f32<float, true, false, GRP_K, EPI_NONE, float>(A, K, dC, N, 0, dB, N, K * N, off, G,
                                                             K, N, M, nullptr, nullptr, nullptr,
                                                             accumulate, s);
}

}  // namespace moe
