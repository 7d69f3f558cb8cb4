// fp32 GEMM family: the router projection and its backward (the router stays
// in FP32 -- "Scalable Training of Mixture-of-Experts Models with Megatron
// Core", section 5, Selective precision: fp32-accurate products on the matrix
// cores) and the fp32 grouped expert GEMMs (section 2, Expert Computation, on
// the vector ALUs).
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


// ---- router GEMMs --------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));
enum { RA_KC_BF16 = 0, RA_KC_F32 = 1, RA_MC_BF16 = 2, RA_MC_F32 = 3 };  // A: k- or m-contiguous
enum { RB_NC = 0, RB_KC = 1 };                                          // B (fp32): n- or k-contiguous

struct RSlice {  // one lane's share of a 16-deep slice of A and B
  float4 a[4];
  float4 b[4];
};

__device__ __forceinline__ float4 ld4_f32(const float* p, bool ok) {
  return ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
}

// 8 bf16 -> two float4
__device__ __forceinline__ void ld8_bf16(const bf16_t* p, bool ok, float4& lo, float4& hi) {
  uint4 v = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
  lo = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                   __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
  hi = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xffff0000u),
                   __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xffff0000u));
}

// ---- router products on the bf16 matrix cores, fp32-accurate ----------------
// An fp32 operand v is split exactly into three bf16 terms, v = hi + mid + lo
// + r: hi = bf16(v), mid = bf16(v - hi), lo = bf16(v - hi - mid), each
// rounded to nearest even; both residuals are exact in fp32 (each is v with
// its leading bits removed), and |r| is about 2^-24 |v|, the rounding of an
// fp32 value.  A product of two split operands keeps the term pairs whose
// combined weight is at least 2^-16 (hi.hi, hi.mid, mid.hi, hi.lo, lo.hi,
// mid.mid); every bf16 product is exact in the fp32 accumulator.  So the
// result carries fp32 accuracy while the matrix cores run at their bf16 rate
// (the router stays FP32 in what it computes).  Activations that are already
// bf16 need no split (one term).
//
// C[m, n] = sum_k A[m, k] B(k, n), one wave per 64 x 64 tile as 2 x 2 MFMA
// 32x32x16 blocks, operands loaded straight into the MFMA fragments: lane
// half h of a 16-deep step holds k = 8 h .. 8 h + 7 of its row (A) or column
// (B).  A is k-contiguous (x: bf16 or fp32; d_logits: fp32).  B is W_r: for
// the logits W_r[k, n] (k strided: eight scalar loads per fragment, L2
// resident), for the router's dx W_r[n, k] (k-contiguous).  SK = 8: the 8
// waves of a workgroup split the contraction of one tile and add their
// partials in wave order through LDS.
typedef __bf16 bf16x8_rt __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_rt __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// eight fp32 values -> their hi, mid and lo bf16 terms
__device__ __forceinline__ void split3x8(const float (&v)[8], bf16x8_rt (&t)[3]) {
#pragma clang fp contract(off)
  u32x4_rt h, m, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = v[2 * i], b = v[2 * i + 1];
    const uint32_t hw = f32x2_to_bf16x2(a, b);
    const float ra = a - bf16_lo_f(hw), rb = b - bf16_hi_f(hw);
    const uint32_t mw = f32x2_to_bf16x2(ra, rb);
    const float sa = ra - bf16_lo_f(mw), sb = rb - bf16_hi_f(mw);
    h[i] = hw;
    m[i] = mw;
    l[i] = f32x2_to_bf16x2(sa, sb);
  }
  t[0] = __builtin_bit_cast(bf16x8_rt, h);
  t[1] = __builtin_bit_cast(bf16x8_rt, m);
  t[2] = __builtin_bit_cast(bf16x8_rt, l);
}

// One 16-deep LDS slice ([k][64] fp32 for A and for B) through bf16 MFMAs:
// lane half h takes k = 8 h .. 8 h + 7 of column r and 32 + r of each operand.
template <bool A_BF16>
__device__ __forceinline__ void mc16_slice(f32x16_t (&acc)[2][2], const float (*As)[64],
                                           const float (*Bs)[64], int r, int h) {
  float va[2][8], vb[2][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int kk = 8 * h + i;
    va[0][i] = As[kk][r]; va[1][i] = As[kk][32 + r];
    vb[0][i] = Bs[kk][r]; vb[1][i] = Bs[kk][32 + r];
  }
  bf16x8_rt a[2][3], b[2][3];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    if (A_BF16) {  // bf16 values: exact in one term
      u32x4_rt u;
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = f32x2_to_bf16x2(va[mi][2 * i], va[mi][2 * i + 1]);
      a[mi][0] = __builtin_bit_cast(bf16x8_rt, u);
    } else {
      split3x8(va[mi], a[mi]);
    }
  }
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) split3x8(vb[ni], b[ni]);
  constexpr int NP = A_BF16 ? 3 : 6;
  constexpr int PA[6] = {0, 0, 1, 0, 2, 1};
  constexpr int PB[6] = {0, 1, 0, 2, 0, 1};
  constexpr int PA1[3] = {0, 0, 0};
  constexpr int PB1[3] = {0, 1, 2};
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            b[ni][A_BF16 ? PB1[q] : PB[q]], a[mi][A_BF16 ? PA1[q] : PA[q]], acc[mi][ni], 0, 0, 0);
}

// ---- router weight gradient: one wave per 64 x 64 output tile, LDS slices ----
// dW_r = x^T . d_logits contracts over tokens, and both operands are strided
// along it, so each wave stages its own 16-deep operand slices in its own
// 8 KiB of LDS as [k][64] (prefetching the next slice into registers while it
// computes, so the main loop has no workgroup barrier) and feeds the split
// bf16 products below from them: a wave owns a 64 x 64 tile as 2 x 2 MFMA
// blocks.  SK = 8: the workgroup's 8 waves split the contraction of one tile
// and add their partial sums through LDS in wave order (deterministic, no
// workspace); SK = 1: the 8 waves take 8 tiles.  Requires 16-byte aligned
// operands, the A and B contiguous extents multiples of 8 (bf16) or 4 (fp32)
// elements.
template <int AL, int BL>
__device__ __forceinline__ void router_load(RSlice& r, const void* A, int64_t lda, const float* B,
                                            int64_t ldb, int64_t m0, int64_t n0, int64_t k0,
                                            int64_t k_hi, int64_t M, int64_t N, int lane) {
  if (AL == RA_KC_BF16 || AL == RA_KC_F32) {
    // lane = row m0 + lane, k0 .. k0 + 15
    const int64_t m = m0 + lane;
    const bool row_ok = m < M;
    if (AL == RA_KC_BF16) {
      const bf16_t* p = static_cast<const bf16_t*>(A) + m * lda + k0;
      ld8_bf16(p, row_ok && k0 + 8 <= k_hi, r.a[0], r.a[1]);
      ld8_bf16(p + 8, row_ok && k0 + 16 <= k_hi, r.a[2], r.a[3]);
    } else {
      const float* p = static_cast<const float*>(A) + m * lda + k0;
#pragma unroll
      for (int j = 0; j < 4; ++j) r.a[j] = ld4_f32(p + 4 * j, row_ok && k0 + 4 * j + 4 <= k_hi);
    }
  } else {
    // lane -> k row k0 + (lane >> 2), rows m0 + 16 (lane & 3) .. + 15
    const int64_t k = k0 + (lane >> 2), m = m0 + 16 * (lane & 3);
    const bool k_ok = k < k_hi;
    if (AL == RA_MC_BF16) {
      const bf16_t* p = static_cast<const bf16_t*>(A) + k * lda + m;
      ld8_bf16(p, k_ok && m + 8 <= M, r.a[0], r.a[1]);
      ld8_bf16(p + 8, k_ok && m + 16 <= M, r.a[2], r.a[3]);
    } else {
      const float* p = static_cast<const float*>(A) + k * lda + m;
#pragma unroll
      for (int j = 0; j < 4; ++j) r.a[j] = ld4_f32(p + 4 * j, k_ok && m + 4 * j + 4 <= M);
    }
  }
  if (BL == RB_NC) {
    const int64_t k = k0 + (lane >> 2), n = n0 + 16 * (lane & 3);
    const float* p = B + k * ldb + n;
#pragma unroll
    for (int j = 0; j < 4; ++j) r.b[j] = ld4_f32(p + 4 * j, k < k_hi && n + 4 * j + 4 <= N);
  } else {
    const int64_t n = n0 + lane;
    const float* p = B + n * ldb + k0;
#pragma unroll
    for (int j = 0; j < 4; ++j) r.b[j] = ld4_f32(p + 4 * j, n < N && k0 + 4 * j + 4 <= k_hi);
  }
}

// slice -> LDS as [k][64] for A and for B
template <int AL, int BL>
__device__ __forceinline__ void router_stage(const RSlice& r, float (*As)[64], float (*Bs)[64],
                                             int lane) {
  if (AL == RA_KC_BF16 || AL == RA_KC_F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      As[4 * j + 0][lane] = r.a[j].x;
      As[4 * j + 1][lane] = r.a[j].y;
      As[4 * j + 2][lane] = r.a[j].z;
      As[4 * j + 3][lane] = r.a[j].w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(&As[lane >> 2][16 * (lane & 3) + 4 * j]) = r.a[j];
  }
  if (BL == RB_NC) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(&Bs[lane >> 2][16 * (lane & 3) + 4 * j]) = r.b[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Bs[4 * j + 0][lane] = r.b[j].x;
      Bs[4 * j + 1][lane] = r.b[j].y;
      Bs[4 * j + 2][lane] = r.b[j].z;
      Bs[4 * j + 3][lane] = r.b[j].w;
    }
  }
}

template <int AL, int BL, int SK, bool BIAS>
__global__ __launch_bounds__(512) void router_gemm_kernel(const void* __restrict__ A, int64_t lda,
                                                          const float* __restrict__ B,
                                                          int64_t ldb, float* __restrict__ C,
                                                          int64_t ldc, int64_t M, int64_t N,
                                                          int64_t K,
                                                          const float* __restrict__ bias) {
  __shared__ __attribute__((aligned(16))) float lds[8][2][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ntn = (N + 63) / 64;
  const int64_t tile = SK > 1 ? static_cast<int64_t>(blockIdx.x)
                              : static_cast<int64_t>(blockIdx.x) * 8 + wave;
  const int64_t m0 = (tile / ntn) * 64, n0 = (tile % ntn) * 64;
  int64_t k_lo = 0, k_hi = K;
  if (SK > 1) {
    const int64_t per = ((K + SK - 1) / SK + 15) / 16 * 16;
    k_lo = min(K, wave * per);
    k_hi = min(K, k_lo + per);
  }
  float(*As)[64] = lds[wave][0];
  float(*Bs)[64] = lds[wave][1];
  // MFMA 32x32x16 bf16, computed as D[n][m] so that lane r of a block holds
  // output row m = r: acc[mi][ni][v] is C[32 mi + r][32 ni + 8 (v / 4) +
  // 4 h + v % 4], h = lane / 32.  Lane half h feeds contraction positions
  // 8 h .. 8 h + 7 of each 16-deep slice, for A and for B alike.
  f32x16_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;
  const int r = lane & 31, h = lane >> 5;

  if (m0 < M) {  // SK == 1: trailing waves of the last block may have no tile
    RSlice rs;
    if (k_lo < k_hi) router_load<AL, BL>(rs, A, lda, B, ldb, m0, n0, k_lo, k_hi, M, N, lane);
    for (int64_t k0 = k_lo; k0 < k_hi; k0 += 16) {
      router_stage<AL, BL>(rs, As, Bs, lane);
      __builtin_amdgcn_wave_barrier();
      if (k0 + 16 < k_hi) router_load<AL, BL>(rs, A, lda, B, ldb, m0, n0, k0 + 16, k_hi, M, N, lane);
      mc16_slice<AL == RA_KC_BF16 || AL == RA_MC_BF16>(acc, As, Bs, r, h);
      __builtin_amdgcn_wave_barrier();
    }
  }

  // columns 32 ni + 8 g + 4 h .. + 3 of row 32 mi + r
  auto quad = [&](int mi, int ni, int g) {
    return make_float4(acc[mi][ni][4 * g], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2],
                       acc[mi][ni][4 * g + 3]);
  };
  if (SK == 1) {
    if (m0 >= M) return;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int64_t m = m0 + 32 * mi + r;
      if (m >= M) continue;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + 32 * ni + 8 * g + 4 * h;
          if (n >= N) continue;
          float4 v = quad(mi, ni, g);
          if (BIAS) {
            v.x += bias[n]; v.y += bias[n + 1]; v.z += bias[n + 2]; v.w += bias[n + 3];
          }
          *reinterpret_cast<float4*>(C + m * ldc + n) = v;
        }
    }
    return;
  }
  // SK > 1: two rounds of 32 rows; wave w's partials in its own 8 KiB as [32][64]
  float* part = &lds[wave][0][0][0];
#pragma unroll
  for (int rnd = 0; rnd < 2; ++rnd) {
    __syncthreads();  // every wave is done with its slices / the previous round
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(part + r * 64 + 32 * ni + 8 * g + 4 * h) = quad(rnd, ni, g);
    __syncthreads();
    // thread t sums elements 4t .. 4t+3 of the 32 x 64 half over the waves in order
    const int e = 4 * static_cast<int>(threadIdx.x);
    float4 sum = *reinterpret_cast<const float4*>(&lds[0][0][0][0] + e);
#pragma unroll
    for (int w = 1; w < 8; ++w) {
      const float4 q = *reinterpret_cast<const float4*>(&lds[w][0][0][0] + e);
      sum.x += q.x; sum.y += q.y; sum.z += q.z; sum.w += q.w;
    }
    const int64_t m = m0 + 32 * rnd + e / 64, n = n0 + (e % 64);
    if (m < M && n < N) {
      if (BIAS) {
        sum.x += bias[n]; sum.y += bias[n + 1]; sum.z += bias[n + 2]; sum.w += bias[n + 3];
      }
      *reinterpret_cast<float4*>(C + m * ldc + n) = sum;
    }
  }
}

template <int AL, int BL, int SK, bool BIAS>
static hipError_t run_router(const void* A, int64_t lda, const float* B, int64_t ldb, float* C,
                             int64_t ldc, int64_t M, int64_t N, int64_t K, const float* bias,
                             hipStream_t s) {
  const int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
  const int64_t blocks = SK > 1 ? tiles : (tiles + 7) / 8;
  if (blocks <= 0) return hipSuccess;
  router_gemm_kernel<AL, BL, SK, BIAS><<<dim3(static_cast<unsigned>(blocks)), 512, 0, s>>>(
      A, lda, B, ldb, C, ldc, M, N, K, bias);
  return hipGetLastError();
}

static bool aligned16p(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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

__device__ __forceinline__ float4 ld4g(const float* p, bool ok) {
  return ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
}

// One lane's raw operand values of one 16-deep step: for each of its two rows
// of A and two columns of B, the 8 values k = k0 .. k0 + 7 of its lane half.
struct RawAB {
  float4 a[2][2];  // fp32 A; a bf16 A keeps its 8 values in a[mi][0] as raw bits
  float b[2][8];
};

// A row m, k = k0 .. k0 + 7 (k0 a multiple of 8; k_hi a multiple of 8 for a
// bf16 A and of 4 for an fp32 A, so every vector lies wholly in or out)
template <bool AF32>
__device__ __forceinline__ void load_a_raw(const void* A, int64_t lda, int64_t m, int64_t M,
                                           int64_t k0, int64_t k_hi, float4 (&a)[2]) {
  const bool ok = m < M && k0 < k_hi;
  if (AF32) {
    const float* p = static_cast<const float*>(A) + m * lda + k0;
    a[0] = ld4g(p, ok);
    a[1] = ld4g(p + 4, ok && k0 + 8 <= k_hi);
  } else {
    const bf16_t* p = static_cast<const bf16_t*>(A) + m * lda + k0;
    const uint4 u = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
    a[0] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                       __uint_as_float(u.w));
  }
}

// B column n, k = k0 .. k0 + 7.  BT: B(k, n) = W[k * ldb + n]; else
// B(k, n) = W[n * ldb + k] (k_hi a multiple of 4)
template <bool BT>
__device__ __forceinline__ void load_b_raw(const float* W, int64_t ldb, int64_t n, int64_t N,
                                           int64_t k0, int64_t k_hi, float (&v)[8]) {
  if (BT) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[i] = (n < N && k0 + i < k_hi) ? W[(k0 + i) * ldb + n] : 0.f;
  } else {
    const bool ok = n < N && k0 < k_hi;
    const float* p = W + n * ldb + k0;
    const float4 u = ld4g(p, ok), w = ld4g(p + 4, ok && k0 + 8 <= k_hi);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    v[4] = w.x; v[5] = w.y; v[6] = w.z; v[7] = w.w;
  }
}

template <bool AF32>
__device__ __forceinline__ void split_a(const float4 (&a)[2], bf16x8_rt (&t)[3]) {
  if (AF32) {
    const float v[8] = {a[0].x, a[0].y, a[0].z, a[0].w, a[1].x, a[1].y, a[1].z, a[1].w};
    split3x8(v, t);
  } else {
    u32x4_rt u;
    u[0] = __float_as_uint(a[0].x); u[1] = __float_as_uint(a[0].y);
    u[2] = __float_as_uint(a[0].z); u[3] = __float_as_uint(a[0].w);
    t[0] = __builtin_bit_cast(bf16x8_rt, u);
  }
}

template <bool AF32, bool BT, int SK, bool BIAS>
__global__ __launch_bounds__(512) void router_mc_kernel(const void* __restrict__ A, int64_t lda,
                                                        const float* __restrict__ W, int64_t ldb,
                                                        float* __restrict__ C, int64_t ldc,
                                                        int64_t M, int64_t N, int64_t K,
                                                        const float* __restrict__ bias) {
  __shared__ __attribute__((aligned(16))) float part_lds[8][32][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ntn = (N + 63) / 64;
  const int64_t tile = SK > 1 ? static_cast<int64_t>(blockIdx.x)
                              : static_cast<int64_t>(blockIdx.x) * 8 + wave;
  const int64_t m0 = (tile / ntn) * 64, n0 = (tile % ntn) * 64;
  int64_t k_lo = 0, k_hi = K;
  if (SK > 1) {
    const int64_t per = ((K + SK - 1) / SK + 15) / 16 * 16;
    k_lo = min(K, wave * per);
    k_hi = min(K, k_lo + per);
  }
  // term pairs (A term, B term) in a fixed order: a split A keeps the six
  // pairs of weight 2^-16 or more, a bf16 A (one term) meets all three B terms
  constexpr int NP = AF32 ? 6 : 3;
  constexpr int PA[6] = {0, 0, 1, 0, 2, 1};
  constexpr int PB[6] = {0, 1, 0, 2, 0, 1};
  constexpr int PA1[3] = {0, 0, 0};
  constexpr int PB1[3] = {0, 1, 2};
  f32x16_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;
  const int r = lane & 31, h = lane >> 5;

  if (m0 < M) {  // SK == 1: trailing waves of the last block may have no tile
    // the raw values of the next two steps are in flight while one computes
    RawAB raw[2];
    auto load_raw = [&](int64_t k0, RawAB& rw) {
      const int64_t kk = k0 + 8 * h;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) load_a_raw<AF32>(A, lda, m0 + 32 * mi + r, M, kk, k_hi, rw.a[mi]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) load_b_raw<BT>(W, ldb, n0 + 32 * ni + r, N, kk, k_hi, rw.b[ni]);
    };
    if (k_lo < k_hi) load_raw(k_lo, raw[0]);
    if (k_lo + 16 < k_hi) load_raw(k_lo + 16, raw[1]);
    for (int64_t k0 = k_lo; k0 < k_hi; k0 += 32) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int64_t ks = k0 + 16 * sub;
        if (ks >= k_hi) break;
        bf16x8_rt a[2][3], b[2][3];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) split_a<AF32>(raw[sub].a[mi], a[mi]);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) split3x8(raw[sub].b[ni], b[ni]);
        if (ks + 32 < k_hi) load_raw(ks + 32, raw[sub]);
#pragma unroll
        for (int q = 0; q < NP; ++q)
#pragma unroll
          for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  b[ni][AF32 ? PB[q] : PB1[q]], a[mi][AF32 ? PA[q] : PA1[q]], acc[mi][ni], 0, 0,
                  0);
      }
    }
  }

  // columns 32 ni + 8 g + 4 h .. + 3 of row 32 mi + r
  auto quad = [&](int mi, int ni, int g) {
    return make_float4(acc[mi][ni][4 * g], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2],
                       acc[mi][ni][4 * g + 3]);
  };
  if (SK == 1) {
    if (m0 >= M) return;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int64_t m = m0 + 32 * mi + r;
      if (m >= M) continue;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + 32 * ni + 8 * g + 4 * h;
          if (n >= N) continue;
          float4 v = quad(mi, ni, g);
          if (BIAS) {
            v.x += bias[n]; v.y += bias[n + 1]; v.z += bias[n + 2]; v.w += bias[n + 3];
          }
          *reinterpret_cast<float4*>(C + m * ldc + n) = v;
        }
    }
    return;
  }
  // SK > 1: two rounds of 32 rows; wave w's partials in its own 8 KiB as [32][64]
  float* part = &part_lds[wave][0][0];
#pragma unroll
  for (int rnd = 0; rnd < 2; ++rnd) {
    __syncthreads();
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(part + r * 64 + 32 * ni + 8 * g + 4 * h) = quad(rnd, ni, g);
    __syncthreads();
    // thread t sums elements 4t .. 4t+3 of the 32 x 64 half over the waves in order
    const int e = 4 * static_cast<int>(threadIdx.x);
    float4 sum = *reinterpret_cast<const float4*>(&part_lds[0][0][0] + e);
#pragma unroll
    for (int w = 1; w < 8; ++w) {
      const float4 q = *reinterpret_cast<const float4*>(&part_lds[w][0][0] + e);
      sum.x += q.x; sum.y += q.y; sum.z += q.z; sum.w += q.w;
    }
    const int64_t m = m0 + 32 * rnd + e / 64, n = n0 + (e % 64);
    if (m < M && n < N) {
      if (BIAS) {
        sum.x += bias[n]; sum.y += bias[n + 1]; sum.z += bias[n + 2]; sum.w += bias[n + 3];
      }
      *reinterpret_cast<float4*>(C + m * ldc + n) = sum;
    }
  }
}

template <bool AF32, bool BT, int SK, bool BIAS>
static hipError_t run_router_mc(const void* A, int64_t lda, const float* W, int64_t ldb, float* C,
                                int64_t ldc, int64_t M, int64_t N, int64_t K, const float* bias,
                                hipStream_t s) {
  const int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
  const int64_t blocks = SK > 1 ? tiles : (tiles + 7) / 8;
  if (blocks <= 0) return hipSuccess;
  router_mc_kernel<AF32, BT, SK, BIAS><<<dim3(static_cast<unsigned>(blocks)), 512, 0, s>>>(
      A, lda, W, ldb, C, ldc, M, N, K, bias);
  return hipGetLastError();
}

hipError_t launch_router_fwd(const void* x, int x_dtype, const float* w_r, const float* bias,
                             int64_t T, int64_t d, int E, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (d % 8 == 0 && E % 4 == 0 && aligned16p(x) && aligned16p(w_r) && aligned16p(logits)) {
    // logits [T, E] = x [T, d] . W_r [d, E] (+ bias): contraction split over the 8 waves
    if (x_dtype == 0)
      return bias ? run_router_mc<true, true, 8, true>(x, d, w_r, E, logits, E, T, E, d, bias, s)
                  : run_router_mc<true, true, 8, false>(x, d, w_r, E, logits, E, T, E, d, bias, s);
    return bias ? run_router_mc<false, true, 8, true>(x, d, w_r, E, logits, E, T, E, d, bias, s)
                : run_router_mc<false, true, 8, false>(x, d, w_r, E, logits, E, T, E, d, bias, s);
  }
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
  const bool fast = d % 8 == 0 && E % 4 == 0 && aligned16p(x) && aligned16p(w_r) &&
                    aligned16p(dz) && aligned16p(dw_r) && aligned16p(dx_r);
  if (fast) {
    if (dw_r) {
      // dW_r [d, E] = x^T [d, T] . dz [T, E]: contraction over tokens split over the 8 waves
      if (T == 0)
        err = launch_fill_zero(dw_r, d * E, s);
      else if (x_dtype == 0)
        err = run_router<RA_MC_F32, RB_NC, 8, false>(x, d, dz, E, dw_r, E, d, E, T, nullptr, s);
      else
        err = run_router<RA_MC_BF16, RB_NC, 8, false>(x, d, dz, E, dw_r, E, d, E, T, nullptr, s);
      if (err != hipSuccess) return err;
    }
    if (dx_r && T > 0)
      // dx_r [T, d] = dz [T, E] . W_r^T (Bop(k = e, n = i) = W_r[i * E + e])
      err = run_router_mc<true, false, 1, false>(dz, E, w_r, E, dx_r, d, T, d, E, nullptr, s);
    return err;
  }
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
