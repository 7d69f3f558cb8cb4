// fp32 GEMM family on the vector ALUs: the router projection and its backward
// (the router stays in FP32 -- "Scalable Training of Mixture-of-Experts Models
// with Megatron Core", section 5, Selective precision) and the fp32 grouped
// expert GEMMs (section 2, Expert Computation).
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


// ---- router products on the fp32 vector ALUs --------------------------------
// The router stays in FP32 (section 5, Selective precision): x . W_r, its
// weight gradient x^T . d_logits and the router's input gradient
// d_logits . W_r^T are fp32 multiply-adds on the vector ALUs; the matrix
// cores serve the expert contractions only.
//
//   C[m, n] = sum_k Aop(m, k) Bop(k, n) (+ bias[n], one fp32 addition after the sum)
//   Aop(m, k) = A[m lda + k]  (AL = RA_KC_*: k contiguous; x or d_logits)
//             = A[k lda + m]  (AL = RA_MC_*: m contiguous; x read as x^T)
//   Bop(k, n) = B[k ldb + n]  (BL = RB_NC: W_r, or d_logits for dW_r)
//             = B[n ldb + k]  (BL = RB_KC: W_r read as W_r^T)
//
// A BM x BN output tile per workgroup of KS x 256 threads.  In each group of
// 256, thread (tx, ty) owns TM x TN outputs: rows ty*4 .. +3 (and BM/2 +
// ty*4 .. +3 when TM = 8), columns tx*4 .. +3 (and BN/2 + tx*4 .. +3 when
// TN = 8), so that every LDS fragment read is one 16-byte vector, the lanes
// of a wave read neighbouring B vectors and share their A vectors.  Operands
// are staged as [k][m] and [k][n] fp32, each group in its own two LDS
// buffers: the next BK-deep slice is loaded into registers while the current
// one is consumed, one barrier per slice.  The KS groups take every KS-th
// slice and their partial tiles are added through LDS in group order at the
// end.  Every output is thus a sum in a fixed order (deterministic), taken in
// levels (per slice, per group, then over the groups) so that its rounding
// error grows with BK + K/(BK KS) + KS rather than K.
enum { RA_KC_BF16 = 0, RA_KC_F32 = 1, RA_MC_BF16 = 2, RA_MC_F32 = 3 };
enum { RB_NC = 0, RB_KC = 1 };

template <int AL> struct RouterA {
  static constexpr bool BF16 = AL == RA_KC_BF16 || AL == RA_MC_BF16;
  static constexpr bool MC = AL == RA_MC_BF16 || AL == RA_MC_F32;
  static constexpr int VEC = BF16 ? 8 : 4;  // elements per 16-byte load
};

template <int BM, int BN, int BK, int TM, int TN, int AL>
struct RouterTile {
  static constexpr int NX = BN / TN, NY = BM / TM;
  static_assert(NX * NY == 256, "256 threads per group");
  static_assert((TM == 4 || TM == 8) && (TN == 4 || TN == 8), "4 or 8 rows / columns per thread");
  static constexpr int AV = RouterA<AL>::VEC;
  static constexpr int A_VECS = BM * BK / AV;               // 16-byte vectors of the A slice
  static constexpr int B_VECS = BN * BK / 4;                // of the B slice
  static constexpr int A_PER = (A_VECS + 255) / 256;
  static constexpr int B_PER = (B_VECS + 255) / 256;
};

template <int A_PER, int B_PER>
struct RouterRegs {
  uint4 a[A_PER];
  float4 b[B_PER];
};

template <int BM, int BN, int BK, int TM, int TN, int AL, int BL, typename R>
__device__ __forceinline__ void router_fetch(R& r, const void* A, int64_t lda, const float* B,
                                             int64_t ldb, int64_t m0, int64_t n0, int64_t k0,
                                             int64_t M, int64_t N, int64_t K, int tid) {
  using TL = RouterTile<BM, BN, BK, TM, TN, AL>;
  constexpr int AV = TL::AV;
#pragma unroll
  for (int i = 0; i < TL::A_PER; ++i) {
    const int v = tid + 256 * i;
    r.a[i] = make_uint4(0u, 0u, 0u, 0u);
    if (v >= TL::A_VECS) continue;
    int64_t m, k;
    if (RouterA<AL>::MC) {  // vectors along m: [k][m / AV]
      m = m0 + (v % (BM / AV)) * AV;
      k = k0 + v / (BM / AV);
      if (m + AV > M || k >= K) continue;
    } else {                // vectors along k: [m][k / AV]
      m = m0 + v / (BK / AV);
      k = k0 + (v % (BK / AV)) * AV;
      if (m >= M || k + AV > K) continue;
    }
    const int64_t e = RouterA<AL>::MC ? k * lda + m : m * lda + k;
    r.a[i] = RouterA<AL>::BF16 ? *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(A) + e)
                               : *reinterpret_cast<const uint4*>(static_cast<const float*>(A) + e);
  }
#pragma unroll
  for (int i = 0; i < TL::B_PER; ++i) {
    const int v = tid + 256 * i;
    r.b[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (v >= TL::B_VECS) continue;
    if (BL == RB_NC) {  // vectors along n: [k][n / 4]
      const int64_t n = n0 + (v % (BN / 4)) * 4, k = k0 + v / (BN / 4);
      if (n + 4 > N || k >= K) continue;
      r.b[i] = *reinterpret_cast<const float4*>(B + k * ldb + n);
    } else {            // vectors along k: [n][k / 4]
      const int64_t n = n0 + v / (BK / 4), k = k0 + (v % (BK / 4)) * 4;
      if (n >= N || k + 4 > K) continue;
      r.b[i] = *reinterpret_cast<const float4*>(B + n * ldb + k);
    }
  }
}

__device__ __forceinline__ void unpack_vec(const uint4& u, bool bf16, float (&v)[8]) {
  if (bf16) {
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
    v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xffff0000u);
    v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xffff0000u);
  } else {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
}

template <int BM, int BN, int BK, int TM, int TN, int AL, int BL, typename R>
__device__ __forceinline__ void router_stage(const R& r, float (*As)[BM], float (*Bs)[BN], int tid) {
  using TL = RouterTile<BM, BN, BK, TM, TN, AL>;
  constexpr int AV = TL::AV;
#pragma unroll
  for (int i = 0; i < TL::A_PER; ++i) {
    const int v = tid + 256 * i;
    if (v >= TL::A_VECS) continue;
    float e[8];
    unpack_vec(r.a[i], RouterA<AL>::BF16, e);
    if (RouterA<AL>::MC) {
      const int m = (v % (BM / AV)) * AV, k = v / (BM / AV);
#pragma unroll
      for (int j = 0; j < AV; j += 4)
        *reinterpret_cast<float4*>(&As[k][m + j]) = make_float4(e[j], e[j + 1], e[j + 2], e[j + 3]);
    } else {
      const int m = v / (BK / AV), k = (v % (BK / AV)) * AV;
#pragma unroll
      for (int j = 0; j < AV; ++j) As[k + j][m] = e[j];
    }
  }
#pragma unroll
  for (int i = 0; i < TL::B_PER; ++i) {
    const int v = tid + 256 * i;
    if (v >= TL::B_VECS) continue;
    if (BL == RB_NC) {
      const int n = (v % (BN / 4)) * 4, k = v / (BN / 4);
      *reinterpret_cast<float4*>(&Bs[k][n]) = r.b[i];
    } else {
      const int n = v / (BK / 4), k = (v % (BK / 4)) * 4;
      Bs[k][n] = r.b[i].x; Bs[k + 1][n] = r.b[i].y; Bs[k + 2][n] = r.b[i].z; Bs[k + 3][n] = r.b[i].w;
    }
  }
}

template <int BM, int BN, int BK, int TM, int TN, int KS, int AL, int BL, bool BIAS>
__global__ __launch_bounds__(256 * KS) void router_valu_kernel(
    const void* __restrict__ A, int64_t lda, const float* __restrict__ B, int64_t ldb,
    float* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t K,
    const float* __restrict__ bias) {
  using TL = RouterTile<BM, BN, BK, TM, TN, AL>;
  // per group: two [BK][BM] A buffers, then two [BK][BN] B buffers; after the
  // last slice the same region holds the group's partial [BM][BN] tile
  constexpr int REGION = 2 * BK * (BM + BN);
  static_assert(KS == 1 || REGION >= BM * BN, "room for a group's partial tile");
  __shared__ __attribute__((aligned(16))) float lds[KS * REGION];
  const int grp = static_cast<int>(threadIdx.x) / 256, tid = static_cast<int>(threadIdx.x) % 256;
  float* region = lds + grp * REGION;
  auto a_buf = [&](int b) { return reinterpret_cast<float(*)[BM]>(region + b * BK * BM); };
  auto b_buf = [&](int b) {
    return reinterpret_cast<float(*)[BN]>(region + 2 * BK * BM + b * BK * BN);
  };
  const int tx = tid % TL::NX, ty = tid / TL::NX;
  const int64_t ntn = (N + BN - 1) / BN;
  const int64_t m0 = (static_cast<int64_t>(blockIdx.x) / ntn) * BM;
  const int64_t n0 = (static_cast<int64_t>(blockIdx.x) % ntn) * BN;

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

  // group grp takes slices grp, grp + KS, ...; every group runs the same count
  const int64_t nslices = (K + BK - 1) / BK;
  const int64_t nsteps = (nslices + KS - 1) / KS;
  RouterRegs<TL::A_PER, TL::B_PER> regs;
  if (nsteps > 0) {
    router_fetch<BM, BN, BK, TM, TN, AL, BL>(regs, A, lda, B, ldb, m0, n0,
                                             static_cast<int64_t>(grp) * BK, M, N, K, tid);
    router_stage<BM, BN, BK, TM, TN, AL, BL>(regs, a_buf(0), b_buf(0), tid);
  }
  __syncthreads();
  for (int64_t s = 0; s < nsteps; ++s) {
    const int buf = static_cast<int>(s & 1);
    const int64_t knext = ((s + 1) * KS + grp) * BK;
    if (s + 1 < nsteps)
      router_fetch<BM, BN, BK, TM, TN, AL, BL>(regs, A, lda, B, ldb, m0, n0, knext, M, N, K, tid);
    float part[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) part[i][j] = 0.f;
    const float(*as)[BM] = a_buf(buf);
    const float(*bs)[BN] = b_buf(buf);
#pragma unroll 4
    for (int kk = 0; kk < BK; ++kk) {
      float a[TM], b[TN];
      const float4 a0 = *reinterpret_cast<const float4*>(&as[kk][ty * 4]);
      a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w;
      if (TM == 8) {
        const float4 a1 = *reinterpret_cast<const float4*>(&as[kk][BM / 2 + ty * 4]);
        a[TM - 4] = a1.x; a[TM - 3] = a1.y; a[TM - 2] = a1.z; a[TM - 1] = a1.w;
      }
      const float4 b0 = *reinterpret_cast<const float4*>(&bs[kk][tx * 4]);
      b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w;
      if (TN == 8) {
        const float4 b1 = *reinterpret_cast<const float4*>(&bs[kk][BN / 2 + tx * 4]);
        b[TN - 4] = b1.x; b[TN - 3] = b1.y; b[TN - 2] = b1.z; b[TN - 1] = b1.w;
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) part[i][j] = fmaf(a[i], b[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] += part[i][j];
    if (s + 1 < nsteps)
      router_stage<BM, BN, BK, TM, TN, AL, BL>(regs, a_buf(buf ^ 1), b_buf(buf ^ 1), tid);
    __syncthreads();
  }

  auto row_of = [&](int i) { return i < 4 ? ty * 4 + i : BM / 2 + ty * 4 + (i - 4); };
  auto col_of = [&](int h) { return h == 0 ? tx * 4 : BN / 2 + tx * 4; };
  if (KS > 1) {
    // groups 1 .. KS-1 leave their partial tiles in their own LDS (the slices
    // are all consumed: the loop ended on a barrier); group 0 adds them in order
    float* mine = region;
    if (grp > 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int h = 0; h < TN / 4; ++h)
          *reinterpret_cast<float4*>(mine + row_of(i) * BN + col_of(h)) =
              make_float4(acc[i][4 * h], acc[i][4 * h + 1], acc[i][4 * h + 2], acc[i][4 * h + 3]);
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < KS; ++g) {
      const float* theirs = lds + g * REGION;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int h = 0; h < TN / 4; ++h) {
          const float4 q = *reinterpret_cast<const float4*>(theirs + row_of(i) * BN + col_of(h));
          acc[i][4 * h] += q.x; acc[i][4 * h + 1] += q.y;
          acc[i][4 * h + 2] += q.z; acc[i][4 * h + 3] += q.w;
        }
    }
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + row_of(i);
    if (m >= M) continue;
#pragma unroll
    for (int h = 0; h < TN / 4; ++h) {
      const int64_t n = n0 + col_of(h);
      if (n + 4 > N) continue;
      float4 v = make_float4(acc[i][4 * h], acc[i][4 * h + 1], acc[i][4 * h + 2], acc[i][4 * h + 3]);
      if (BIAS) {
        v.x += bias[n]; v.y += bias[n + 1]; v.z += bias[n + 2]; v.w += bias[n + 3];
      }
      *reinterpret_cast<float4*>(C + m * ldc + n) = v;
    }
  }
}

template <int BM, int BN, int BK, int TM, int TN, int KS, int AL, int BL, bool BIAS>
static hipError_t run_router_valu(const void* A, int64_t lda, const float* B, int64_t ldb,
                                  float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                  const float* bias, hipStream_t s) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles <= 0) return hipSuccess;
  router_valu_kernel<BM, BN, BK, TM, TN, KS, AL, BL, BIAS>
      <<<dim3(static_cast<unsigned>(tiles)), 256 * KS, 0, s>>>(A, lda, B, ldb, C, ldc, M, N, K,
                                                               bias);
  return hipGetLastError();
}

// Products whose output width is the expert count E (logits, dW_r): the tile
// spans up to 256 experts (256 / 128 / 64 columns by E), two groups of 256
// threads split the contraction (eight waves per CU).  Measured on the
// DeepSeek-V3 layer's router (T = 8192, d = 7168, E = 256): logits 0.77 ->
// 0.46 ms with two groups and 8 x 4 outputs per thread; dW_r 0.86 -> 0.51 ms
// with two groups and 4 x 8.
template <int TM, int TN, int AL, int BL, bool BIAS>
static hipError_t run_router_e(const void* A, int64_t lda, const float* B, int64_t ldb, float* C,
                               int64_t ldc, int64_t M, int64_t N, int64_t K, const float* bias,
                               hipStream_t s) {
  // 256 threads per group: BN / TN across the columns, so BM = TM * TN * 256 / BN rows
  if (N > 128)
    return run_router_valu<TM * TN, 256, 32, TM, TN, 2, AL, BL, BIAS>(A, lda, B, ldb, C, ldc, M, N,
                                                                      K, bias, s);
  if (N > 64)
    return run_router_valu<TM * TN * 2, 128, 32, TM, TN, 2, AL, BL, BIAS>(A, lda, B, ldb, C, ldc,
                                                                          M, N, K, bias, s);
  return run_router_valu<TM * TN * 4, 64, 32, TM, TN, 2, AL, BL, BIAS>(A, lda, B, ldb, C, ldc, M,
                                                                       N, K, bias, s);
}

// Logits for few experts (E <= 32, E % 4 == 0): a tile as wide as 64 experts
// would leave most columns empty and the launch a few dozen workgroups.  Here
// a workgroup takes 8 rows; 8 lanes of a wave share a row, and the 4 waves
// split the row's 16-byte pieces: lane slice s of wave w reads the pieces
// k = 8 s + 64 (w + 4 i) (8 consecutive x values), so that the 8 lanes of a
// row read 128 contiguous bytes and every W_r value fetched from cache serves
// 8 rows.  Each piece's 8 products per expert are summed and added to the
// lane's running sum; the 8 lanes of a row are added in a fixed tree and the
// 4 waves' sums in wave order: the result does not depend on scheduling.
template <int EP, bool XF32, bool BIAS>
__global__ __launch_bounds__(256) void router_narrow_kernel(const void* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ out, int64_t T,
                                                            int64_t d, int E) {
  __shared__ float part_w[3][8][EP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 3, sl = lane & 7;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 8 + r;
  const bool ok = row < T;
  const int64_t xr = ok ? row : 0;
  float acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.f;
#pragma unroll 2
  for (int64_t k0 = sl * 8 + 64 * wave; k0 < d; k0 += 256) {
    float xv[8];
    if (XF32) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + xr * d + k0);
      const float4 a = p[0], b = p[1];
      xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
      xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(x) + xr * d + k0);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[2 * i] = __uint_as_float(u[i] << 16);
        xv[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    }
    float part[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) part[e] = 0.f;
    // the piece's W_r rows are fetched before any is used (half of them at a
    // time for 32 expert slots), so that the loads are in flight together;
    // slots past E repeat the last four experts (in bounds, no branch between
    // the loads) and their sums are never stored
    constexpr int RH = EP > 16 ? 4 : 8;  // W_r rows per batch
#pragma unroll
    for (int i0 = 0; i0 < 8; i0 += RH) {
      float4 q[RH][EP / 4];
#pragma unroll
      for (int i = 0; i < RH; ++i)
#pragma unroll
        for (int e = 0; e < EP; e += 4)
          q[i][e / 4] = *reinterpret_cast<const float4*>(w + (k0 + i0 + i) * E + min(e, E - 4));
#pragma unroll
      for (int i = 0; i < RH; ++i)
#pragma unroll
        for (int e = 0; e < EP; e += 4) {
          const float xi = xv[i0 + i];
          part[e] = fmaf(xi, q[i][e / 4].x, part[e]);
          part[e + 1] = fmaf(xi, q[i][e / 4].y, part[e + 1]);
          part[e + 2] = fmaf(xi, q[i][e / 4].z, part[e + 2]);
          part[e + 3] = fmaf(xi, q[i][e / 4].w, part[e + 3]);
        }
    }
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] += part[e];
  }
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    float v = acc[e];
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    acc[e] = v;
  }
  if (wave > 0 && sl == 0) {
#pragma unroll
    for (int e = 0; e < EP; ++e) part_w[wave - 1][r][e] = acc[e];
  }
  __syncthreads();
  if (wave != 0 || !ok || sl != 0) return;
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] += part_w[q][r][e];
#pragma unroll
  for (int e = 0; e < EP; e += 4) {
    if (e < E) {
      float4 v = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
      if (BIAS) {
        v.x += bias[e]; v.y += bias[e + 1]; v.z += bias[e + 2]; v.w += bias[e + 3];
      }
      *reinterpret_cast<float4*>(out + row * E + e) = v;
    }
  }
}

template <int EP, bool XF32>
static hipError_t run_router_narrow(const void* x, const float* w, const float* bias, float* out,
                                    int64_t T, int64_t d, int E, hipStream_t s) {
  const int64_t blocks = (T + 7) / 8;
  if (bias)
    router_narrow_kernel<EP, XF32, true><<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(
        x, w, bias, out, T, d, E);
  else
    router_narrow_kernel<EP, XF32, false><<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(
        x, w, bias, out, T, d, E);
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

hipError_t launch_router_fwd(const void* x, int x_dtype, const float* w_r, const float* bias,
                             int64_t T, int64_t d, int E, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (d % 8 == 0 && E % 4 == 0 && aligned16p(x) && aligned16p(w_r) && aligned16p(logits)) {
    // logits [T, E] = x [T, d] . W_r [d, E] (+ bias)
    if (E <= 32) {
      if (E <= 8)
        return x_dtype == 0 ? run_router_narrow<8, true>(x, w_r, bias, logits, T, d, E, s)
                            : run_router_narrow<8, false>(x, w_r, bias, logits, T, d, E, s);
      if (E <= 16)
        return x_dtype == 0 ? run_router_narrow<16, true>(x, w_r, bias, logits, T, d, E, s)
                            : run_router_narrow<16, false>(x, w_r, bias, logits, T, d, E, s);
      return x_dtype == 0 ? run_router_narrow<32, true>(x, w_r, bias, logits, T, d, E, s)
                          : run_router_narrow<32, false>(x, w_r, bias, logits, T, d, E, s);
    }
    if (x_dtype == 0)
      return bias ? run_router_e<8, 4, RA_KC_F32, RB_NC, true>(x, d, w_r, E, logits, E, T, E, d,
                                                               bias, s)
                  : run_router_e<8, 4, RA_KC_F32, RB_NC, false>(x, d, w_r, E, logits, E, T, E, d,
                                                                bias, s);
    return bias ? run_router_e<8, 4, RA_KC_BF16, RB_NC, true>(x, d, w_r, E, logits, E, T, E, d,
                                                              bias, s)
                : run_router_e<8, 4, RA_KC_BF16, RB_NC, false>(x, d, w_r, E, logits, E, T, E, d,
                                                               bias, s);
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
      // dW_r [d, E] = x^T [d, T] . dz [T, E]
      if (T == 0)
        err = launch_fill_zero(dw_r, d * E, s);
      else if (x_dtype == 0)
        err = run_router_e<4, 8, RA_MC_F32, RB_NC, false>(x, d, dz, E, dw_r, E, d, E, T, nullptr,
                                                          s);
      else
        err = run_router_e<4, 8, RA_MC_BF16, RB_NC, false>(x, d, dz, E, dw_r, E, d, E, T, nullptr,
                                                           s);
      if (err != hipSuccess) return err;
    }
    if (dx_r && T > 0)
      // dx_r [T, d] = dz [T, E] . W_r^T (Bop(k = e, n = i) = W_r[i * E + e])
      // (16-deep slices: 0.466 -> 0.456 ms on the DeepSeek-V3 layer's router)
      err = run_router_valu<128, 128, 16, 8, 8, 1, RA_KC_F32, RB_KC, false>(
          dz, E, w_r, E, dx_r, d, T, d, E, nullptr, s);
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

// ---- router backward when d_logits lives on each token's chosen experts ------
// With renormalised or sigmoid routing (and no auxiliary loss) the route's
// backward leaves d_logits zero outside each token's k chosen experts, so the
// two products need only those entries: T k d multiply-adds each instead of
// T E d, still fp32 on the vector ALUs and summed in a fixed order.

// dx_router[t, i] = sum_j d_logits[t, e_j] * W_r[i, e_j], slots in order.
// Block: 64 columns i0 .. i0+63 (lane = column) x a chunk of tokens, 16
// waves, wave w taking every 16th token.  W_r's 64 rows are staged in LDS as
// [64][E + 1] so that lanes reading one expert's column hit distinct banks.
// A wave fetches the experts and key gradients of 64 / k tokens at once (lane
// = token, slot) and broadcasts them with shuffles, the next batch already in
// flight, so the dependent index -> gradient loads are not paid per slot;
// (token, slot) is uniform over the wave, so the broadcasts are lane reads
// into scalar registers and only the W_r reads use the LDS.
constexpr int kDxCols = 64, kDxTokens = 1024, kDxWaves = 16;
__global__ __launch_bounds__(1024) void router_dx_topk_kernel(const float* __restrict__ w_r,
                                                              const float* __restrict__ dz,
                                                              const int32_t* __restrict__ topk_idx,
                                                              int64_t T, int64_t d, int E, int k,
                                                              float* __restrict__ dx) {
  __shared__ float wl[kDxCols * 257];  // [kDxCols][E + 1], E <= 256
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kDxCols;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kDxTokens;
  const int cols = static_cast<int>(min<int64_t>(kDxCols, d - i0));
  for (int q = threadIdx.x; q < cols * E; q += 64 * kDxWaves) {
    const int r = q / E, e = q - r * E;
    wl[r * (E + 1) + e] = w_r[(i0 + r) * E + e];
  }
  __syncthreads();
  const int64_t t1 = min<int64_t>(T, t0 + kDxTokens);
  const int nb = 64 / k;                      // tokens per batch
  const int u = lane / k, j = lane - u * k;   // this lane's (token, slot) of a batch
  auto fetch = [&](int64_t tb, int& e, float& g) {
    const int64_t t = tb + static_cast<int64_t>(u) * kDxWaves;
    e = -1;
    g = 0.f;
    if (u < nb && t < t1) {
      const int ee = topk_idx[t * k + j];
      if (ee >= 0 && ee < E) {
        e = ee;
        g = dz[t * E + ee];
      }
    }
  };
  int e_cur, e_nxt;
  float g_cur, g_nxt;
  int64_t tb = t0 + wave;
  if (tb < t1) fetch(tb, e_cur, g_cur);
  for (; tb < t1; tb += static_cast<int64_t>(nb) * kDxWaves) {
    const int64_t tn = tb + static_cast<int64_t>(nb) * kDxWaves;
    if (tn < t1) fetch(tn, e_nxt, g_nxt);
    for (int uu = 0; uu < nb; ++uu) {
      const int64_t t = tb + static_cast<int64_t>(uu) * kDxWaves;
      if (t >= t1) break;
      float acc = 0.f;
      for (int jj = 0; jj < k; ++jj) {
        const int e = __builtin_amdgcn_readlane(e_cur, uu * k + jj);
        const float g = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g_cur), uu * k + jj));
        if (e >= 0 && lane < cols) acc = fmaf(g, wl[lane * (E + 1) + e], acc);
      }
      if (lane < cols) dx[t * d + i0 + lane] = acc;
    }
    e_cur = e_nxt;
    g_cur = g_nxt;
  }
}

// dW_r[i, e] = sum over expert e's rows r (ascending) of x[src_token[r], i] *
// d_logits[src_token[r], e].  Block: expert e x 64 VN columns (VN per lane,
// one 16-byte load), 16 waves, wave w taking every 16th row of the segment.
// A wave gathers the tokens and key gradients of its next 64 rows at once
// (lane = row), then keeps 8 rows' x loads in flight; the 16 waves' sums are
// added through LDS in wave order.
constexpr int kDwWaves = 16;
template <int VN>
__global__ __launch_bounds__(1024) void router_dw_topk_kernel(const void* __restrict__ x,
                                                              const float* __restrict__ dz,
                                                              const int64_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ src_token,
                                                              int64_t T, int64_t d, int E,
                                                              int64_t n_rows,
                                                              float* __restrict__ dw) {
  __shared__ float part[kDwWaves - 1][64 * VN];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.y;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64 * VN + lane * VN;
  const bool col_ok = c0 + VN <= d;
  int64_t lo = offsets[e], hi = offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > n_rows ? n_rows : lo);
  hi = hi < lo ? lo : (hi > n_rows ? n_rows : hi);
  float acc[VN];
#pragma unroll
  for (int v = 0; v < VN; ++v) acc[v] = 0.f;
  constexpr int UNR = 8;
  for (int64_t rb = lo + wave; rb < hi; rb += 64 * kDwWaves) {
    // this wave's next 64 rows: rb, rb + 16, ...; lane l gathers row rb + 16 l
    const int64_t rl = rb + static_cast<int64_t>(lane) * kDwWaves;
    int tok = -1;
    float gl = 0.f;
    if (rl < hi) {
      const int32_t t = src_token[rl];
      if (t >= 0 && t < T) {
        tok = t;
        gl = dz[static_cast<int64_t>(t) * E + e];
      }
    }
    const int cnt = static_cast<int>(min<int64_t>(64, (hi - rb + kDwWaves - 1) / kDwWaves));
    for (int u0 = 0; u0 < cnt; u0 += UNR) {
      uint4 raw[UNR];
      float g[UNR];
#pragma unroll
      for (int uu = 0; uu < UNR; ++uu) {
        const int t = __builtin_amdgcn_readlane(tok, (u0 + uu) & 63);
        g[uu] = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gl), (u0 + uu) & 63));
        raw[uu] = make_uint4(0u, 0u, 0u, 0u);
        if (u0 + uu < cnt && t >= 0 && col_ok)
          raw[uu] = VN == 8
                        ? *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(x) +
                                                          static_cast<int64_t>(t) * d + c0)
                        : *reinterpret_cast<const uint4*>(static_cast<const float*>(x) +
                                                          static_cast<int64_t>(t) * d + c0);
        if (!(u0 + uu < cnt && t >= 0)) g[uu] = 0.f;
      }
#pragma unroll
      for (int uu = 0; uu < UNR; ++uu) {
        float v[8];
        unpack_vec(raw[uu], VN == 8, v);
#pragma unroll
        for (int q = 0; q < VN; ++q) acc[q] = fmaf(v[q], g[uu], acc[q]);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int q = 0; q < VN; ++q) part[wave - 1][lane * VN + q] = acc[q];
  }
  __syncthreads();
  if (wave != 0 || !col_ok) return;
  for (int w = 0; w < kDwWaves - 1; ++w)
#pragma unroll
    for (int q = 0; q < VN; ++q) acc[q] += part[w][lane * VN + q];
#pragma unroll
  for (int q = 0; q < VN; ++q) dw[(c0 + q) * E + e] = acc[q];
}

hipError_t launch_router_bwd_topk(const void* x, int x_dtype, const float* w_r, const float* dz,
                                  const int32_t* topk_idx, const int64_t* offsets,
                                  const int32_t* src_token, int64_t T, int64_t d, int E, int k,
                                  float* dw_r, float* dx_r, hipStream_t s) {
  if (dw_r) {
    if (T == 0) {
      hipError_t err = launch_fill_zero(dw_r, d * E, s);
      if (err != hipSuccess) return err;
    } else {
      const int vn = x_dtype == 0 ? 4 : 8;
      const dim3 g(static_cast<unsigned>((d + 64 * vn - 1) / (64 * vn)), static_cast<unsigned>(E));
      if (x_dtype == 0)
        router_dw_topk_kernel<4><<<g, 64 * kDwWaves, 0, s>>>(x, dz, offsets, src_token, T, d, E,
                                                             T * k, dw_r);
      else
        router_dw_topk_kernel<8><<<g, 64 * kDwWaves, 0, s>>>(x, dz, offsets, src_token, T, d, E,
                                                             T * k, dw_r);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  if (dx_r && T > 0) {
    const dim3 g(static_cast<unsigned>((d + kDxCols - 1) / kDxCols),
                 static_cast<unsigned>((T + kDxTokens - 1) / kDxTokens));
    router_dx_topk_kernel<<<g, 64 * kDxWaves, 0, s>>>(w_r, dz, topk_idx, T, d, E, k, dx_r);
    return hipGetLastError();
  }
  return hipSuccess;
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
