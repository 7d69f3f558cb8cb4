// bf16 grouped GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulation): the experts' SwiGLU FFNs of "Scalable Training of
// Mixture-of-Experts Models with Megatron Core", section 2, Expert Computation
// (the local experts' GEMMs run together over their ragged row groups).
//
// Three products, each over G groups (experts):
//   forward  C[rows g]  = A[rows g] . B[g]       A [M,K]  B [G,K,N]   (NN)
//   dgrad    dA[rows g] = dC[rows g] . B[g]^T    dC [M,N] B [G,K,N]   (NT)
//   wgrad    dB[g]      = A[rows g]^T . dC[rows g]                   (TN)
//
// Design (MI355X):
//  * Persistent grid of 2 workgroups per CU.  Each workgroup rebuilds the
//    per-group row-tile prefix from the device offsets in LDS (no host sync,
//    no workspace), then walks tiles tau = v, v + P, ...  The virtual id v
//    makes the workgroups of one XCD (hardware dispatches workgroup b to XCD
//    b mod 8) own consecutive tiles, so the N tiles of one expert row block run
//    on one XCD and share its activations in that XCD's L2, while each weight
//    tile is streamed from HBM once per row block.
//  * 128 x 128 x 64 tiles, 4 waves in a 2 x 2 arrangement, each wave 64 x 64 =
//    2 x 2 MFMA 32x32x16 blocks.  LDS holds both operands k-contiguous
//    ([row][k], pitch 72 elements = 144 B, so 16 consecutive rows fall in 16
//    distinct bank quads); two buffers, one barrier per k step, the next k
//    step's global loads in flight during the MFMAs.
//  * Operands whose contraction axis is strided in memory (the weights in the
//    forward, both operands of wgrad) are loaded as 8 x 8 blocks of 16-byte
//    vectors and transposed in registers before the LDS store.
//  * Epilogues: SwiGLU (H = silu(A) * B from the fp32 sums; the tile holds
//    matching gate and up columns) and SwiGLU backward (dH -> dAB, reading AB).
#include "common.h"
#include "internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LP = BK + 8;  // LDS row pitch (bf16 elements)
constexpr int MAX_GROUPS = 1024;

enum { MODE_FWD = 0, MODE_FWD_SWIGLU = 1, MODE_DGRAD = 2, MODE_DGRAD_SWIGLU_BWD = 3 };

static int g_cu_count[64];

static int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// ---- operand staging -----------------------------------------------------

// k-contiguous operand: 128 rows x 64 k = 1024 16-byte vectors, 4 per thread.
__device__ __forceinline__ void kc_load(uint4 (&r)[4], const bf16_t* __restrict__ base, int64_t ld,
                                        int rows_valid, int tid) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int idx = tid + v * 256;
    const int row = idx >> 3, c = idx & 7;
    r[v] = row < rows_valid ? *reinterpret_cast<const uint4*>(base + row * ld + c * 8)
                            : make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ void kc_store(bf16_t* __restrict__ lds, const uint4 (&r)[4], int tid) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int idx = tid + v * 256;
    const int row = idx >> 3, c = idx & 7;
    *reinterpret_cast<uint4*>(lds + row * LP + c * 8) = r[v];
  }
}

// Row-contiguous operand (contraction strided): thread lt < 128 owns the 8 x 8
// block kb = lt % 8 (k), rb = lt / 8 (rows).  Element (kk, row) of the tile is
// at base + kk * ld + row; `col` is this thread's row offset for its block.
__device__ __forceinline__ void nc_load(uint4 (&r)[8], const bf16_t* __restrict__ base, int64_t ld,
                                        int64_t col, int k_valid, int lt) {
  const int kb = lt & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int kk = kb * 8 + i;
    r[i] = kk < k_valid ? *reinterpret_cast<const uint4*>(base + kk * ld + col)
                        : make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ uint32_t wsel(const uint4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

__device__ __forceinline__ void nc_store(bf16_t* __restrict__ lds, const uint4 (&r)[8], int lt) {
  const int kb = lt & 7, rb = lt >> 3;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = wsel(r[2 * p], q >> 1), hi = wsel(r[2 * p + 1], q >> 1);
      o[p] = (q & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    *reinterpret_cast<uint4*>(lds + (rb * 8 + q) * LP + kb * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---- MFMA on one staged k step ---------------------------------------------

__device__ __forceinline__ void mma_step(f32x16_t (&acc)[2][2], const bf16_t* __restrict__ As,
                                         const bf16_t* __restrict__ Bs, int wm, int wn, int lane) {
  const int r = lane & 31, kq = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < BK; kk += 16) {
    bf16x8_t a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 64 + i * 32 + r) * LP + kk + kq);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * 64 + j * 32 + r) * LP + kk + kq);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// row (within the 128 x 128 tile) of accumulator element v of block (i, .)
__device__ __forceinline__ int acc_row(int wm, int i, int v, int lane) {
  return wm * 64 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
}

__device__ __forceinline__ int virtual_block() {
  const int P = gridDim.x, b = blockIdx.x;
  return (P % 8 == 0) ? (b % 8) * (P / 8) + b / 8 : b;
}

// ---- row-grouped products: forward and dgrad ---------------------------------
//
// MODE_FWD*:   A [M, Kc] (lda = Kc); B_g = B + g * Kc * N, element (k, n) at k * N + n.
//              NONE: tile columns nt * 128 + c of C [M, N].
//              SWIGLU: N = 2f; tile = 64 h columns; B rows of the tile are
//              [gate 0..31 | up 0..31] for wave column 0 then for wave column 1.
// MODE_DGRAD*: A = dC [M, Kc] (Kc = N); B_g = B + g * Nout * Kc, element (k, n)
//              at n * Kc + k; product columns Nout = K.
template <int MODE>
__global__ __launch_bounds__(256) void gg_bf16_rows_kernel(const bf16_t* __restrict__ A,
                                                           const bf16_t* __restrict__ B,
                                                           const int64_t* __restrict__ off, int G,
                                                           int64_t M, int64_t Kc, int64_t Nout,
                                                           bf16_t* __restrict__ C,
                                                           bf16_t* __restrict__ H,
                                                           const bf16_t* __restrict__ ab) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LP];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LP];
  __shared__ int s_pre[MAX_GROUPS + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr bool FWD = MODE == MODE_FWD || MODE == MODE_FWD_SWIGLU;
  constexpr bool SWI = MODE == MODE_FWD_SWIGLU;

  // row-tile prefix over groups, built by wave 0
  if (wave == 0) {
    const int per = (G + 63) / 64;
    const int g0 = lane * per, g1 = min(G, g0 + per);
    int sum = 0;
    for (int g = g0; g < g1; ++g) {
      const int64_t lo = clamp64(off[g], 0, M), hi = clamp64(off[g + 1], lo, M);
      sum += static_cast<int>((hi - lo + BM - 1) / BM);
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    int run = incl - sum;
    for (int g = g0; g < g1; ++g) {
      s_pre[g] = run;
      const int64_t lo = clamp64(off[g], 0, M), hi = clamp64(off[g + 1], lo, M);
      run += static_cast<int>((hi - lo + BM - 1) / BM);
    }
    if (lane == 63) s_pre[G] = incl;
  }
  __syncthreads();

  const int64_t NT = SWI ? Nout / 128 : Nout / BN;  // SWIGLU: Nout = 2f, 64 h columns per tile
  const int64_t fh = Nout / 2;
  const int64_t total = static_cast<int64_t>(s_pre[G]) * NT;
  const int P = gridDim.x;
  const int nk = static_cast<int>(Kc / BK);
  const int lt = tid & 127;
  const bool b_loader = !FWD || tid < 128;

  for (int64_t tau = virtual_block(); tau < total; tau += P) {
    const int mtg = static_cast<int>(tau / NT);
    const int64_t nt = tau % NT;
    int glo = 0, ghi = G;
    while (ghi - glo > 1) {
      const int mid = (glo + ghi) >> 1;
      if (s_pre[mid] <= mtg) glo = mid; else ghi = mid;
    }
    const int g = glo;
    const int64_t lo = clamp64(off[g], 0, M), hi = clamp64(off[g + 1], lo, M);
    const int64_t row0 = lo + static_cast<int64_t>(mtg - s_pre[g]) * BM;
    const int rows = static_cast<int>(min<int64_t>(BM, hi - row0));

    const bf16_t* Ab = A + row0 * Kc;
    const bf16_t* Bb;
    int64_t bcol = 0;
    if (FWD) {
      Bb = B + static_cast<int64_t>(g) * Kc * Nout;
      const int rb = lt >> 3;
      if (SWI)
        bcol = ((rb >> 2) & 1) * fh + nt * 64 + (rb >> 3) * 32 + (rb & 3) * 8;
      else
        bcol = nt * BN + rb * 8;
    } else {
      Bb = B + static_cast<int64_t>(g) * Nout * Kc + nt * BN * Kc;
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    uint4 ra[4], rbk[4], rbn[8];
    kc_load(ra, Ab, Kc, rows, tid);
    if (FWD) {
      if (b_loader) nc_load(rbn, Bb, Nout, bcol, BK, lt);
    } else {
      kc_load(rbk, Bb, Kc, BN, tid);
    }
    kc_store(sA[0], ra, tid);
    if (FWD) {
      if (b_loader) nc_store(sB[0], rbn, lt);
    } else {
      kc_store(sB[0], rbk, tid);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        const int64_t k0 = static_cast<int64_t>(kt + 1) * BK;
        kc_load(ra, Ab + k0, Kc, rows, tid);
        if (FWD) {
          if (b_loader) nc_load(rbn, Bb + k0 * Nout, Nout, bcol, BK, lt);
        } else {
          kc_load(rbk, Bb + k0, Kc, BN, tid);
        }
      }
      mma_step(acc, sA[cur], sB[cur], wm, wn, lane);
      if (more) {
        kc_store(sA[cur ^ 1], ra, tid);
        if (FWD) {
          if (b_loader) nc_store(sB[cur ^ 1], rbn, lt);
        } else {
          kc_store(sB[cur ^ 1], rbk, tid);
        }
      }
      __syncthreads();
    }

    // epilogue
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = acc_row(wm, i, v, lane);
        if (rl >= rows) continue;
        const int64_t row = row0 + rl;
        if (SWI) {
          const int64_t hc = nt * 64 + wn * 32 + (lane & 31);
          const float a = acc[i][0][v], b = acc[i][1][v];
          if (C) {
            C[row * Nout + hc] = f32_to_bf16(a);
            C[row * Nout + fh + hc] = f32_to_bf16(b);
          }
          H[row * fh + hc] = f32_to_bf16(a / (1.0f + expf(-a)) * b);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int64_t col = nt * BN + wn * 64 + j * 32 + (lane & 31);
            const float x = acc[i][j][v];
            if (MODE == MODE_DGRAD_SWIGLU_BWD) {
              const float a = bf16_to_f32(ab[row * 2 * Nout + col]);
              const float b = bf16_to_f32(ab[row * 2 * Nout + Nout + col]);
              const float s = 1.0f / (1.0f + expf(-a));
              C[row * 2 * Nout + col] = f32_to_bf16(x * b * s * (1.0f + a * (1.0f - s)));
              C[row * 2 * Nout + Nout + col] = f32_to_bf16(x * a * s);
            } else {
              C[row * Nout + col] = f32_to_bf16(x);
            }
          }
        }
      }
    }
  }
}

// ---- wgrad: dB[g] = A[rows g]^T . dC[rows g] ---------------------------------
// Output tile (mt, nt) of group g; contraction over the group's rows in steps
// of 64 (the last one zero-padded).  Threads 0..127 stage A, 128..255 stage dC.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void gg_bf16_wgrad_kernel(const bf16_t* __restrict__ A,
                                                            const bf16_t* __restrict__ dC,
                                                            const int64_t* __restrict__ off, int G,
                                                            int64_t M, int64_t K, int64_t N,
                                                            void* __restrict__ dB, int accumulate) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LP];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lt = tid & 127;
  const bool loads_a = tid < 128;
  const int64_t MT = K / BM, NT = N / BN;
  const int64_t total = static_cast<int64_t>(G) * MT * NT;
  const int P = gridDim.x;

  for (int64_t tau = virtual_block(); tau < total; tau += P) {
    const int g = static_cast<int>(tau / (MT * NT));
    const int64_t rem = tau % (MT * NT);
    const int64_t mt = rem / NT, nt = rem % NT;
    const int64_t lo = clamp64(off[g], 0, M), hi = clamp64(off[g + 1], lo, M);
    const int64_t nrows = hi - lo;
    const int nk = static_cast<int>((nrows + BK - 1) / BK);
    const int rb = lt >> 3;
    const bf16_t* base = loads_a ? A + lo * K + mt * BM : dC + lo * N + nt * BN;
    const int64_t ld = loads_a ? K : N;
    bf16_t(*sX)[BM * LP] = loads_a ? sA : sB;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    if (nk > 0) {
      uint4 r[8];
      nc_load(r, base, ld, rb * 8, static_cast<int>(min<int64_t>(BK, nrows)), lt);
      nc_store(sX[0], r, lt);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
          const int64_t k0 = static_cast<int64_t>(kt + 1) * BK;
          nc_load(r, base + k0 * ld, ld, rb * 8, static_cast<int>(min<int64_t>(BK, nrows - k0)), lt);
        }
        mma_step(acc, sA[cur], sB[cur], wm, wn, lane);
        if (more) nc_store(sX[cur ^ 1], r, lt);
        __syncthreads();
      }
    } else if (accumulate) {
      continue;
    }

#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = mt * BM + acc_row(wm, i, v, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = nt * BN + wn * 64 + j * 32 + (lane & 31);
          const int64_t o = static_cast<int64_t>(g) * K * N + row * N + col;
          float x = acc[i][j][v];
          if (OUT_F32) {
            float* p = static_cast<float*>(dB) + o;
            if (accumulate) x += *p;
            *p = x;
          } else {
            bf16_t* p = static_cast<bf16_t*>(dB) + o;
            if (accumulate) x += bf16_to_f32(*p);
            *p = f32_to_bf16(x);
          }
        }
      }
    }
  }
}

static unsigned persistent_grid(int64_t tiles_upper_bound) {
  int64_t p = static_cast<int64_t>(cu_count()) * 2;
  if (tiles_upper_bound < p) p = tiles_upper_bound;
  if (p < 1) p = 1;
  return static_cast<unsigned>(p);
}

hipError_t launch_gg_bf16_fwd(const void* A, const void* B, const int64_t* off, int G, int64_t M,
                              int64_t K, int64_t N, int epi, void* C, void* H, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t nt = epi == EPI_SWIGLU ? N / 128 : N / BN;
  const dim3 grid(persistent_grid((M / BM + G) * nt));
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* b = static_cast<const bf16_t*>(B);
  if (epi == EPI_SWIGLU)
    gg_bf16_rows_kernel<MODE_FWD_SWIGLU><<<grid, 256, 0, s>>>(
        a, b, off, G, M, K, N, static_cast<bf16_t*>(C), static_cast<bf16_t*>(H), nullptr);
  else
    gg_bf16_rows_kernel<MODE_FWD><<<grid, 256, 0, s>>>(a, b, off, G, M, K, N,
                                                       static_cast<bf16_t*>(C), nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_gg_bf16_dgrad(const void* dC, const void* B, const int64_t* off, int G,
                                int64_t M, int64_t K, int64_t N, int epi, const void* ab, void* dA,
                                hipStream_t s) {
  if (M == 0) return hipSuccess;
  const dim3 grid(persistent_grid((M / BM + G) * (K / BN)));
  const bf16_t* a = static_cast<const bf16_t*>(dC);
  const bf16_t* b = static_cast<const bf16_t*>(B);
  if (epi == EPI_SWIGLU_BWD)
    gg_bf16_rows_kernel<MODE_DGRAD_SWIGLU_BWD><<<grid, 256, 0, s>>>(
        a, b, off, G, M, N, K, static_cast<bf16_t*>(dA), nullptr, static_cast<const bf16_t*>(ab));
  else
    gg_bf16_rows_kernel<MODE_DGRAD><<<grid, 256, 0, s>>>(a, b, off, G, M, N, K,
                                                         static_cast<bf16_t*>(dA), nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_gg_bf16_wgrad(const void* A, const void* dC, const int64_t* off, int G,
                                int64_t M, int64_t K, int64_t N, int db_f32, int accumulate,
                                void* dB, hipStream_t s) {
  const int64_t tiles = static_cast<int64_t>(G) * (K / BM) * (N / BN);
  if (tiles == 0) return hipSuccess;
  const dim3 grid(persistent_grid(tiles));
  const bf16_t* a = static_cast<const bf16_t*>(A);
  const bf16_t* c = static_cast<const bf16_t*>(dC);
  if (db_f32)
    gg_bf16_wgrad_kernel<true><<<grid, 256, 0, s>>>(a, c, off, G, M, K, N, dB, accumulate);
  else
    gg_bf16_wgrad_kernel<false><<<grid, 256, 0, s>>>(a, c, off, G, M, K, N, dB, accumulate);
  return hipGetLastError();
}

}  // namespace moe
