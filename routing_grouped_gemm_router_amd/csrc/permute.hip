// Dispatch and Combine data movement (HBM-bound): permute into
// expert-contiguous rows, its adjoint, the weighted unpermute/combine and its
// backward, and the standalone SwiGLU kernels.
//
// Definition: "Scalable Training of Mixture-of-Experts Models with Megatron
// Core", section 2, Dispatch (tokens permuted by destination expert) and
// Combine (rows return to sequence order, weighted, plus a shared expert).
//
// Layout: 16-byte vectors along a row, 64 lanes of a wavefront side by side,
// so each instruction moves 1 KiB of one row.  The permutation is
// token-major: a token row is read once and written to its k destinations
// (and the combine reads its k rows and writes once), which is the
// algorithmic minimum of bytes.  Every load of a step (the k rows of a slot
// batch, several vectors per lane) is issued before the first is used, so a
// wave keeps many requests in flight.  Accumulation is fp32 with one rounding
// at the end.
#include "common.h"
#include "internal.h"

namespace moe {

template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(const uint4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ uint4 pack(const float (&f)[4]) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float (&f)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(f[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(f[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// 16-byte loads and stores with the non-temporal hint: rows that are read
// exactly once in a pass (the permuted rows in combine and the backward
// gathers) stream past the caches instead of evicting reused lines.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Index of this wavefront in the grid (4 waves per 256-thread block), as a
// wave-uniform value.
__device__ __forceinline__ int64_t wave_index() {
  return __builtin_amdgcn_readfirstlane(static_cast<int64_t>(blockIdx.x) * 4 +
                                        (threadIdx.x >> 6));
}

// Work decomposition of the row kernels: a unit is one token and one chunk of
// 64*U 16-byte vectors of its row (U per lane).  Chunks of one token are
// adjacent units, so neighbouring waves read neighbouring pieces of the same
// rows.  A wave takes units w, w + n_waves, ... (one each at the usual grid).
struct RowChunks {
  int64_t nvec, cpr, units;
  __device__ __forceinline__ RowChunks(int64_t T_, int64_t d, int vn, int U) {
    nvec = d / vn;
    cpr = (nvec + 64 * U - 1) / (64 * U);
    units = T_ * cpr;
  }
};

static dim3 unit_grid(int64_t units) {
  int64_t b = (units + 3) / 4;
  if (b > (int64_t(1) << 30)) b = int64_t(1) << 30;  // the unit loop covers the rest
  if (b < 1) b = 1;
  return dim3(static_cast<unsigned>(b));
}
static int64_t host_units(int64_t T_, int64_t d, int vn, int U) {
  const int64_t nvec = d / vn;
  return T_ * ((nvec + 64 * U - 1) / (64 * U));
}

// xp[dst_row[t, j]] = x[t]: each chunk of x is loaded once (U vectors per
// lane in flight) and stored to the token's k rows.
constexpr int kPermuteU = 4;
template <typename T>
__global__ __launch_bounds__(256) void permute_kernel(const T* __restrict__ x,
                                                      const int32_t* __restrict__ dst_row, int64_t T_,
                                                      int64_t d, int k, int64_t nrows,
                                                      T* __restrict__ xp) {
  constexpr int U = kPermuteU;
  const RowChunks rc(T_, d, Vec<T>::N, U);
  const int lane = threadIdx.x & 63;
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t un = wave_index(); un < rc.units; un += n_waves) {
    const int64_t t = un / rc.cpr, v0 = (un - t * rc.cpr) * 64 * U;
    const uint4* src = reinterpret_cast<const uint4*>(x + t * d);
    uint4 val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * 64 + lane;
      if (v < rc.nvec) val[u] = load_stream(src + v);
    }
    for (int j = 0; j < k; ++j) {
      const int64_t r = dst_row[t * k + j];
      if (r < 0 || r >= nrows) continue;
      uint4* dst = reinterpret_cast<uint4*>(xp + r * d);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        if (v < rc.nvec) dst[v] = val[u];
      }
    }
  }
}

// Rows of slots j0 .. j0+KB-1 of token t (wave-uniform; -1 for an absent or
// dropped slot) and their weights (0 for those).
template <int KB>
__device__ __forceinline__ void slot_batch(const int32_t* __restrict__ dst_row,
                                           const float* __restrict__ w, int64_t t, int k, int j0,
                                           int64_t nrows, int64_t (&rr)[KB], float (&ww)[KB]) {
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    int64_t r = -1;
    float wj = 0.f;
    if (j0 + j < k) {
      r = dst_row[t * k + j0 + j];
      if (r < 0 || r >= nrows) r = -1;
      else wj = w ? w[t * k + j0 + j] : 1.0f;
    }
    rr[j] = r;
    ww[j] = wj;
  }
}

// dx[t] = sum_j dxp[dst_row[t, j]] + addend[t] + addend_f32[t], fp32 sums in
// slot order; the slots' rows are loaded KB at a time.
template <typename T, int KB, int U>
__global__ __launch_bounds__(256) void permute_bwd_kernel(const T* __restrict__ dxp,
                                                          const int32_t* __restrict__ dst_row,
                                                          int64_t T_, int64_t d, int k,
                                                          int64_t nrows,
                                                          const T* __restrict__ addend,
                                                          const float* __restrict__ addend_f32,
                                                          T* __restrict__ dx) {
  constexpr int VN = Vec<T>::N;
  const RowChunks rc(T_, d, VN, U);
  const int lane = threadIdx.x & 63;
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t un = wave_index(); un < rc.units; un += n_waves) {
    const int64_t t = un / rc.cpr, v0 = (un - t * rc.cpr) * 64 * U;
    // the addends' chunks are requested first, with the rows of the first batch
    uint4 ad[U];
    uint4 af[U][VN / 4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * 64 + lane;
      if (v >= rc.nvec) continue;
      if (addend) ad[u] = load_stream(reinterpret_cast<const uint4*>(addend + t * d) + v);
      if (addend_f32) {
        const uint4* a = reinterpret_cast<const uint4*>(addend_f32 + t * d + v * VN);
#pragma unroll
        for (int i = 0; i < VN / 4; ++i) af[u][i] = load_stream(a + i);
      }
    }
    float acc[U][VN];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < VN; ++i) acc[u][i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += KB) {
      int64_t rr[KB];
      float ww[KB];
      slot_batch<KB>(dst_row, nullptr, t, k, j0, nrows, rr, ww);
      uint4 val[KB][U];
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + u * 64 + lane;
          if (rr[j] >= 0 && v < rc.nvec)
            val[j][u] = load_stream(reinterpret_cast<const uint4*>(dxp + rr[j] * d) + v);
        }
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        if (rr[j] < 0) continue;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float tmp[VN];
          Vec<T>::unpack(val[j][u], tmp);
#pragma unroll
          for (int i = 0; i < VN; ++i) acc[u][i] += tmp[i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * 64 + lane;
      if (v >= rc.nvec) continue;
      if (addend) {
        float tmp[VN];
        Vec<T>::unpack(ad[u], tmp);
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[u][i] += tmp[i];
      }
      if (addend_f32) {
#pragma unroll
        for (int i = 0; i < VN / 4; ++i) {
          acc[u][4 * i] += __uint_as_float(af[u][i].x);
          acc[u][4 * i + 1] += __uint_as_float(af[u][i].y);
          acc[u][4 * i + 2] += __uint_as_float(af[u][i].z);
          acc[u][4 * i + 3] += __uint_as_float(af[u][i].w);
        }
      }
      reinterpret_cast<uint4*>(dx + t * d)[v] = Vec<T>::pack(acc[u]);
    }
  }
}

// out[t] = sum_j w[t, j] * y[dst_row[t, j]] + shared[t]  (w = 1 without
// topk_w), fp32 sums in slot order, then the shared row, one rounding.
template <typename T, int KB, int U>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ dst_row,
                                                      const T* __restrict__ shared, int64_t T_,
                                                      int64_t d, int k, int64_t nrows,
                                                      T* __restrict__ out) {
  constexpr int VN = Vec<T>::N;
  const RowChunks rc(T_, d, VN, U);
  const int lane = threadIdx.x & 63;
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t un = wave_index(); un < rc.units; un += n_waves) {
    const int64_t t = un / rc.cpr, v0 = (un - t * rc.cpr) * 64 * U;
    uint4 sh[U];
    if (shared) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        if (v < rc.nvec) sh[u] = load_stream(reinterpret_cast<const uint4*>(shared + t * d) + v);
      }
    }
    float acc[U][VN];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < VN; ++i) acc[u][i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += KB) {
      int64_t rr[KB];
      float ww[KB];
      slot_batch<KB>(dst_row, topk_w, t, k, j0, nrows, rr, ww);
      uint4 val[KB][U];
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + u * 64 + lane;
          if (rr[j] >= 0 && v < rc.nvec)
            val[j][u] = load_stream(reinterpret_cast<const uint4*>(y + rr[j] * d) + v);
        }
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        if (rr[j] < 0) continue;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float tmp[VN];
          Vec<T>::unpack(val[j][u], tmp);
#pragma unroll
          for (int i = 0; i < VN; ++i) acc[u][i] += ww[j] * tmp[i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * 64 + lane;
      if (v >= rc.nvec) continue;
      if (shared) {
        float tmp[VN];
        Vec<T>::unpack(sh[u], tmp);
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[u][i] += tmp[i];
      }
      reinterpret_cast<uint4*>(out + t * d)[v] = Vec<T>::pack(acc[u]);
    }
  }
}

// dy[dst_row[t, j]] = w[t, j] * dout[t];  d_w[t, j] = <dout[t], y[dst_row[t, j]]>
// One workgroup per token, its 4 waves on 4 quarters of the row (so each
// wave's chain of dependent steps is a quarter as long); slots KB at a time,
// U vectors per lane, every row load of a step issued before its use.  The
// dot products are summed over each wave, then over the 4 waves in order
// through LDS (deterministic).
template <typename T, int KB, int U>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dout,
                                                          const T* __restrict__ y,
                                                          const float* __restrict__ topk_w,
                                                          const int32_t* __restrict__ dst_row,
                                                          int64_t T_, int64_t d, int k,
                                                          int64_t nrows, T* __restrict__ dy,
                                                          float* __restrict__ d_w) {
  constexpr int VN = Vec<T>::N;
  __shared__ float part[4][KB];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nvec = d / VN;
  const int64_t q = (nvec + 3) / 4;  // vectors of each wave's quarter
  const int64_t vb = wave * q, ve = min(nvec, vb + q);
  const uint4* g_row = reinterpret_cast<const uint4*>(dout + t * d);
  for (int j0 = 0; j0 < k; j0 += KB) {
    int64_t rr[KB];
    float ww[KB], dot[KB];
    slot_batch<KB>(dst_row, topk_w, t, k, j0, nrows, rr, ww);
#pragma unroll
    for (int j = 0; j < KB; ++j) dot[j] = 0.f;
    for (int64_t v0 = vb; v0 < ve; v0 += 64 * U) {
      uint4 gv[U], val[KB][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        if (v < ve) gv[u] = g_row[v];
      }
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + u * 64 + lane;
          if (rr[j] >= 0 && v < ve)
            val[j][u] = load_stream(reinterpret_cast<const uint4*>(y + rr[j] * d) + v);
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * 64 + lane;
        if (v >= ve) continue;
        float g[VN];
        Vec<T>::unpack(gv[u], g);
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          if (rr[j] < 0) continue;
          float tmp[VN], o[VN], sdot = 0.f;
          Vec<T>::unpack(val[j][u], tmp);
#pragma unroll
          for (int i = 0; i < VN; ++i) {
            sdot += g[i] * tmp[i];
            o[i] = ww[j] * g[i];
          }
          dot[j] += sdot;
          reinterpret_cast<uint4*>(dy + rr[j] * d)[v] = Vec<T>::pack(o);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const float sw = wave_sum(dot[j]);
      if (lane == 0) part[wave][j] = sw;
    }
    __syncthreads();
    if (threadIdx.x < KB && j0 + static_cast<int>(threadIdx.x) < k) {
      const int j = threadIdx.x;
      d_w[t * k + j0 + j] = ((part[0][j] + part[1][j]) + part[2][j]) + part[3][j];
    }
    __syncthreads();
  }
}

// Routing weight of every permuted row: w_perm[dst_row[t, j]] = w[t, j].
__global__ __launch_bounds__(256) void permute_weights_kernel(const float* __restrict__ topk_w,
                                                              const int32_t* __restrict__ dst_row,
                                                              int64_t n, float* __restrict__ w_perm) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t r = dst_row[i];
  if (r >= 0 && r < n) w_perm[r] = topk_w[i];
}

// Gradient of the routing weights applied inside the experts:
// d_w[t, j] = sum_c gate_part[dst_row[t, j], c], c = 0 .. P-1 in order.
__global__ __launch_bounds__(256) void gate_grad_kernel(const float* __restrict__ gate_part,
                                                        int64_t P,
                                                        const int32_t* __restrict__ dst_row,
                                                        int64_t n, float* __restrict__ d_w) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t r = dst_row[i];
  float s = 0.0f;
  if (r >= 0 && r < n)
    for (int64_t c = 0; c < P; ++c) s += gate_part[r * P + c];
  d_w[i] = s;
}

// h = silu(a) * b over rows of ab = [a | b]
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(const T* __restrict__ ab, int64_t M, int64_t f,
                                                     T* __restrict__ h) {
  constexpr int VN = Vec<T>::N;
  const int64_t nv = f / VN;
  const int64_t total = M * nv;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t m = i / nv, v = i % nv;
    float a[VN], b[VN], o[VN];
    Vec<T>::unpack(reinterpret_cast<const uint4*>(ab + m * 2 * f)[v], a);
    Vec<T>::unpack(reinterpret_cast<const uint4*>(ab + m * 2 * f + f)[v], b);
#pragma unroll
    for (int e = 0; e < VN; ++e) o[e] = a[e] / (1.0f + expf(-a[e])) * b[e];
    reinterpret_cast<uint4*>(h + m * f)[v] = Vec<T>::pack(o);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const T* __restrict__ dh,
                                                         const T* __restrict__ ab, int64_t M,
                                                         int64_t f, T* __restrict__ dab) {
  constexpr int VN = Vec<T>::N;
  const int64_t nv = f / VN;
  const int64_t total = M * nv;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t m = i / nv, v = i % nv;
    float a[VN], b[VN], g[VN], da[VN], db[VN];
    Vec<T>::unpack(reinterpret_cast<const uint4*>(ab + m * 2 * f)[v], a);
    Vec<T>::unpack(reinterpret_cast<const uint4*>(ab + m * 2 * f + f)[v], b);
    Vec<T>::unpack(reinterpret_cast<const uint4*>(dh + m * f)[v], g);
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      const float s = 1.0f / (1.0f + expf(-a[e]));
      da[e] = g[e] * b[e] * s * (1.0f + a[e] * (1.0f - s));
      db[e] = g[e] * a[e] * s;
    }
    reinterpret_cast<uint4*>(dab + m * 2 * f)[v] = Vec<T>::pack(da);
    reinterpret_cast<uint4*>(dab + m * 2 * f + f)[v] = Vec<T>::pack(db);
  }
}

static dim3 elem_grid(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return dim3(static_cast<unsigned>(b));
}

// Slot batch size: all of a token's slots at once up to 8, else batches of 8.
#define MOE_SLOT_BATCH_DISPATCH(k, KERNEL, ...) \
  do {                                          \
    if ((k) <= 2) KERNEL(2, __VA_ARGS__);       \
    else if ((k) <= 4) KERNEL(4, __VA_ARGS__);  \
    else KERNEL(8, __VA_ARGS__);                \
  } while (0)

hipError_t launch_permute(const void* x, int dtype, const int32_t* dst_row, int64_t T, int64_t d,
                          int k, int64_t nrows, void* xp, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 0)
    permute_kernel<float><<<unit_grid(host_units(T, d, 4, kPermuteU)), 256, 0, s>>>(
        static_cast<const float*>(x), dst_row, T, d, k, nrows, static_cast<float*>(xp));
  else
    permute_kernel<bf16_t><<<unit_grid(host_units(T, d, 8, kPermuteU)), 256, 0, s>>>(
        static_cast<const bf16_t*>(x), dst_row, T, d, k, nrows, static_cast<bf16_t*>(xp));
  return hipGetLastError();
}

constexpr int kPermuteBwdU = 1;
template <typename T>
static void permute_bwd_dispatch(const T* dxp, const int32_t* dst, int64_t Tn, int64_t d, int k,
                                 int64_t nrows, const T* addend, const float* addend_f32, T* dx,
                                 hipStream_t s) {
  const dim3 g = unit_grid(host_units(Tn, d, Vec<T>::N, kPermuteBwdU));
#define MOE_PBWD(KB, ...) \
  permute_bwd_kernel<T, KB, kPermuteBwdU><<<g, 256, 0, s>>>(dxp, dst, Tn, d, k, nrows, addend, \
                                                            addend_f32, dx)
  MOE_SLOT_BATCH_DISPATCH(k, MOE_PBWD, 0);
#undef MOE_PBWD
}

hipError_t launch_permute_bwd(const void* dxp, int dtype, const int32_t* dst_row, int64_t T,
                              int64_t d, int k, int64_t nrows, const void* addend,
                              const float* addend_f32, void* dx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 0)
    permute_bwd_dispatch<float>(static_cast<const float*>(dxp), dst_row, T, d, k, nrows,
                                static_cast<const float*>(addend), addend_f32,
                                static_cast<float*>(dx), s);
  else
    permute_bwd_dispatch<bf16_t>(static_cast<const bf16_t*>(dxp), dst_row, T, d, k, nrows,
                                 static_cast<const bf16_t*>(addend), addend_f32,
                                 static_cast<bf16_t*>(dx), s);
  return hipGetLastError();
}

constexpr int kCombineU = 1;
template <typename T>
static void combine_dispatch(const T* y, const float* w, const int32_t* dst, const T* shared,
                             int64_t Tn, int64_t d, int k, int64_t nrows, T* out, hipStream_t s) {
  const dim3 g = unit_grid(host_units(Tn, d, Vec<T>::N, kCombineU));
#define MOE_COMB(KB, ...) \
  combine_kernel<T, KB, kCombineU><<<g, 256, 0, s>>>(y, w, dst, shared, Tn, d, k, nrows, out)
  MOE_SLOT_BATCH_DISPATCH(k, MOE_COMB, 0);
#undef MOE_COMB
}

hipError_t launch_combine(const void* y, int dtype, const float* topk_w, const int32_t* dst_row,
                          const void* shared, int64_t T, int64_t d, int k, int64_t nrows,
                          void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 0)
    combine_dispatch<float>(static_cast<const float*>(y), topk_w, dst_row,
                            static_cast<const float*>(shared), T, d, k, nrows,
                            static_cast<float*>(out), s);
  else
    combine_dispatch<bf16_t>(static_cast<const bf16_t*>(y), topk_w, dst_row,
                             static_cast<const bf16_t*>(shared), T, d, k, nrows,
                             static_cast<bf16_t*>(out), s);
  return hipGetLastError();
}

constexpr int kCombineBwdU = 2;
template <typename T>
static void combine_bwd_dispatch(const T* dout, const T* y, const float* w, const int32_t* dst,
                                 int64_t Tn, int64_t d, int k, int64_t nrows, T* dy, float* dw,
                                 hipStream_t s) {
  const dim3 g(static_cast<unsigned>(Tn));  // one workgroup per token
#define MOE_CBWD(KB, ...) \
  combine_bwd_kernel<T, KB, kCombineBwdU><<<g, 256, 0, s>>>(dout, y, w, dst, Tn, d, k, nrows, dy, dw)
  MOE_SLOT_BATCH_DISPATCH(k, MOE_CBWD, 0);
#undef MOE_CBWD
}

hipError_t launch_combine_bwd(const void* dout, const void* y, int dtype, const float* topk_w,
                              const int32_t* dst_row, int64_t T, int64_t d, int k, int64_t nrows,
                              void* dy, float* d_w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 0)
    combine_bwd_dispatch<float>(static_cast<const float*>(dout), static_cast<const float*>(y),
                                topk_w, dst_row, T, d, k, nrows, static_cast<float*>(dy), d_w, s);
  else
    combine_bwd_dispatch<bf16_t>(static_cast<const bf16_t*>(dout), static_cast<const bf16_t*>(y),
                                 topk_w, dst_row, T, d, k, nrows, static_cast<bf16_t*>(dy), d_w, s);
  return hipGetLastError();
}

hipError_t launch_permute_weights(const float* topk_w, const int32_t* dst_row, int64_t T, int k,
                                  float* w_perm, hipStream_t s) {
  const int64_t n = T * k;
  if (n == 0) return hipSuccess;
  permute_weights_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, s>>>(
      topk_w, dst_row, n, w_perm);
  return hipGetLastError();
}

hipError_t launch_gate_grad(const float* gate_part, int64_t P, const int32_t* dst_row, int64_t T,
                            int k, float* d_topk_w, hipStream_t s) {
  const int64_t n = T * k;
  if (n == 0) return hipSuccess;
  gate_grad_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, s>>>(
      gate_part, P, dst_row, n, d_topk_w);
  return hipGetLastError();
}

hipError_t launch_swiglu(const void* ab, int dtype, int64_t M, int64_t f, void* h, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (dtype == 0)
    swiglu_kernel<float><<<elem_grid(M * f / 4), 256, 0, s>>>(static_cast<const float*>(ab), M, f,
                                                              static_cast<float*>(h));
  else
    swiglu_kernel<bf16_t><<<elem_grid(M * f / 8), 256, 0, s>>>(static_cast<const bf16_t*>(ab), M,
                                                               f, static_cast<bf16_t*>(h));
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* dh, const void* ab, int dtype, int64_t M, int64_t f,
                             void* dab, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (dtype == 0)
    swiglu_bwd_kernel<float><<<elem_grid(M * f / 4), 256, 0, s>>>(
        static_cast<const float*>(dh), static_cast<const float*>(ab), M, f,
        static_cast<float*>(dab));
  else
    swiglu_bwd_kernel<bf16_t><<<elem_grid(M * f / 8), 256, 0, s>>>(
        static_cast<const bf16_t*>(dh), static_cast<const bf16_t*>(ab), M, f,
        static_cast<bf16_t*>(dab));
  return hipGetLastError();
}

// Zero the rows of a permuted buffer that hold no (token, slot) pair
// (src_token < 0: the padding of a pad-to-max layout), 16 bytes per lane.
__global__ __launch_bounds__(256) void zero_unmapped_rows_kernel(uint4* __restrict__ buf,
                                                                 const int32_t* __restrict__ src_token,
                                                                 int64_t M, int64_t chunks) {
  const int64_t r = blockIdx.x;
  if (r >= M || src_token[r] >= 0) return;
  uint4* row = buf + r * chunks;
  for (int64_t c = threadIdx.x; c < chunks; c += 256) row[c] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero_unmapped_rows(void* buf, int64_t row_bytes, const int32_t* src_token,
                                     int64_t M, hipStream_t s) {
  if (M == 0) return hipSuccess;
  zero_unmapped_rows_kernel<<<dim3(static_cast<unsigned>(M)), 256, 0, s>>>(
      static_cast<uint4*>(buf), src_token, M, row_bytes / 16);
  return hipGetLastError();
}

}  // namespace moe
