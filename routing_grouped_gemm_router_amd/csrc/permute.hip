// Dispatch and Combine data movement (HBM-bound): permute into
// expert-contiguous rows, its adjoint, the weighted unpermute/combine and its
// backward, and the standalone SwiGLU kernels.
//
// Definition: "Scalable Training of Mixture-of-Experts Models with Megatron
// Core", section 2, Dispatch (tokens permuted by destination expert) and
// Combine (rows return to sequence order, weighted, plus a shared expert).
//
// Layout: one wavefront per token row, 16-byte vectors along the row, so each
// instruction moves 1 KiB of one row.  The permutation is token-major: a token
// row is read once and written to its k destinations (and the combine reads
// its k rows and writes once), which is the algorithmic minimum of bytes.
// Accumulation is fp32 with one rounding at the end.
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

__device__ __forceinline__ int64_t wave_token(int per_block) {
  // the token handled by this wavefront, as a wave-uniform value
  return __builtin_amdgcn_readfirstlane(static_cast<int64_t>(blockIdx.x) * per_block +
                                        (threadIdx.x >> 6));
}

template <typename T>
__global__ __launch_bounds__(256) void permute_kernel(const T* __restrict__ x,
                                                      const int32_t* __restrict__ dst_row, int64_t T_,
                                                      int64_t d, int k, int64_t nrows,
                                                      T* __restrict__ xp) {
  const int64_t t = wave_token(4);
  if (t >= T_) return;
  const int lane = threadIdx.x & 63;
  const int64_t nvec = d / Vec<T>::N;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * d);
  for (int64_t v = lane; v < nvec; v += 64) {
    const uint4 val = src[v];
    for (int j = 0; j < k; ++j) {
      const int64_t r = dst_row[t * k + j];
      if (r >= 0 && r < nrows) reinterpret_cast<uint4*>(xp + r * d)[v] = val;
    }
  }
}

// dx[t] = sum_j dxp[dst_row[t, j]] + addend[t] + addend_f32[t]
template <typename T>
__global__ __launch_bounds__(256) void permute_bwd_kernel(const T* __restrict__ dxp,
                                                          const int32_t* __restrict__ dst_row,
                                                          int64_t T_, int64_t d, int k,
                                                          int64_t nrows,
                                                          const T* __restrict__ addend,
                                                          const float* __restrict__ addend_f32,
                                                          T* __restrict__ dx) {
  constexpr int VN = Vec<T>::N;
  const int64_t t = wave_token(4);
  if (t >= T_) return;
  const int lane = threadIdx.x & 63;
  const int64_t nvec = d / VN;
  for (int64_t v = lane; v < nvec; v += 64) {
    float acc[VN] = {};
    float tmp[VN];
    for (int j = 0; j < k; ++j) {
      const int64_t r = dst_row[t * k + j];
      if (r < 0 || r >= nrows) continue;
      Vec<T>::unpack(reinterpret_cast<const uint4*>(dxp + r * d)[v], tmp);
#pragma unroll
      for (int i = 0; i < VN; ++i) acc[i] += tmp[i];
    }
    if (addend) {
      Vec<T>::unpack(reinterpret_cast<const uint4*>(addend + t * d)[v], tmp);
#pragma unroll
      for (int i = 0; i < VN; ++i) acc[i] += tmp[i];
    }
    if (addend_f32) {
      const float* a = addend_f32 + t * d + v * VN;
#pragma unroll
      for (int i = 0; i < VN; i += 4) {
        const float4 q = *reinterpret_cast<const float4*>(a + i);
        acc[i] += q.x; acc[i + 1] += q.y; acc[i + 2] += q.z; acc[i + 3] += q.w;
      }
    }
    reinterpret_cast<uint4*>(dx + t * d)[v] = Vec<T>::pack(acc);
  }
}

// out[t] = sum_j w[t, j] * y[dst_row[t, j]] + shared[t]  (w = 1 without topk_w)
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ dst_row,
                                                      const T* __restrict__ shared, int64_t T_,
                                                      int64_t d, int k, int64_t nrows,
                                                      T* __restrict__ out) {
  constexpr int VN = Vec<T>::N;
  const int64_t t = wave_token(4);
  if (t >= T_) return;
  const int lane = threadIdx.x & 63;
  const int64_t nvec = d / VN;
  for (int64_t v = lane; v < nvec; v += 64) {
    float acc[VN] = {};
    float tmp[VN];
    for (int j = 0; j < k; ++j) {
      const int64_t r = dst_row[t * k + j];
      if (r < 0 || r >= nrows) continue;
      Vec<T>::unpack(reinterpret_cast<const uint4*>(y + r * d)[v], tmp);
      if (topk_w) {
        const float w = topk_w[t * k + j];
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] += w * tmp[i];
      } else {
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] += tmp[i];
      }
    }
    if (shared) {
      Vec<T>::unpack(reinterpret_cast<const uint4*>(shared + t * d)[v], tmp);
#pragma unroll
      for (int i = 0; i < VN; ++i) acc[i] += tmp[i];
    }
    reinterpret_cast<uint4*>(out + t * d)[v] = Vec<T>::pack(acc);
  }
}

// dy[dst_row[t, j]] = w[t, j] * dout[t];  d_w[t, j] = <dout[t], y[dst_row[t, j]]>
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dout,
                                                          const T* __restrict__ y,
                                                          const float* __restrict__ topk_w,
                                                          const int32_t* __restrict__ dst_row,
                                                          int64_t T_, int64_t d, int k,
                                                          int64_t nrows, T* __restrict__ dy,
                                                          float* __restrict__ d_w) {
  constexpr int VN = Vec<T>::N;
  const int64_t t = wave_token(4);
  if (t >= T_) return;
  const int lane = threadIdx.x & 63;
  const int64_t nvec = d / VN;
  float dot[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) dot[j] = 0.f;
  for (int64_t v = lane; v < nvec; v += 64) {
    float g[VN], tmp[VN], o[VN];
    Vec<T>::unpack(reinterpret_cast<const uint4*>(dout + t * d)[v], g);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) continue;
      const int64_t r = dst_row[t * k + j];
      if (r < 0 || r >= nrows) continue;
      const float w = topk_w[t * k + j];
      Vec<T>::unpack(reinterpret_cast<const uint4*>(y + r * d)[v], tmp);
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < VN; ++i) {
        s += g[i] * tmp[i];
        o[i] = w * g[i];
      }
      dot[j] += s;
      reinterpret_cast<uint4*>(dy + r * d)[v] = Vec<T>::pack(o);
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= k) continue;
    const float s = wave_sum(dot[j]);
    if (lane == 0) d_w[t * k + j] = s;
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

static dim3 token_grid(int64_t T) { return dim3(static_cast<unsigned>((T + 3) / 4)); }

static dim3 elem_grid(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return dim3(static_cast<unsigned>(b));
}

hipError_t launch_permute(const void* x, int dtype, const int32_t* dst_row, int64_t T, int64_t d,
                          int k, int64_t nrows, void* xp, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 0)
    permute_kernel<float><<<token_grid(T), 256, 0, s>>>(static_cast<const float*>(x), dst_row, T, d,
                                                        k, nrows, static_cast<float*>(xp));
  else
    permute_kernel<bf16_t><<<token_grid(T), 256, 0, s>>>(static_cast<const bf16_t*>(x), dst_row, T,
                                                         d, k, nrows, static_cast<bf16_t*>(xp));
  return hipGetLastError();
}

hipError_t launch_permute_bwd(const void* dxp, int dtype, const int32_t* dst_row, int64_t T,
                              int64_t d, int k, int64_t nrows, const void* addend,
                              const float* addend_f32, void* dx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 0)
    permute_bwd_kernel<float><<<token_grid(T), 256, 0, s>>>(
        static_cast<const float*>(dxp), dst_row, T, d, k, nrows,
        static_cast<const float*>(addend), addend_f32, static_cast<float*>(dx));
  else
    permute_bwd_kernel<bf16_t><<<token_grid(T), 256, 0, s>>>(
        static_cast<const bf16_t*>(dxp), dst_row, T, d, k, nrows,
        static_cast<const bf16_t*>(addend), addend_f32, static_cast<bf16_t*>(dx));
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, int dtype, const float* topk_w, const int32_t* dst_row,
                          const void* shared, int64_t T, int64_t d, int k, int64_t nrows,
                          void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 0)
    combine_kernel<float><<<token_grid(T), 256, 0, s>>>(static_cast<const float*>(y), topk_w,
                                                        dst_row, static_cast<const float*>(shared),
                                                        T, d, k, nrows, static_cast<float*>(out));
  else
    combine_kernel<bf16_t><<<token_grid(T), 256, 0, s>>>(
        static_cast<const bf16_t*>(y), topk_w, dst_row, static_cast<const bf16_t*>(shared), T, d,
        k, nrows, static_cast<bf16_t*>(out));
  return hipGetLastError();
}

template <typename T>
static void combine_bwd_dispatch(const T* dout, const T* y, const float* w, const int32_t* dst,
                                 int64_t Tn, int64_t d, int k, int64_t nrows, T* dy, float* dw,
                                 hipStream_t s) {
  const dim3 g = token_grid(Tn);
  if (k <= 2)
    combine_bwd_kernel<T, 2><<<g, 256, 0, s>>>(dout, y, w, dst, Tn, d, k, nrows, dy, dw);
  else if (k <= 4)
    combine_bwd_kernel<T, 4><<<g, 256, 0, s>>>(dout, y, w, dst, Tn, d, k, nrows, dy, dw);
  else if (k <= 8)
    combine_bwd_kernel<T, 8><<<g, 256, 0, s>>>(dout, y, w, dst, Tn, d, k, nrows, dy, dw);
  else if (k <= 16)
    combine_bwd_kernel<T, 16><<<g, 256, 0, s>>>(dout, y, w, dst, Tn, d, k, nrows, dy, dw);
  else if (k <= 32)
    combine_bwd_kernel<T, 32><<<g, 256, 0, s>>>(dout, y, w, dst, Tn, d, k, nrows, dy, dw);
  else
    combine_bwd_kernel<T, 64><<<g, 256, 0, s>>>(dout, y, w, dst, Tn, d, k, nrows, dy, dw);
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
