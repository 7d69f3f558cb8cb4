// Route stage kernels: top-k selection and routing weights (or routing
// replayed from given experts), the per-expert histogram with prefix-sum
// offsets, and the permutation map; plus the backward of the routing weights.
//
// Definition: "Scalable Training of Mixture-of-Experts Models with Megatron
// Core", section 2, Route (logits -> probabilities -> top-k experts, routing
// weights and assignment) and Dispatch (tokens permuted by destination
// expert).  Selection is on the fp32 key (monotone in the probability); equal
// keys go to the lower expert index; segment rows are in ascending token order.
//
// Determinism without order-deciding atomics: tokens are processed in tiles of
// 64; each tile records, per expert, a 64-bit mask of its tokens that chose the
// expert (built with LDS bitwise OR, which is order independent).  A scan over
// tiles gives each (tile, expert) its base row; a token's rank inside its tile
// is the popcount of the mask below its bit.
#include <atomic>

#include "common.h"
#include "internal.h"

namespace moe {

constexpr int ROUTE_TILE = 64;  // tokens per tile = bits of one mask word
// threads of the per-tile selection kernels: 16 waves, 4 tokens each, so the
// serial k-step selection of one token runs on many waves at once
constexpr int ROUTE_THREADS = 1024;
constexpr int ROUTE_WAVES = ROUTE_THREADS / 64;

// Selection-only expert bias (the auxiliary-loss-free biasing that section 7,
// Load Balancing, lists): the key of expert e is sigmoid(z) + b[e]; the
// routing weights stay the unbiased sigmoid scores.  The key decides integer
// results, so the sigmoid is specified step by step, every step one correctly
// rounded fp32 operation (contraction into fused multiply-adds is switched
// off for the function; HIP's __f*_rn helpers are plain operators that the
// default -ffp-contract=fast would fuse):
//   x = clamp(-z, -87, 87); n = rint(x * log2e);
//   r = (x - n * LN2_HI) - n * LN2_LO;  p = Horner of 1/i!, i = 7 .. 0, at r
//   (each step a multiply, then an add);  sigma = 1 / (1 + ldexp(p, n)).
// LN2_HI has 15 significant bits, so n * LN2_HI is exact; the clamp keeps
// exp(x) and sigma normal.
__device__ __forceinline__ float sigmoid_spec(float z) {
#pragma clang fp contract(off)
  constexpr float LOG2E = 1.44269504f, LN2_HI = 0.693145751953125f, LN2_LO = 1.42860677e-06f;
  constexpr float C[8] = {1.0f, 1.0f, 0.5f, 1.0f / 6.0f, 1.0f / 24.0f, 1.0f / 120.0f,
                          1.0f / 720.0f, 1.0f / 5040.0f};
  const float x = fminf(fmaxf(-z, -87.0f), 87.0f);
  const float n = __builtin_rintf(x * LOG2E);
  const float hi = n * LN2_HI;
  const float lo = n * LN2_LO;
  const float r = (x - hi) - lo;
  float p = C[7];
#pragma unroll
  for (int i = 6; i >= 0; --i) {
    const float pr = p * r;
    p = pr + C[i];
  }
  const float e = ldexpf(p, static_cast<int>(n));
  return 1.0f / (1.0f + e);
}

// Strict order on (key, index): larger key first, then lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int EPL>
__global__ __launch_bounds__(ROUTE_THREADS) void topk_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                   int k, int score, int renorm,
                                                   const float* __restrict__ sel_bias,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w,
                                                   unsigned long long* __restrict__ tile_bits) {
  __shared__ unsigned long long bits[1024];
  const int tid = threadIdx.x;
  const int64_t tile = blockIdx.x;
  for (int e = tid; e < E; e += ROUTE_THREADS) bits[e] = 0ull;
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  for (int tt = wave; tt < ROUTE_TILE; tt += ROUTE_WAVES) {
    const int64_t t = tile * ROUTE_TILE + tt;
    if (t >= T) break;
    const float* row = logits + t * E;
    float v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? row[e] : 0.f;
      if (sel_bias && e < E) v[i] = __fadd_rn(sigmoid_spec(v[i]), sel_bias[e]);
    }
    unsigned taken = 0;  // bit i: element i of this lane already selected
    int my_idx = -1;
    float my_key = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = 0.f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !((taken >> i) & 1u) && (bi == 0x7fffffff || better(v[i], e, bv, bi))) {
          bv = v[i];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == j) {
        my_idx = bi;
        my_key = bv;
      }
    }
    // routing weights from the chosen keys (slot 0 holds the largest key)
    const bool active = lane < k;
    float w;
    if (score == 0) {  // softmax
      const float m = __shfl(my_key, 0, 64);
      const float ex = active ? expf(my_key - m) : 0.f;
      float denom;
      if (renorm) {
        denom = wave_sum(ex);
      } else {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i < E) part += expf(v[i] - m);
        denom = wave_sum(part);
      }
      w = ex / denom;
    } else if (sel_bias) {  // sigmoid, biased selection: weights from the logits
      const float s = active ? sigmoid_spec(row[my_idx]) : 0.f;
      w = renorm ? s / wave_sum(s) : s;
    } else {  // sigmoid
      const float s = active ? 1.0f / (1.0f + expf(-my_key)) : 0.f;
      w = renorm ? s / wave_sum(s) : s;
    }
    if (active) {
      topk_idx[t * k + lane] = my_idx;
      topk_w[t * k + lane] = w;
      atomicOr(&bits[my_idx], 1ull << tt);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += ROUTE_THREADS) tile_bits[tile * E + e] = bits[e];
}

// Router replay: the k experts of every token are given, in slot order; the
// routing weights are computed from the logits as in the top-k route.  A slot
// whose expert is outside [0, E) or repeats an earlier slot of the token is
// replaced, in slot order, by the smallest expert the token does not use yet,
// and *status (if given) is set to 1: the dispatch map stays a bijection.
template <int EPL>
__global__ __launch_bounds__(ROUTE_THREADS) void replay_kernel(const float* __restrict__ logits,
                                                     const int32_t* __restrict__ idx_in,
                                                     int64_t T, int E, int k, int score,
                                                     int renorm, int32_t* __restrict__ topk_idx,
                                                     float* __restrict__ topk_w,
                                                     unsigned long long* __restrict__ tile_bits,
                                                     int32_t* __restrict__ status) {
  __shared__ unsigned long long bits[1024];
  const int tid = threadIdx.x;
  const int64_t tile = blockIdx.x;
  for (int e = tid; e < E; e += ROUTE_THREADS) bits[e] = 0ull;
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  for (int tt = wave; tt < ROUTE_TILE; tt += ROUTE_WAVES) {
    const int64_t t = tile * ROUTE_TILE + tt;
    if (t >= T) break;
    const float* row = logits + t * E;
    const bool active = lane < k;
    int my = active ? idx_in[t * k + lane] : -1;
    bool ok = active && my >= 0 && my < E;
    for (int i = 0; i < k; ++i) {
      const int o = __shfl(my, i, 64);
      if (i < lane && o == my) ok = false;
    }
    const unsigned long long bad = __ballot(active && !ok);
    if (bad) {
      for (int j = 0; j < k; ++j) {
        if (!((bad >> j) & 1ull)) continue;  // uniform across the wave
        int best = 0x7fffffff;
        for (int e = lane; e < E; e += 64) {
          bool used = false;
          for (int sl = 0; sl < k; ++sl) {
            const int o = __shfl(my, sl, 64);
            if (sl != j && o == e) used = true;
          }
          if (!used) best = min(best, e);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) best = min(best, __shfl_xor(best, o, 64));
        if (lane == j) my = best;
      }
      if (lane == 0 && status) status[0] = 1;
    }
    const float key = active ? row[my] : 0.f;
    float w;
    if (score == 0) {  // softmax
      float m;
      if (renorm) {
        m = active ? key : -INFINITY;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      } else {
        m = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i < E) m = fmaxf(m, row[lane + 64 * i]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      }
      const float ex = active ? expf(key - m) : 0.f;
      float denom;
      if (renorm) {
        denom = wave_sum(ex);
      } else {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i < E) part += expf(row[lane + 64 * i] - m);
        denom = wave_sum(part);
      }
      w = ex / denom;
    } else {  // sigmoid
      const float sg = active ? 1.0f / (1.0f + expf(-key)) : 0.f;
      w = renorm ? sg / wave_sum(sg) : sg;
    }
    if (active) {
      topk_idx[t * k + lane] = my;
      topk_w[t * k + lane] = w;
      atomicOr(&bits[my], 1ull << tt);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += ROUTE_THREADS) tile_bits[tile * E + e] = bits[e];
}

// One block: per expert, the running row count over tiles (tile_base), the
// totals (counts) and their exclusive prefix sum (offsets).
__global__ __launch_bounds__(1024) void route_scan_kernel(const unsigned long long* __restrict__ tile_bits,
                                                          int64_t ntiles, int E,
                                                          int32_t* __restrict__ tile_base,
                                                          int32_t* __restrict__ counts,
                                                          int64_t* __restrict__ offsets) {
  __shared__ long long s[1024];
  const int e = threadIdx.x;
  long long run = 0;
  if (e < E) {
    for (int64_t tl = 0; tl < ntiles; ++tl) {
      tile_base[tl * E + e] = static_cast<int32_t>(run);
      run += __popcll(tile_bits[tl * E + e]);
    }
    counts[e] = static_cast<int32_t>(run);
  }
  s[e] = e < E ? run : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const long long add = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += add;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = s[e];
  if (e == 0) offsets[0] = 0;
}

__global__ __launch_bounds__(256) void route_rank_kernel(const int32_t* __restrict__ topk_idx,
                                                         const unsigned long long* __restrict__ tile_bits,
                                                         const int32_t* __restrict__ tile_base,
                                                         const int64_t* __restrict__ offsets, int64_t T,
                                                         int E, int k, int32_t* __restrict__ dst_row,
                                                         int32_t* __restrict__ src_token) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= T * k) return;
  const int64_t t = i / k;
  const int e = topk_idx[i];
  if (e < 0 || e >= E) return;
  const int64_t tile = t / ROUTE_TILE;
  const int bit = static_cast<int>(t % ROUTE_TILE);
  const unsigned long long below = bit ? (tile_bits[tile * E + e] & ((1ull << bit) - 1ull)) : 0ull;
  const int64_t r = offsets[e] + tile_base[tile * E + e] + __popcll(below);
  if (r < 0 || r >= T * k) return;
  dst_row[i] = static_cast<int32_t>(r);
  src_token[r] = static_cast<int32_t>(t);
}

// d_logits from d_topk_w: one wave per token.
template <int EPL>
__global__ __launch_bounds__(256) void route_bwd_kernel(const float* __restrict__ logits,
                                                        const int32_t* __restrict__ topk_idx,
                                                        const float* __restrict__ topk_w,
                                                        const float* __restrict__ d_topk_w, int64_t T,
                                                        int E, int k, int score, int renorm,
                                                        float* __restrict__ d_logits) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * E;
  const bool active = lane < k;
  int e_j = active ? topk_idx[t * k + lane] : -1;
  if (e_j >= E) e_j = -1;
  const float w_j = active ? topk_w[t * k + lane] : 0.f;
  const float dw_j = active ? d_topk_w[t * k + lane] : 0.f;
  const float g = wave_sum(w_j * dw_j);
  float dz_j = 0.f;
  if (score == 1) {
    const float z = e_j >= 0 ? row[e_j] : 0.f;
    const float s = 1.0f / (1.0f + expf(-z));
    if (renorm) {
      const float S = wave_sum(active ? s : 0.f);
      dz_j = (dw_j - g) / S * s * (1.0f - s);
    } else {
      dz_j = dw_j * s * (1.0f - s);
    }
  } else if (renorm) {
    dz_j = w_j * (dw_j - g);
  }
  float v[EPL];
  float m = -INFINITY, denom = 0.f;
  if (score == 0 && !renorm) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? row[e] : -INFINITY;
      m = fmaxf(m, v[i]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i < E) part += expf(v[i] - m);
    denom = wave_sum(part);
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    float out = 0.f;
    float G = 0.f;
    bool chosen = false;
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(e_j, j, 64);
      const float dzj = __shfl(dz_j, j, 64);
      const float dwj = __shfl(dw_j, j, 64);
      if (ej == e) {
        chosen = true;
        out = dzj;
        G = dwj;
      }
    }
    if (score == 0 && !renorm) {
      const float p = e < E ? expf(v[i] - m) / denom : 0.f;
      out = p * (G - g);
    } else if (!chosen) {
      out = 0.f;
    }
    if (e < E) d_logits[t * E + e] = out;
  }
}

static int epl_for(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int score, int renorm,
                             const float* sel_bias, int32_t* topk_idx, float* topk_w,
                             int32_t* counts, int64_t* offsets, int32_t* dst_row,
                             int32_t* src_token, void* ws, hipStream_t stream) {
  const int64_t ntiles = (T + ROUTE_TILE - 1) / ROUTE_TILE;
  unsigned long long* tile_bits = static_cast<unsigned long long*>(ws);
  int32_t* tile_base = reinterpret_cast<int32_t*>(tile_bits + ntiles * E);
  if (ntiles > 0) {
    switch (epl_for(E)) {
#define MOE_TOPK(n)                                                                               \
  case n:                                                                                         \
    topk_kernel<n><<<dim3(static_cast<unsigned>(ntiles)), ROUTE_THREADS, 0, stream>>>(                      \
        logits, T, E, k, score, renorm, sel_bias, topk_idx, topk_w, tile_bits);                   \
    break;
      MOE_TOPK(1) MOE_TOPK(2) MOE_TOPK(4) MOE_TOPK(8) MOE_TOPK(16)
#undef MOE_TOPK
    }
  }
  route_scan_kernel<<<1, 1024, 0, stream>>>(tile_bits, ntiles, E, tile_base, counts, offsets);
  if (T > 0) {
    const int64_t n = T * k;
    route_rank_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, stream>>>(
        topk_idx, tile_bits, tile_base, offsets, T, E, k, dst_row, src_token);
  }
  return hipGetLastError();
}

// ---- the allocation-free route -----------------------------------------------
// Scratch of moe_route_topk_noalloc: the tile masks and per-tile row bases
// that moe_route_topk keeps in the caller's workspace, in a fixed array that
// each device holds for the life of the process.  Host code reaches it only
// through the device address hipGetSymbolAddress returns (the array's name on
// the host is not a device address), looked up once per device.
constexpr size_t kRouteScratchBytes = size_t(4) << 20;
__device__ __align__(256) unsigned char scratch[kRouteScratchBytes];

size_t route_noalloc_scratch_bytes() { return kRouteScratchBytes; }

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t route_scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // every caller on this device gets the same address, so a race only repeats the lookup
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_route_replay(const float* logits, const int32_t* idx_in, int64_t T, int E, int k,
                               int score, int renorm, int32_t* topk_idx, float* topk_w,
                               int32_t* counts, int64_t* offsets, int32_t* dst_row,
                               int32_t* src_token, int32_t* status, void* ws, hipStream_t stream) {
  const int64_t ntiles = (T + ROUTE_TILE - 1) / ROUTE_TILE;
  unsigned long long* tile_bits = static_cast<unsigned long long*>(ws);
  int32_t* tile_base = reinterpret_cast<int32_t*>(tile_bits + ntiles * E);
  if (ntiles > 0) {
    switch (epl_for(E)) {
#define MOE_REPLAY(n)                                                                             \
  case n:                                                                                         \
    replay_kernel<n><<<dim3(static_cast<unsigned>(ntiles)), ROUTE_THREADS, 0, stream>>>(                    \
        logits, idx_in, T, E, k, score, renorm, topk_idx, topk_w, tile_bits, status);             \
    break;
      MOE_REPLAY(1) MOE_REPLAY(2) MOE_REPLAY(4) MOE_REPLAY(8) MOE_REPLAY(16)
#undef MOE_REPLAY
    }
  }
  route_scan_kernel<<<1, 1024, 0, stream>>>(tile_bits, ntiles, E, tile_base, counts, offsets);
  if (T > 0) {
    const int64_t n = T * k;
    route_rank_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, stream>>>(
        topk_idx, tile_bits, tile_base, offsets, T, E, k, dst_row, src_token);
  }
  return hipGetLastError();
}

// Capacity-limited dropping on a dropless dispatch map: expert e keeps the
// first C of its rows (its lowest tokens, rows being in ascending token order
// inside a segment); kept rows are renumbered into the new segments, dropped
// (token, slot) pairs get dst_row = -1.
__global__ __launch_bounds__(1024) void capacity_scan_kernel(const int32_t* __restrict__ counts,
                                                             int E, int64_t C,
                                                             int32_t* __restrict__ counts_out,
                                                             int64_t* __restrict__ offsets_out) {
  __shared__ long long s[1024];
  const int e = threadIdx.x;
  const long long kept = e < E ? min(static_cast<long long>(counts[e]), static_cast<long long>(C)) : 0;
  s[e] = kept;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan
    const long long v = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  if (e < E) {
    counts_out[e] = static_cast<int32_t>(kept);
    offsets_out[e + 1] = s[e];
  }
  if (e == 0) offsets_out[0] = 0;
}

__global__ __launch_bounds__(256) void capacity_remap_kernel(
    const int32_t* __restrict__ topk_idx, const int64_t* __restrict__ offsets,
    const int32_t* __restrict__ dst_row, int64_t n, int E, int k, int64_t C,
    const int64_t* __restrict__ offsets_out, int32_t* __restrict__ dst_out,
    int32_t* __restrict__ src_out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int e = topk_idx[i];
  const int64_t r = dst_row[i];
  int32_t out = -1;
  if (e >= 0 && e < E && r >= 0) {
    const int64_t rank = r - offsets[e];
    if (rank >= 0 && rank < C) {
      const int64_t row = offsets_out[e] + rank;
      out = static_cast<int32_t>(row);
      src_out[row] = static_cast<int32_t>(i / k);
    }
  }
  dst_out[i] = out;
}

hipError_t launch_apply_capacity(const int32_t* topk_idx, const int32_t* counts,
                                 const int64_t* offsets, const int32_t* dst_row, int64_t T, int E,
                                 int k, int64_t C, int32_t* counts_out, int64_t* offsets_out,
                                 int32_t* dst_out, int32_t* src_out, hipStream_t stream) {
  capacity_scan_kernel<<<1, 1024, 0, stream>>>(counts, E, C, counts_out, offsets_out);
  const int64_t n = T * k;
  if (n > 0)
    capacity_remap_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, stream>>>(
        topk_idx, offsets, dst_row, n, E, k, C, offsets_out, dst_out, src_out);
  return hipGetLastError();
}

// Auxiliary load-balancing loss L = coeff * E * sum_e f_e P_e, with
// f_e = counts[e] / (T k) and P_e = mean over tokens of the router
// probability p[t, e] (softmax of the keys, or the sigmoid scores normalised
// over the E experts).  One pass: per 64-token tile, the column sums of p
// (fixed order: waves, then lanes) go to part[tile, e]; optionally the
// gradient dL/dz (f held fixed) is added into d_logits:
//   softmax: dz_e = p_e (g_e - sum p g),  sigmoid: dz_e = s_e (1 - s_e) / S (g_e - sum p g),
//   g_e = coeff * E * f_e / T.
template <int EPL>
__global__ __launch_bounds__(256) void aux_loss_kernel(const float* __restrict__ logits,
                                                       const int32_t* __restrict__ counts,
                                                       int64_t T, int E, int k, int score,
                                                       float coeff, float* __restrict__ part,
                                                       float* __restrict__ d_logits) {
  __shared__ float colsum[4][1024];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t tile = blockIdx.x;
  float g[EPL], acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    g[i] = e < E ? coeff * E * (static_cast<float>(counts[e]) / static_cast<float>(T * k)) /
                       static_cast<float>(T)
                 : 0.f;
    acc[i] = 0.f;
  }
  for (int tt = wave; tt < ROUTE_TILE; tt += 4) {
    const int64_t t = tile * ROUTE_TILE + tt;
    if (t >= T) break;
    const float* row = logits + t * E;
    float v[EPL], pr[EPL], sv[EPL];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? row[e] : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    float denom = 0.f;
    if (score == 0) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        pr[i] = lane + 64 * i < E ? expf(v[i] - m) : 0.f;
        denom += pr[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        sv[i] = lane + 64 * i < E ? 1.0f / (1.0f + expf(-v[i])) : 0.f;
        pr[i] = sv[i];
        denom += pr[i];
      }
    }
    denom = wave_sum(denom);
    float pg = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      pr[i] /= denom;
      acc[i] += pr[i];
      pg += pr[i] * g[i];
    }
    if (d_logits) {
      pg = wave_sum(pg);
      float* drow = d_logits + t * E;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e >= E) continue;
        const float dz = score == 0 ? pr[i] * (g[i] - pg)
                                    : sv[i] * (1.0f - sv[i]) / denom * (g[i] - pg);
        drow[e] += dz;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) colsum[wave][e] = acc[i];
  }
  __syncthreads();
  if (part)
    for (int e = tid; e < E; e += 256)
      part[tile * E + e] = ((colsum[0][e] + colsum[1][e]) + colsum[2][e]) + colsum[3][e];
}

// loss = coeff * E * sum_e f_e * (sum_tiles part[tile, e]) / T, fixed order
__global__ __launch_bounds__(1024) void aux_loss_final_kernel(const float* __restrict__ part,
                                                             int64_t ntiles,
                                                             const int32_t* __restrict__ counts,
                                                             int64_t T, int E, int k, float coeff,
                                                             float* __restrict__ loss) {
  __shared__ float s[1024];
  const int e = threadIdx.x;
  float v = 0.f;
  if (e < E) {
    float P = 0.f;
    for (int64_t tl = 0; tl < ntiles; ++tl) P += part[tl * E + e];
    v = (static_cast<float>(counts[e]) / static_cast<float>(T * k)) * (P / static_cast<float>(T));
  }
  s[e] = v;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (e < o) s[e] += s[e + o];
    __syncthreads();
  }
  if (e == 0) loss[0] = coeff * static_cast<float>(E) * s[0];
}

size_t aux_loss_workspace(int64_t T, int E) {
  return static_cast<size_t>((T + ROUTE_TILE - 1) / ROUTE_TILE) * E * sizeof(float) + 256;
}

hipError_t launch_aux_loss(const float* logits, const int32_t* counts, int64_t T, int E, int k,
                           int score, float coeff, float* loss, float* d_logits, void* ws,
                           hipStream_t stream) {
  const int64_t ntiles = (T + ROUTE_TILE - 1) / ROUTE_TILE;
  float* part = loss ? static_cast<float*>(ws) : nullptr;
  if (ntiles > 0) {
    switch (epl_for(E)) {
#define MOE_AUX(n)                                                                        \
  case n:                                                                                 \
    aux_loss_kernel<n><<<dim3(static_cast<unsigned>(ntiles)), 256, 0, stream>>>(         \
        logits, counts, T, E, k, score, coeff, part, d_logits);                           \
    break;
      MOE_AUX(1) MOE_AUX(2) MOE_AUX(4) MOE_AUX(8) MOE_AUX(16)
#undef MOE_AUX
    }
  }
  if (loss)
    aux_loss_final_kernel<<<1, 1024, 0, stream>>>(part, ntiles, counts, T, E, k, coeff, loss);
  return hipGetLastError();
}

size_t route_topk_workspace(int64_t T, int E) {
  const int64_t ntiles = (T + ROUTE_TILE - 1) / ROUTE_TILE;
  return static_cast<size_t>(ntiles) * E * (sizeof(unsigned long long) + sizeof(int32_t)) + 256;
}

hipError_t launch_route_topk_bwd(const float* logits, const int32_t* topk_idx, const float* topk_w,
                                 const float* d_topk_w, int64_t T, int E, int k, int score,
                                 int renorm, float* d_logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((T + 3) / 4));
  switch (epl_for(E)) {
#define MOE_RB(n)                                                                        \
  case n:                                                                                \
    route_bwd_kernel<n><<<grid, 256, 0, stream>>>(logits, topk_idx, topk_w, d_topk_w, T, \
                                                  E, k, score, renorm, d_logits);        \
    break;
    MOE_RB(1) MOE_RB(2) MOE_RB(4) MOE_RB(8) MOE_RB(16)
#undef MOE_RB
  }
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// b[e] += rate * sign(sum(counts) - E * counts[e]): one workgroup; the sum is
// an exact integer reduction, the update one fp32 addition.
__global__ __launch_bounds__(1024) void expert_bias_update_kernel(const int32_t* __restrict__ counts,
                                                                 int E, float rate,
                                                                 float* __restrict__ bias) {
  __shared__ long long part[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long sum = 0;
  for (int e = tid; e < E; e += 1024) sum += counts[e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane == 0) part[wave] = sum;
  __syncthreads();
  long long total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) total += part[w];
  for (int e = tid; e < E; e += 1024) {
    const long long d = total - static_cast<long long>(E) * counts[e];
    const float step = d > 0 ? rate : (d < 0 ? -rate : 0.0f);
    bias[e] = __fadd_rn(bias[e], step);
  }
}

hipError_t launch_expert_bias_update(const int32_t* counts, int E, float rate, float* bias,
                                     hipStream_t stream) {
  expert_bias_update_kernel<<<1, 1024, 0, stream>>>(counts, E, rate, bias);
  return hipGetLastError();
}

// status |= 1 when any of the n values is a NaN or an infinity (exponent
// field all ones).  Only the value 1 is ever written, so concurrent writers
// agree and the result does not depend on their order.
__global__ __launch_bounds__(256) void check_finite_kernel(const float* __restrict__ p, int64_t n,
                                                           int32_t* __restrict__ status) {
  const int64_t nvec = n / 4;
  bool bad = false;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < nvec; i += stride) {
    const uint4 u = reinterpret_cast<const uint4*>(p)[i];
    bad |= ((u.x & 0x7f800000u) == 0x7f800000u) | ((u.y & 0x7f800000u) == 0x7f800000u) |
           ((u.z & 0x7f800000u) == 0x7f800000u) | ((u.w & 0x7f800000u) == 0x7f800000u);
  }
  if (blockIdx.x == 0 && threadIdx.x < n - nvec * 4)
    bad |= (__float_as_uint(p[nvec * 4 + threadIdx.x]) & 0x7f800000u) == 0x7f800000u;
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) *status = 1;
}

// Invariants of a dispatch map (counts, offsets, dst_row, src_token of the
// route, capacity or pad-to-max calls), each violation OR-ed into *status as
// one bit (OR is order-independent, so the word is deterministic):
//   1  offsets[0] != 0, offsets decreasing, a segment shorter than its count,
//      or offsets[E] beyond the rows
//   2  a pair's row outside its expert's filled segment [offsets[e],
//      offsets[e] + counts[e]) (dropped pairs, row -1, are allowed)
//   4  src_token[row] is not the pair's token
//   8  a segment's tokens not in ascending order
//   16 a pair's expert outside [0, E)
// Every index is range-checked before it is dereferenced.
__global__ __launch_bounds__(256) void check_dispatch_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ counts,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ dst_row,
    const int32_t* __restrict__ src_token, int64_t T, int E, int k, int64_t n_rows,
    int32_t* __restrict__ status) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  int bits = 0;
  if (i <= E) {  // per expert (and the end of the offsets)
    const int64_t lo = offsets[i];
    if (i == 0 && lo != 0) bits |= 1;
    if (i == E) {
      if (lo < 0 || lo > n_rows) bits |= 1;
    } else {
      const int64_t hi = offsets[i + 1];
      const int64_t c = counts[i];
      if (c < 0 || lo < 0 || hi < lo || hi - lo < c || hi > n_rows) bits |= 1;
      else
        for (int64_t r = lo + 1; r < lo + c; ++r)
          if (src_token[r] <= src_token[r - 1]) { bits |= 8; break; }
    }
  }
  if (i < T * k) {  // per (token, slot) pair
    const int64_t t = i / k;
    const int e = topk_idx[i];
    const int64_t r = dst_row[i];
    if (e < 0 || e >= E) {
      bits |= 16;
    } else if (r != -1) {
      const int64_t lo = offsets[e], c = counts[e];
      if (r < lo || r >= lo + c || r < 0 || r >= n_rows) bits |= 2;
      else if (src_token[r] != t) bits |= 4;
    }
  }
  if (bits) atomicOr(status, bits);
}

hipError_t launch_check_dispatch(const int32_t* topk_idx, const int32_t* counts,
                                 const int64_t* offsets, const int32_t* dst_row,
                                 const int32_t* src_token, int64_t T, int E, int k, int64_t n_rows,
                                 int32_t* status, hipStream_t stream) {
  const int64_t n = T * k > E + 1 ? T * k : E + 1;
  check_dispatch_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, stream>>>(
      topk_idx, counts, offsets, dst_row, src_token, T, E, k, n_rows, status);
  return hipGetLastError();
}

hipError_t launch_check_finite(const float* p, int64_t n, int32_t* status, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  check_finite_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(p, n, status);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// Pad-to-max (section 7, Load Balancing: static shapes from variable expert
// counts): every expert's segment gets C rows at e * C; a pair keeps its rank
// in the dropless segment (token order) when that rank is below C, else it is
// dropped -- the kept pairs of capacity-limited dropping.
__global__ __launch_bounds__(256) void pad_map_kernel(const int32_t* __restrict__ topk_idx,
                                                      const int64_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ dst_row,
                                                      int64_t n, int E, int64_t C,
                                                      int32_t* __restrict__ dst_row_out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int e = topk_idx[i];
  const int64_t row = dst_row[i];
  int32_t out = -1;
  if (e >= 0 && e < E && row >= 0) {
    const int64_t rank = row - offsets[e];
    if (rank >= 0 && rank < C) out = static_cast<int32_t>(e * C + rank);
  }
  dst_row_out[i] = out;
}

// rows of the padded layout: row e * C + q holds the q-th token of expert e
// while q < min(counts[e], C), else padding (-1)
__global__ __launch_bounds__(256) void pad_rows_kernel(const int32_t* __restrict__ counts,
                                                       const int64_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ src_token,
                                                       int64_t n_in, int E, int64_t C,
                                                       int32_t* __restrict__ counts_out,
                                                       int64_t* __restrict__ offsets_out,
                                                       int32_t* __restrict__ src_token_out) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (r <= E) {
    offsets_out[r] = r * C;
    if (r < E) {
      const int64_t c = counts[r];
      counts_out[r] = static_cast<int32_t>(c < 0 ? 0 : (c < C ? c : C));
    }
  }
  if (r >= static_cast<int64_t>(E) * C) return;
  const int e = static_cast<int>(r / C);
  const int64_t q = r - e * C;
  const int64_t c = counts[e];
  const int64_t src = offsets[e] + q;
  src_token_out[r] = q < c && q < C && src >= 0 && src < n_in ? src_token[src] : -1;
}

hipError_t launch_pad_to_max(const int32_t* topk_idx, const int32_t* counts,
                             const int64_t* offsets, const int32_t* dst_row,
                             const int32_t* src_token, int64_t T, int E, int k, int64_t C,
                             int32_t* counts_out, int64_t* offsets_out, int32_t* dst_row_out,
                             int32_t* src_token_out, hipStream_t stream) {
  const int64_t n = T * k;
  if (n > 0)
    pad_map_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, stream>>>(
        topk_idx, offsets, dst_row, n, E, C, dst_row_out);
  const int64_t rows = static_cast<int64_t>(E) * C;
  const int64_t m = rows > E + 1 ? rows : E + 1;
  pad_rows_kernel<<<dim3(static_cast<unsigned>((m + 255) / 256)), 256, 0, stream>>>(
      counts, offsets, src_token, n, E, C, counts_out, offsets_out, src_token_out);
  return hipGetLastError();
}

}  // namespace moe
