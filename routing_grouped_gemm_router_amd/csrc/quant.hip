// FP8 E4M3 block quantizers for the fp8 expert GEMMs.
//
// Granularity from "Scalable Training of Mixture-of-Experts Models with
// Megatron Core", section 5, Platform-specific recipes (blockwise FP8): 1 x 128
// tiles for activations and gradients, 128 x 128 blocks for weights; the
// weight gradients contract over tokens, so their operands use 128-token x 1
// tiles with each expert's rows zero-padded to a multiple of 128.
//
// Codes: OCP E4M3 ("FN": bias 7, no infinities, 448 the largest finite).
// Per block: amax = max |v|; scale = amax / 448 and inv = 448 / amax (one IEEE
// fp32 division each; 1 and 1 when amax = 0); code = nearest E4M3 value of
// v * inv, ties to the even code, saturated to +-448.
//
// MXFP8 (the same section's microscaling recipe, in the OCP Microscaling
// Formats encoding): 1 x 32 blocks along each operand's contraction axis, one
// E8M0 scale 2^X per block with X = floor(log2 amax) - 8 clamped to
// [-127, 127] (8 = exponent of E4M3's largest power of two), stored as the
// byte X + 127; code = nearest E4M3 value of v * 2^-X (an exact scaling),
// ties to even, saturated to +-448.  Layouts (codes as for the fp8 GEMM,
// scale bytes contiguous along each row's blocks):
//   rows         q [M, K],           bytes [M, K/32]
//   weights      qf [G, N, K] with bf [G, N, K/32]   (blocks along k)
//                qd [G, K, N] with bd [G, K, N/32]   (blocks along n)
//   token tiles  qT [K, ldm],        bytes [K, ldm/32] (32-token blocks)
// The row and token-tile quantizers can gather their rows through a row map
// (the permutation's src_token), so that the permuted bf16 activations are
// never written.
//
// Output layouts are chosen for the fp8 GEMM, which reads every scale as a
// contiguous vector over a tile's rows and every operand k-contiguous except
// the forward's weights (read transposed through LDS):
//   rows         q [M, K],           scales [K/128, M]
//   weights      q [G, K, N] (w's own layout, both GEMMs) with
//                sf [G, K/128, N] (forward) and sd [G, N/128, K] (dgrad):
//                one 128 x 128 block scale, repeated along the block's rows
//   token tiles  qT [K, ldm],        scales [ldm/128, K], rows of group g at
//                padded offsets poff[g] .. poff[g+1]-1
#include "common.h"
#include "internal.h"

namespace moe {

// Nearest E4M3 codes of finite fp32 values, ties to the even code, saturated
// to +-448: gfx950's v_cvt_pk_fp8_f32 (OCP E4M3FN, round to nearest even,
// subnormals kept) after a clamp to +-448, so that nothing overflows.  Checked
// equal, on every finite fp32 value, to an encoder written from the format's
// definition (sign; for |v| < 2^-6 the subnormal step 2^-9; else 3 mantissa
// bits at the value's binade, a carry into the next binade, saturation).
__device__ __forceinline__ float e4m3_clamp(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// four codes in one dword, byte i from v[i]
__device__ __forceinline__ uint32_t e4m3_encode4(float v0, float v1, float v2, float v3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(v0), e4m3_clamp(v1), 0, false);
  return static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(v2), e4m3_clamp(v3), lo, true));
}

__device__ __forceinline__ void block_scale(float amax, float& scale, float& inv) {
  if (amax == 0.0f) {
    scale = 1.0f;
    inv = 1.0f;
  } else {
    scale = __fdiv_rn(amax, 448.0f);
    inv = __fdiv_rn(448.0f, amax);
  }
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// an 8-byte store with the non-temporal hint: for the blockwise weight codes
// (16 lanes write a 128-byte run of one row) 2 % faster than a plain store;
// the MXFP8 weight quantizer's 32-byte runs take twice as long with it
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store8_nt(uint8_t* p, uint2 v) {
  u32x2_t x;
  x.x = v.x;
  x.y = v.y;
  __builtin_nontemporal_store(x, reinterpret_cast<u32x2_t*>(p));
}

__device__ __forceinline__ uint2 encode8(const float (&f)[8], float inv) {
  return make_uint2(e4m3_encode4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv),
                    e4m3_encode4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv));
}

// ---- 1 x 128 tiles along rows: 16 lanes per block, 4 blocks per wave -------
__global__ __launch_bounds__(256) void quant_rows_kernel(const bf16_t* __restrict__ x, int64_t M,
                                                         int64_t K, uint8_t* __restrict__ q,
                                                         float* __restrict__ sT) {
  const int64_t nb = K / 128;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t chunks = (nb + 3) / 4;
  const int64_t row = wid / chunks;
  if (row >= M) return;
  const int64_t b = (wid % chunks) * 4 + (lane >> 4);
  const bool active = b < nb;
  float f[8] = {};
  float amax = 0.f;
  const int64_t off = row * K + b * 128 + (lane & 15) * 8;
  if (active) {
    unpack8(*reinterpret_cast<const uint4*>(x + off), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  float scale, inv;
  block_scale(amax, scale, inv);
  if (active) {
    *reinterpret_cast<uint2*>(q + off) = encode8(f, inv);
    if ((lane & 15) == 0) sT[b * M + row] = scale;
  }
}

// ---- 128 x 128 weight blocks --------------------------------------------------
// One code layout serves both GEMMs: the data gradient reads w's own layout
// k-contiguous, the forward reads it transposed through LDS.  The block scale
// is written expanded along each GEMM's output columns.
__global__ __launch_bounds__(256) void quant_weights_kernel(const bf16_t* __restrict__ w, int G,
                                                            int64_t K, int64_t N,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ sf,
                                                            float* __restrict__ sd) {
  __shared__ float red[4];
  const int64_t nkb = K / 128, nnb = N / 128;
  const int64_t blk = blockIdx.x;
  const int64_t g = blk / (nkb * nnb);
  const int64_t kb = (blk / nnb) % nkb, nb = blk % nnb;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c8 = (t & 15) * 8, r8 = (t >> 4) * 8;  // 8 columns x 8 rows per thread
  const int64_t base = (g * K + kb * 128) * N + nb * 128;
  float f[8][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    unpack8(*reinterpret_cast<const uint4*>(w + base + (r8 + i) * N + c8), f[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[i][j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float scale, inv;
  block_scale(amax, scale, inv);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    store8_nt(q + base + (r8 + i) * N + c8, encode8(f[i], inv));
  if (t < 128) {
    sf[(g * nkb + kb) * N + nb * 128 + t] = scale;
    sd[(g * nnb + nb) * K + kb * 128 + t] = scale;
  }
}

// ---- padded group offsets ---------------------------------------------------------
__global__ __launch_bounds__(1024) void padded_offsets_kernel(const int64_t* __restrict__ off, int G,
                                                              int64_t M, int64_t align,
                                                              int64_t* __restrict__ poff) {
  __shared__ int64_t s[1024];
  const int g = threadIdx.x;
  int64_t n = 0;
  if (g < G) {
    int64_t lo = off[g], hi = off[g + 1];
    lo = lo < 0 ? 0 : (lo > M ? M : lo);
    hi = hi < lo ? lo : (hi > M ? M : hi);
    n = (hi - lo + align - 1) / align * align;
  }
  s[g] = n;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int64_t add = g >= o ? s[g - o] : 0;
    __syncthreads();
    s[g] += add;
    __syncthreads();
  }
  if (g < G) poff[g + 1] = s[g];
  if (g == 0) poff[0] = 0;
}

// ---- 128-token x 1 tiles, padded per group, written transposed --------------
// One workgroup per (padded 128-row block, 128 columns).
__global__ __launch_bounds__(256) void quant_token_tiles_kernel(
    const bf16_t* __restrict__ x, const int64_t* __restrict__ off,
    const int64_t* __restrict__ poff, int G, int64_t M, int64_t K, int64_t ldm,
    uint8_t* __restrict__ qT, float* __restrict__ s) {
  __shared__ uint8_t tile[128][128 + 8];
  __shared__ float cmax[16][128];
  const int64_t rb = blockIdx.y;               // padded row block
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 128;
  const int64_t prow0 = rb * 128;
  if (prow0 >= poff[G]) return;
  // the group whose padded range holds this block
  int lo_g = 0, hi_g = G;
  while (hi_g - lo_g > 1) {
    const int mid = (lo_g + hi_g) >> 1;
    if (poff[mid] <= prow0) lo_g = mid; else hi_g = mid;
  }
  int64_t glo = off[lo_g], ghi = off[lo_g + 1];
  glo = glo < 0 ? 0 : (glo > M ? M : glo);
  ghi = ghi < glo ? glo : (ghi > M ? M : ghi);
  const int64_t row0 = glo + (prow0 - poff[lo_g]);  // first source row of the block
  const int64_t nvalid = min<int64_t>(128, ghi - row0);
  const int t = threadIdx.x;
  const int c8 = (t & 15) * 8, r8 = (t >> 4) * 8;
  float f[8][8];
  float mx[8] = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (r8 + i < nvalid) {
      unpack8(*reinterpret_cast<const uint4*>(x + (row0 + r8 + i) * K + c0 + c8), f[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[i][j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) mx[j] = fmaxf(mx[j], fabsf(f[i][j]));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) cmax[t >> 4][c8 + j] = mx[j];
  __syncthreads();
  float inv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float a = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) a = fmaxf(a, cmax[r][c8 + j]);
    float sc;
    block_scale(a, sc, inv[j]);
    if ((t >> 4) == 0) s[rb * K + c0 + c8 + j] = sc;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint2*>(&tile[r8 + i][c8]) = make_uint2(
        e4m3_encode4(f[i][0] * inv[0], f[i][1] * inv[1], f[i][2] * inv[2], f[i][3] * inv[3]),
        e4m3_encode4(f[i][4] * inv[4], f[i][5] * inv[5], f[i][6] * inv[6], f[i][7] * inv[7]));
  __syncthreads();
  // transposed store: column c holds this block's 128 token codes
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = (t >> 4) * 8 + i;
    const int r0 = (t & 15) * 8;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= static_cast<uint32_t>(tile[r0 + j][c]) << (8 * j);
      hi |= static_cast<uint32_t>(tile[r0 + 4 + j][c]) << (8 * j);
    }
    *reinterpret_cast<uint2*>(qT + (c0 + c) * ldm + prow0 + r0) = make_uint2(lo, hi);
  }
}

// ---- MXFP8 -------------------------------------------------------------------

// E8M0 byte of a block whose largest magnitude is amax: with e the biased
// exponent field of amax, floor(log2 amax) = e - 127 for normal amax, so the
// byte X + 127 is e - 8; zero and subnormal amax (e = 0) and e < 8 clamp to
// X = -127, byte 0.
__device__ __forceinline__ uint32_t mx_byte(float amax) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);
  return static_cast<uint32_t>(e > 8 ? e - 8 : 0);
}

// codes of v * 2^-X = v * 2^(127 - byte), an exact power-of-two scaling
__device__ __forceinline__ uint2 encode8_mx(const float (&f)[8], uint32_t byte) {
  const int e = 127 - static_cast<int>(byte);
  return make_uint2(
      e4m3_encode4(ldexpf(f[0], e), ldexpf(f[1], e), ldexpf(f[2], e), ldexpf(f[3], e)),
      e4m3_encode4(ldexpf(f[4], e), ldexpf(f[5], e), ldexpf(f[6], e), ldexpf(f[7], e)));
}

// bf16 row `r` of the quantizer's input, through the row map if there is one;
// a map entry outside [0, x_rows) reads as a zero row
__device__ __forceinline__ void load_row8(const bf16_t* __restrict__ x, int64_t x_rows,
                                          const int32_t* __restrict__ src, int64_t r, int64_t K,
                                          int64_t col, float (&f)[8]) {
  const int64_t sr = src ? static_cast<int64_t>(src[r]) : r;
  if (sr >= 0 && sr < x_rows) {
    unpack8(*reinterpret_cast<const uint4*>(x + sr * K + col), f);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = 0.f;
  }
}

// 1 x 32 blocks along rows: one lane per 8 elements, 4 lanes per block, 16
// lanes per 128 elements (whose 4 scale bytes go out as one dword).  Rows at
// and past *rows_end (when given) are not written.
__global__ __launch_bounds__(256) void quant_mx_rows_kernel(
    const bf16_t* __restrict__ x, int64_t x_rows, const int32_t* __restrict__ src,
    const int64_t* __restrict__ rows_end, int64_t M, int64_t K, uint8_t* __restrict__ q,
    uint8_t* __restrict__ e) {
  const int64_t per_row = K / 8;  // a multiple of 16
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = idx / per_row;
  const int64_t c = idx - row * per_row;
  int64_t end = M;
  if (rows_end) {
    const int64_t v = *rows_end;
    end = v < 0 ? 0 : (v > M ? M : v);
  }
  const bool live = row < end;  // uniform over each 16-lane run (one row)
  float f[8] = {};
  if (live) load_row8(x, x_rows, src, row, K, c * 8, f);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const uint32_t b = mx_byte(amax);
  if (live) *reinterpret_cast<uint2*>(q + row * K + c * 8) = encode8_mx(f, b);
  const int base = static_cast<int>(threadIdx.x & 63) & ~15;
  const uint32_t w = __shfl(b, base, 64) | (__shfl(b, base + 4, 64) << 8) |
                     (__shfl(b, base + 8, 64) << 16) | (__shfl(b, base + 12, 64) << 24);
  if (live && (c & 15) == 0) *reinterpret_cast<uint32_t*>(e + row * (K / 32) + c / 4) = w;
}

// The same 1 x 32 row blocks in token order: token t is read and quantized
// once, and its codes and scale dword go to each of its k dispatch rows
// dst_row[t k + j] that lies in [0, min(M, *rows_end)) (a dropped slot, -1,
// is skipped).  Lane layout as above, so a 16-lane run shares one token.
__global__ __launch_bounds__(256) void quant_mx_scatter_kernel(
    const bf16_t* __restrict__ x, int64_t T, int64_t K, const int32_t* __restrict__ dst_row, int k,
    const int64_t* __restrict__ rows_end, int64_t M, uint8_t* __restrict__ q,
    uint8_t* __restrict__ e) {
  const int64_t per_row = K / 8;  // a multiple of 16
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t t = idx / per_row;
  const int64_t c = idx - t * per_row;
  const bool live = t < T;
  float f[8] = {};
  if (live) unpack8(*reinterpret_cast<const uint4*>(x + t * K + c * 8), f);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const uint32_t b = mx_byte(amax);
  const int base = static_cast<int>(threadIdx.x & 63) & ~15;
  const uint32_t w = __shfl(b, base, 64) | (__shfl(b, base + 4, 64) << 8) |
                     (__shfl(b, base + 8, 64) << 16) | (__shfl(b, base + 12, 64) << 24);
  if (!live) return;
  int64_t end = M;
  if (rows_end) {
    const int64_t v = *rows_end;
    end = v < 0 ? 0 : (v > M ? M : v);
  }
  const uint2 codes = encode8_mx(f, b);
  const int32_t* d = dst_row + t * k;
  for (int j = 0; j < k; ++j) {
    const int64_t r = d[j];
    if (r < 0 || r >= end) continue;
    *reinterpret_cast<uint2*>(q + r * K + c * 8) = codes;
    if ((c & 15) == 0) *reinterpret_cast<uint32_t*>(e + r * (K / 32) + c / 4) = w;
  }
}

// 128 x 128 tile of one expert's w [K, N], quantized twice: 32-column blocks
// of each row for dgrad (4 neighbouring lanes), 32-row blocks of each column
// for the forward (one wave holds 32 rows).  A thread holds 8 rows x 8
// columns, so its forward codes are already transposed: column c8 + j's
// codes of rows r8 .. r8 + 7 are one 8-byte run of the forward layout's row.
__global__ __launch_bounds__(256) void quant_mx_weights_kernel(
    const bf16_t* __restrict__ w, int G, int64_t K, int64_t N, uint8_t* __restrict__ qf,
    uint8_t* __restrict__ ef, uint8_t* __restrict__ qd, uint8_t* __restrict__ ed) {
  __shared__ uint8_t kbyte[4][128];  // forward: per 32-row block, per column
  __shared__ uint8_t nbyte[128][4];  // dgrad: per row, per 32-column block
  const int64_t nkb = K / 128, nnb = N / 128;
  const int64_t blk = blockIdx.x;
  const int64_t g = blk / (nkb * nnb);
  const int64_t kb = (blk / nnb) % nkb, nb = blk % nnb;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c8 = (t & 15) * 8, r8 = (t >> 4) * 8;  // 8 columns x 8 rows per thread
  const bf16_t* src = w + (g * K + kb * 128) * N + nb * 128;
  float f[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) unpack8(*reinterpret_cast<const uint4*>(src + (r8 + i) * N + c8), f[i]);
  // dgrad operand: blocks of 32 columns
  uint8_t* dq = qd + (g * K + kb * 128) * N + nb * 128;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float am = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(f[i][j]));
    am = fmaxf(am, __shfl_xor(am, 1, 64));
    am = fmaxf(am, __shfl_xor(am, 2, 64));
    const uint32_t b = mx_byte(am);
    *reinterpret_cast<uint2*>(dq + (r8 + i) * N + c8) = encode8_mx(f[i], b);
    if ((t & 3) == 0) nbyte[r8 + i][(t & 15) >> 2] = static_cast<uint8_t>(b);
  }
  // forward operand: blocks of 32 rows, row n of qf holds this tile's k codes
  uint8_t* fq = qf + (g * N + nb * 128 + c8) * K + kb * 128 + r8;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(f[i][j]));
    am = fmaxf(am, __shfl_xor(am, 16, 64));
    am = fmaxf(am, __shfl_xor(am, 32, 64));
    const uint32_t b = mx_byte(am);
    if (lane < 16) kbyte[wave][c8 + j] = static_cast<uint8_t>(b);
    const int ex = 127 - static_cast<int>(b);  // the exact scaling 2^-X
    *reinterpret_cast<uint2*>(fq + static_cast<int64_t>(j) * K) = make_uint2(
        e4m3_encode4(ldexpf(f[0][j], ex), ldexpf(f[1][j], ex), ldexpf(f[2][j], ex),
                     ldexpf(f[3][j], ex)),
        e4m3_encode4(ldexpf(f[4][j], ex), ldexpf(f[5][j], ex), ldexpf(f[6][j], ex),
                     ldexpf(f[7][j], ex)));
  }
  __syncthreads();
  if (t < 128) {
    const uint32_t wf = kbyte[0][t] | (kbyte[1][t] << 8) | (kbyte[2][t] << 16) |
                        (static_cast<uint32_t>(kbyte[3][t]) << 24);
    *reinterpret_cast<uint32_t*>(ef + (g * N + nb * 128 + t) * (K / 32) + kb * 4) = wf;
    const uint32_t wd = nbyte[t][0] | (nbyte[t][1] << 8) | (nbyte[t][2] << 16) |
                        (static_cast<uint32_t>(nbyte[t][3]) << 24);
    *reinterpret_cast<uint32_t*>(ed + (g * K + kb * 128 + t) * (N / 32) + nb * 4) = wd;
  }
}

// 32-token x 1 blocks, groups padded to 128 rows, written transposed.  One
// workgroup per (padded 128-row block, 128 columns); wave w holds the block's
// rows 32 w .. 32 w + 31.
__global__ __launch_bounds__(256) void quant_mx_token_tiles_kernel(
    const bf16_t* __restrict__ x, int64_t x_rows, const int32_t* __restrict__ src,
    const int64_t* __restrict__ off, const int64_t* __restrict__ poff, int G, int64_t M, int64_t K,
    int64_t ldm, uint8_t* __restrict__ qT, uint8_t* __restrict__ eT) {
  __shared__ uint8_t tile[128][128 + 8];
  __shared__ uint8_t kbyte[4][128];
  const int64_t rb = blockIdx.y;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 128;
  const int64_t prow0 = rb * 128;
  if (prow0 >= poff[G]) return;
  int lo_g = 0, hi_g = G;
  while (hi_g - lo_g > 1) {
    const int mid = (lo_g + hi_g) >> 1;
    if (poff[mid] <= prow0) lo_g = mid; else hi_g = mid;
  }
  int64_t glo = off[lo_g], ghi = off[lo_g + 1];
  glo = glo < 0 ? 0 : (glo > M ? M : glo);
  ghi = ghi < glo ? glo : (ghi > M ? M : ghi);
  const int64_t row0 = glo + (prow0 - poff[lo_g]);
  const int64_t nvalid = min<int64_t>(128, ghi - row0);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c8 = (t & 15) * 8, r8 = (t >> 4) * 8;
  float f[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (r8 + i < nvalid) {
      load_row8(x, x_rows, src, row0 + r8 + i, K, c0 + c8, f[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[i][j] = 0.f;
    }
  }
  int ex[8];  // per column: 127 - byte, the exponent of the exact scaling
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(f[i][j]));
    am = fmaxf(am, __shfl_xor(am, 16, 64));
    am = fmaxf(am, __shfl_xor(am, 32, 64));
    const uint32_t b = mx_byte(am);
    ex[j] = 127 - static_cast<int>(b);
    if (lane < 16) kbyte[wave][c8 + j] = static_cast<uint8_t>(b);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint2*>(&tile[r8 + i][c8]) = make_uint2(
        e4m3_encode4(ldexpf(f[i][0], ex[0]), ldexpf(f[i][1], ex[1]), ldexpf(f[i][2], ex[2]),
                     ldexpf(f[i][3], ex[3])),
        e4m3_encode4(ldexpf(f[i][4], ex[4]), ldexpf(f[i][5], ex[5]), ldexpf(f[i][6], ex[6]),
                     ldexpf(f[i][7], ex[7])));
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = (t >> 4) * 8 + i;
    const int r0 = (t & 15) * 8;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= static_cast<uint32_t>(tile[r0 + j][c]) << (8 * j);
      hi |= static_cast<uint32_t>(tile[r0 + 4 + j][c]) << (8 * j);
    }
    *reinterpret_cast<uint2*>(qT + (c0 + c) * ldm + prow0 + r0) = make_uint2(lo, hi);
  }
  if (t < 128) {
    const uint32_t wv = kbyte[0][t] | (kbyte[1][t] << 8) | (kbyte[2][t] << 16) |
                        (static_cast<uint32_t>(kbyte[3][t]) << 24);
    *reinterpret_cast<uint32_t*>(eT + (c0 + t) * (ldm / 32) + prow0 / 32) = wv;
  }
}

hipError_t launch_quant_mx_rows(const void* x, int64_t x_rows, const int32_t* src,
                                const int64_t* rows_end, int64_t M, int64_t K, uint8_t* q,
                                uint8_t* e, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t threads = M * (K / 8);
  quant_mx_rows_kernel<<<dim3(static_cast<unsigned>((threads + 255) / 256)), 256, 0, s>>>(
      static_cast<const bf16_t*>(x), x_rows, src, rows_end, M, K, q, e);
  return hipGetLastError();
}

hipError_t launch_quant_mx_scatter(const void* x, int64_t T, int64_t K, const int32_t* dst_row,
                                   int k, const int64_t* rows_end, int64_t M, uint8_t* q,
                                   uint8_t* e, hipStream_t s) {
  if (T == 0 || M == 0) return hipSuccess;
  const int64_t threads = T * (K / 8);
  quant_mx_scatter_kernel<<<dim3(static_cast<unsigned>((threads + 255) / 256)), 256, 0, s>>>(
      static_cast<const bf16_t*>(x), T, K, dst_row, k, rows_end, M, q, e);
  return hipGetLastError();
}

hipError_t launch_quant_mx_weights(const void* w, int G, int64_t K, int64_t N, uint8_t* qf,
                                   uint8_t* ef, uint8_t* qd, uint8_t* ed, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(G) * (K / 128) * (N / 128);
  if (blocks == 0) return hipSuccess;
  quant_mx_weights_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(
      static_cast<const bf16_t*>(w), G, K, N, qf, ef, qd, ed);
  return hipGetLastError();
}

hipError_t launch_quant_mx_token_tiles(const void* x, int64_t x_rows, const int32_t* src,
                                       const int64_t* off, const int64_t* poff, int G, int64_t M,
                                       int64_t K, int64_t ldm, uint8_t* qT, uint8_t* eT,
                                       hipStream_t st) {
  if (ldm == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(K / 128), static_cast<unsigned>(ldm / 128));
  quant_mx_token_tiles_kernel<<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(x), x_rows, src,
                                                    off, poff, G, M, K, ldm, qT, eT);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, int64_t M, int64_t K, uint8_t* q, float* sT,
                             hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t waves = M * ((K / 128 + 3) / 4);
  quant_rows_kernel<<<dim3(static_cast<unsigned>((waves + 3) / 4)), 256, 0, s>>>(
      static_cast<const bf16_t*>(x), M, K, q, sT);
  return hipGetLastError();
}

hipError_t launch_quant_weights(const void* w, int G, int64_t K, int64_t N, uint8_t* q, float* sf,
                                float* sd, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(G) * (K / 128) * (N / 128);
  if (blocks == 0) return hipSuccess;
  quant_weights_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(
      static_cast<const bf16_t*>(w), G, K, N, q, sf, sd);
  return hipGetLastError();
}

hipError_t launch_padded_offsets(const int64_t* off, int G, int64_t M, int64_t align,
                                 int64_t* poff, hipStream_t s) {
  padded_offsets_kernel<<<1, 1024, 0, s>>>(off, G, M, align, poff);
  return hipGetLastError();
}

hipError_t launch_quant_token_tiles(const void* x, const int64_t* off, const int64_t* poff, int G,
                                    int64_t M, int64_t K, int64_t ldm, uint8_t* qT, float* s,
                                    hipStream_t st) {
  if (ldm == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(K / 128), static_cast<unsigned>(ldm / 128));
  quant_token_tiles_kernel<<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(x), off, poff, G, M, K,
                                                 ldm, qT, s);
  return hipGetLastError();
}

}  // namespace moe
