// Internal helpers shared by the HIP kernels of the MoE hot path (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (gfx950's v_cvt_pk_bf16_f32;
// a NaN stays a NaN).  Branch-free: no per-element divergence in epilogues.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));

// two fp32 -> two bf16 in one 32-bit word (a in the low half), one instruction
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const f32x2_cvt_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt_t));
}

// Element-type traits: load/store one element as fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Sigmoid and SiLU in fp32.
__device__ __forceinline__ float sigmoid_f32(float a) { return 1.0f / (1.0f + __expf(-a)); }

// Wave64 sum with a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace moe
