// Shared device helpers for the MI355X (gfx950) sparse-MoE kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 stored as its 16-bit pattern

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes moved as one unit (8 bf16 or 4 fp32).
struct alignas(16) vec16 {
  uint32_t w[4];
};

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ void unpack_bf16x8(const vec16& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v.w[i] << 16);
    f[2 * i + 1] = __uint_as_float(v.w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ vec16 pack_bf16x8(const float* f) {
  vec16 v;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v.w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  return v;
}

enum { ACT_RELU = 0, ACT_GELU = 1, ACT_SWISH = 2 };

__device__ __forceinline__ float apply_act(int act, float z) {
  if (act == ACT_RELU) return fmaxf(z, 0.0f);
  if (act == ACT_GELU) return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
  return z / (1.0f + expf(-z));  // swish / SiLU
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
