// Shared device helpers for the MI355X (gfx950) sparse-MoE kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 stored as its 16-bit pattern

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 16 bytes moved as one unit (8 bf16 or 4 fp32).
struct alignas(16) vec16 {
  uint32_t w[4];
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte global store at agent scope (sc1).  On MI355X a plain store leaves
// the line dirty in this XCD's L2 until the write-back at the end of the
// kernel, which then runs after the last wave; an agent-scope store writes
// the line through as it is issued, so a pass's output drains while other
// blocks still compute (measured on the 8-expert default layer: expert up
// pass 19.2 -> 17.9 us, down pass 16.0 -> 15.0 us, combine 3.7 -> 3.4 us).
// Same bytes, and the end-of-kernel release still orders them.
// A VALU write to the data VGPRs of a store wider than 8 bytes must come at
// least two wait states after the store on gfx950; the compiler inserts them
// after its own stores but cannot see into inline asm, so the s_nop 1 is part
// of the asm (without it a following VALU may overwrite the data before the
// store reads it, corrupting 16-byte chunks now and then).
__device__ __forceinline__ void store16_agent(void* dst, const vec16& v) {
  const u32x4_t q = {v.w[0], v.w[1], v.w[2], v.w[3]};
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(dst), "v"(q) : "memory");
}

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.  One
// v_cvt_pk_bf16_f32 on gfx950 (checked on MI355X against the integer
// round-to-nearest-even formula over all 2^32 fp32 bit patterns: identical).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

__device__ __forceinline__ void unpack_bf16x8(const vec16& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v.w[i] << 16);
    f[2 * i + 1] = __uint_as_float(v.w[i] & 0xffff0000u);
  }
}

// Two fp32 -> two bf16 in one dword (low half first): one v_cvt_pk_bf16_f32,
// the same rounding as f32_to_bf16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ vec16 pack_bf16x8(const float* f) {
  vec16 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

enum { ACT_RELU = 0, ACT_GELU = 1, ACT_SWISH = 2 };

// GELU(z) = z Phi(z) = 0.5 z (1 + erf(z / sqrt 2)).  Since
// erf(z / sqrt 2) = sign(z) (1 - erfc(|z| / sqrt 2)), this is
//   GELU(z) = max(z, 0) - 0.5 |z| erfc(|z| / sqrt 2).
// erfc(x) for x >= 0 by Abramowitz & Stegun 7.1.26 (t = 1 / (1 + p x),
// erfc = t (a1 + t (a2 + ...)) e^{-x^2}, |error| <= 1.5e-7), evaluated on
// s = z / sqrt(2 ln 2), so that e^{-x^2} = 2^{-s^2} (the hardware exp2) and
// 0.5 |z| = sqrt(ln 2 / 2) |s|, with the polynomial made monic and its
// leading coefficient a5 sqrt(ln 2 / 2) = 2^-L moved into the exponent:
//   GELU(z) = max(z, 0) - |s| t (c0 + t (c1 + t (c2 + t (c3 + t)))) 2^{-(s^2 + L)},
//   t = 1 / (1 + p sqrt(ln 2) |s|),  c_i = a_{i+1} / a5.
// Twelve VALU instructions with the bias add and no constant moves (every
// literal lands in an instruction that takes one), plus two transcendentals.
__device__ __forceinline__ float gelu_erf(float z) {
  const float s = z * 0.84932180028801907f;  // 1 / sqrt(2 ln 2)
  const float as = fabsf(s);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.27273748088f, as, 1.0f));
  float h = t + -1.3690829039f;
  h = fmaf(h, t, 1.3391807712f);
  h = fmaf(h, t, -0.26803776222f);
  h = fmaf(h, t, 0.24008694985f);
  h *= t;
  const float e = __builtin_amdgcn_exp2f(-fmaf(s, s, 0.67840735333f));
  return fmaf(-as, h * e, fmaxf(z, 0.0f));
}

// Swish / SiLU z sigmoid(z) = z / (1 + e^{-z}), with the hardware exp2 and
// reciprocal (each within about 1 ulp).
__device__ __forceinline__ float swish(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * z));
}

__device__ __forceinline__ float apply_act(int act, float z) {
  if (act == ACT_RELU) return fmaxf(z, 0.0f);
  if (act == ACT_GELU) return gelu_erf(z);
  return swish(z);
}

// Compile-time activation (-1: none), for epilogues with no per-element branch.
template <int ACT>
__device__ __forceinline__ float act_static(float z) {
  if constexpr (ACT == ACT_RELU) return fmaxf(z, 0.0f);
  else if constexpr (ACT == ACT_GELU) return gelu_erf(z);
  else if constexpr (ACT == ACT_SWISH) return swish(z);
  else return z;
}

// Exchange with lane ^ M.  Inside a 16-lane row this is DPP (quad permutes for
// M = 1, 2; row rotates for M = 4, 8), a plain VALU move; M = 16, 32 are the
// permlane swaps, also VALU.  Every lane must be active.
template <int M>
__device__ __forceinline__ int xor_lane(int v) {
  if constexpr (M == 1) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    // rotate the row by 4 one way or the other: each lane keeps the rotation
    // that brings it lane ^ 4 (decided from the lane ids themselves)
    const int lid = (int)__lane_id();
    const int a = __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);  // row_ror:4
    const int b = __builtin_amdgcn_update_dpp(0, v, 0x12C, 0xF, 0xF, false);  // row_ror:12
    const int src_a = __builtin_amdgcn_update_dpp(0, lid, 0x124, 0xF, 0xF, false);
    return src_a == (lid ^ 4) ? a : b;
  } else if constexpr (M == 8) {
    return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8 (= lane ^ 8)
  } else if constexpr (M == 16 || M == 32) {
    // gfx950 lane swaps: permlane16_swap(v, v) leaves rows 0, 2 with their own
    // value in the first result and row 1, 3's in the second (and the other
    // way round on rows 1, 3); permlane32_swap likewise for the two halves
    const auto p = M == 16 ? __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false)
                           : __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)(((int)__lane_id() & M) ? p[0] : p[1]);
  } else {
    return __shfl_xor(v, M, 64);
  }
}

template <int M>
__device__ __forceinline__ double xor_lane_d(double v) {
  const long long u = __double_as_longlong(v);
  const int lo = xor_lane<M>((int)(u & 0xffffffffll));
  const int hi = xor_lane<M>((int)(u >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
