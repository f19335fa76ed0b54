// Measurement support: the on-chip ceilings the layer's kernels are compared
// with, taken on the machine that runs them.
//  * copy: dst = src over `bytes`, 16-byte vector loads and stores, eight
//    vectors a thread in flight, grid-stride over many blocks;
//  * read: the same loads folded into one xor (no store but a guarded
//    one-word write that never fires for real data), a streaming-read ceiling;
//  * mfma: every wave runs independent chains of v_mfma_f32_32x32x16_bf16 on
//    register operands, a dense bf16 ceiling.
// The launch shapes are the fastest measured on MI355X over blocks, vectors in
// flight and MFMA shape (the 16 x 16 x 32 form peaks near half the rate of the
// 32 x 32 x 16 one).
// None of this is the layer's arithmetic.

#include "moe_calib.h"

#include <hip/hip_runtime.h>

#include "common.h"

namespace moe {

constexpr int kCalibThreads = 256;
constexpr int kCalibUnroll = 8;

__global__ __launch_bounds__(kCalibThreads) void calib_copy_kernel(const vec16* __restrict__ src,
                                                                   vec16* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kCalibThreads;
  int64_t i = (int64_t)blockIdx.x * kCalibThreads + threadIdx.x;
  for (; i + (kCalibUnroll - 1) * stride < n; i += kCalibUnroll * stride) {
    vec16 v[kCalibUnroll];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kCalibThreads) void calib_read_kernel(const vec16* __restrict__ src, int64_t n,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kCalibThreads;
  int64_t i = (int64_t)blockIdx.x * kCalibThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kCalibUnroll - 1) * stride < n; i += kCalibUnroll * stride) {
    vec16 v[kCalibUnroll];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) acc ^= v[u].w[0] ^ v[u].w[1] ^ v[u].w[2] ^ v[u].w[3];
  }
  for (; i < n; i += stride) acc ^= src[i].w[0] ^ src[i].w[1] ^ src[i].w[2] ^ src[i].w[3];
  if (acc == 0x9e3779b9u) *sink = acc;  // keeps the loads; data never hits it by design of the caller
}

constexpr int kCalibChains = 4;  // independent accumulators a wave

__global__ __launch_bounds__(kCalibThreads) void calib_mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
  }
  f32x16_t acc[kCalibChains];
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kCalibChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kCalibChains; ++c) s += acc[c][0] + acc[c][15];
  if (s < -1.0f) *sink = s;  // never true (non-negative operands); keeps the chains
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || bytes % 16 != 0) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return MOE_ERR_INVALID_ARG;
  if (bytes == 0) return MOE_OK;
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t want = (n + kCalibThreads * kCalibUnroll - 1) / (kCalibThreads * kCalibUnroll);
  const unsigned blocks = (unsigned)(want < 32768 ? want : 32768);
  hipLaunchKernelGGL(calib_copy_kernel, dim3(blocks), dim3(kCalibThreads), 0, stream, (const vec16*)src,
                     (vec16*)dst, n);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_calib_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || bytes % 16 != 0 || ((uintptr_t)src & 15u)) return MOE_ERR_INVALID_ARG;
  if (bytes == 0) return MOE_OK;
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t want = (n + kCalibThreads * kCalibUnroll - 1) / (kCalibThreads * kCalibUnroll);
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(calib_read_kernel, dim3(blocks), dim3(kCalibThreads), 0, stream, (const vec16*)src, n,
                     sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_calib_mfma(int32_t blocks, int32_t iters, float* sink, double* flops, hipStream_t stream) {
  if (blocks < 1 || iters < 1 || sink == nullptr || flops == nullptr) return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)blocks), dim3(kCalibThreads), 0, stream, iters, sink);
  // 2 * 32 * 32 * 16 flops per MFMA, kCalibChains a wave per iteration
  *flops = (double)blocks * (kCalibThreads / 64) * (double)iters * kCalibChains * (2.0 * 32 * 32 * 16);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
