// Gate-weighted combine (the un-scatter of the dispatch).
//
// y[t] = sum_{j: row(t,j) >= 0} g[t,j] * expert_out[row(t,j)]  (+ shared_out[t])
// Page "Code Walkthrough -- SER", the gating / routing path: the expert outputs
// are combined, weighted by the gate weights; page "Appendix C -- Acronyms &
// Symbols", Capacity & communication: the combine tensor is the gate-weighted
// un-scatter, and Parameter accounting: shared experts are always on (weight 1).
// Dropped choices add nothing.  fp32 accumulation in fixed j order, then the
// shared term, then one rounding of the result.
//
// One wavefront per token; lanes stride the row in 16-byte vectors.  Lane j < k
// fetches (row, gate) of choice j once into LDS for the whole wave.

#include "common.h"
#include "internal.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const vec16* __restrict__ yd,
                                                      const int32_t* __restrict__ row,
                                                      const float* __restrict__ gate,
                                                      const vec16* __restrict__ ysh, int64_t T,
                                                      int k, int64_t vpr, vec16* __restrict__ y) {
  constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte vector
  __shared__ int s_row[4][kMaxTopK];
  __shared__ float s_g[4][kMaxTopK];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + w;
  if (t < T && lane < k) {
    s_row[w][lane] = row[t * k + lane];
    s_g[w][lane] = gate[t * k + lane];
  }
  __syncthreads();
  if (t >= T) return;
  for (int64_t v = lane; v < vpr; v += 64) {
    float acc[EPV];
#pragma unroll
    for (int q = 0; q < EPV; ++q) acc[q] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = s_row[w][j];
      const float g = s_g[w][j];
      if (r >= 0) {
        const vec16 q = yd[(int64_t)r * vpr + v];
        float f[EPV];
        if constexpr (BF16) unpack_bf16x8(q, f);
        else {
#pragma unroll
          for (int u = 0; u < 4; ++u) f[u] = __uint_as_float(q.w[u]);
        }
#pragma unroll
        for (int u = 0; u < EPV; ++u) acc[u] = fmaf(g, f[u], acc[u]);
      }
    }
    if (ysh != nullptr) {
      const vec16 q = ysh[t * vpr + v];
      float f[EPV];
      if constexpr (BF16) unpack_bf16x8(q, f);
      else {
#pragma unroll
        for (int u = 0; u < 4; ++u) f[u] = __uint_as_float(q.w[u]);
      }
#pragma unroll
      for (int u = 0; u < EPV; ++u) acc[u] += f[u];
    }
    vec16 o;
    if constexpr (BF16) o = pack_bf16x8(acc);
    else {
#pragma unroll
      for (int u = 0; u < 4; ++u) o.w[u] = __float_as_uint(acc[u]);
    }
    store16_agent(y + t * vpr + v, o);
  }
}

hipError_t launch_combine(const void* expert_out, const int32_t* row, const float* gate,
                          const void* shared_out, int64_t T, int k, int d_out, bool bf16,
                          void* y, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int64_t vpr = (int64_t)d_out * (bf16 ? 2 : 4) / 16;
  const dim3 grid((unsigned)((T + 3) / 4));
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, st, (const vec16*)expert_out, row,
                       gate, (const vec16*)shared_out, T, k, vpr, (vec16*)y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, st, (const vec16*)expert_out, row,
                       gate, (const vec16*)shared_out, T, k, vpr, (vec16*)y);
  return hipGetLastError();
}

}  // namespace moe
