// Device pieces of the batch routing statistics shared by the statistics
// kernels and the fused routing pass, so both produce bit-identical values.
//
// Page "Appendix C -- Acronyms & Symbols", Balancing:
//   f_e   = count_e / (k T)            P_e = (1/T) sum_t softmax(h_t)_e
//   L_aux = alpha E sum_e f_e P_e      L_z = beta (1/T) sum_t lse_t^2
// All sums are fp64 in a fixed order: per block of kStatsTokens tokens first,
// then over the blocks in block order.
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {

// One 256-thread block: softmax mass per expert and the lse^2 sum over tokens
// [t0, t1) (t1 - t0 <= 256) into out[0..E-1] and out[E].  s_red: 256 doubles.
__device__ __forceinline__ void stats_block_partials(const float* __restrict__ logits,
                                                     const float* __restrict__ lse, int64_t t0,
                                                     int64_t t1, int E, double* s_red,
                                                     double* __restrict__ out) {
  const int tid = threadIdx.x;
  // thread (grp, e) sums the mass of tokens t0 + grp, t0 + grp + ngrp, ...
  const int ngrp = 256 / E;
  const int e = tid % E, grp = tid / E;
  double m = 0.0;
  if (grp < ngrp) {
    // tokens in order; eight loads issued ahead of their eight ordered adds
    int64_t t = t0 + grp;
    for (; t + 7 * ngrp < t1; t += 8 * ngrp) {
      float h[8], l[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        h[u] = logits[(t + u * ngrp) * E + e];
        l[u] = lse[t + u * ngrp];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) m += (double)expf(h[u] - l[u]);
    }
    for (; t < t1; t += ngrp) m += (double)expf(logits[t * E + e] - lse[t]);
  }
  s_red[tid] = m;
  __syncthreads();
  if (tid < E) {
    double s = 0.0;
    for (int q = 0; q < ngrp; ++q) s += s_red[q * E + tid];
    out[tid] = s;
  }
  __syncthreads();
  const int64_t t = t0 + tid;
  double z = 0.0;
  if (t < t1) {
    const double l = (double)lse[t];
    z = l * l;
  }
  s_red[tid] = z;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] += s_red[tid + w];
    __syncthreads();
  }
  if (tid == 0) out[E] = s_red[0];
  __syncthreads();
}

// One 256-thread block: f, P and the losses from the block partials
// part[nparts][E + 1] and the pre-capacity counts.  Fixed order, all partial
// loads in flight together: expert column e is summed by Q = 256 / E threads,
// thread q taking partials q, q + Q, ... in order, then the Q sums in q order;
// the lse^2 column by all 256 threads (partials tid, tid + 256, ...) and a
// pairwise tree.  s_red: 256 doubles; s_z: 256 doubles.
__device__ __forceinline__ void stats_finish(const double* __restrict__ part, int nparts,
                                             const int32_t* count, int64_t T, int E, int k,
                                             float alpha, float beta, float* __restrict__ f,
                                             float* __restrict__ Pm, float* __restrict__ losses,
                                             double* s_red, double* s_z) {
  const int tid = threadIdx.x;
  const int C = E + 1;
  const int Q = 256 / E;
  {
    const int e = tid % E, q = tid / E;
    double s = 0.0;
    if (q < Q) {
      int b = q;
      for (; b + 3 * Q < nparts; b += 4 * Q) {
        const double v0 = part[(int64_t)b * C + e], v1 = part[(int64_t)(b + Q) * C + e];
        const double v2 = part[(int64_t)(b + 2 * Q) * C + e], v3 = part[(int64_t)(b + 3 * Q) * C + e];
        s += v0;
        s += v1;
        s += v2;
        s += v3;
      }
      for (; b < nparts; b += Q) s += part[(int64_t)b * C + e];
    }
    double z = 0.0;
    for (int b = tid; b < nparts; b += 256) z += part[(int64_t)b * C + E];
    s_red[tid] = s;
    s_z[tid] = z;
  }
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s_z[tid] += s_z[tid + w];
    __syncthreads();
  }
  double fp_e = 0.0;
  if (tid < E) {
    double s = 0.0;
    for (int q = 0; q < Q; ++q) s += s_red[q * E + tid];
    const double pe = s / (double)T;
    const double fe = (double)count[tid] / ((double)k * (double)T);
    Pm[tid] = (float)pe;
    f[tid] = (float)fe;
    fp_e = fe * pe;
  }
  __syncthreads();
  if (tid < E) s_red[tid] = fp_e;
  __syncthreads();
  if (tid == 0) {
    double fp = 0.0;
    for (int ee = 0; ee < E; ++ee) fp += s_red[ee];
    const double la = (double)alpha * (double)E * fp;
    const double lz = (double)beta * s_z[0] / (double)T;
    losses[0] = (float)la;
    losses[1] = (float)lz;
    losses[2] = (float)(la + lz);
  }
}

}  // namespace moe
