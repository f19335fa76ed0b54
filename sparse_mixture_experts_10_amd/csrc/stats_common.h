// Device pieces of the batch routing statistics shared by the statistics
// kernels and the fused routing pass, so both produce bit-identical values.
//
// Page "Appendix C -- Acronyms & Symbols", Balancing:
//   f_e   = count_e / (k T)            P_e = (1/T) sum_t softmax(h_t)_e
//   L_aux = alpha E sum_e f_e P_e      L_z = beta (1/T) sum_t lse_t^2
// All sums are fp64 in one fixed order, whichever kernel takes them:
//   sub-partial  = sum over a block of kStatsSub tokens, in token order, from 0
//   group value  = sum of the group's sub-partials (kStatsTokens tokens), in order
//   total        = stats_finish's fixed order over the group values
// The softmax mass of a token is expf(logit - lse) on the stored fp32 values.
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kStatsSubs = kStatsTokens / kStatsSub;  // sub-partials per group

// One 256-thread block: the group value of tokens [t0, t1) (t1 - t0 <= 256):
// softmax mass per expert into out[0..E-1], lse^2 into out[E].  Thread
// (i, el) sums sub-block i of experts e0 + el, e0 + 16 + el, ... for up to four
// rounds of 16 experts whose loads are all issued before any wait (64 experts
// a pass).  s_red: 256 doubles; s_grp: 4 * 256 doubles.
__device__ __forceinline__ void stats_block_partials(const float* __restrict__ logits,
                                                     const float* __restrict__ lse, int64_t t0,
                                                     int64_t t1, int E, double* s_red,
                                                     double* __restrict__ out, double* s_grp) {
  constexpr int R = 4;  // expert rounds per pass
  const int tid = threadIdx.x;
  const int i = tid / kStatsSub, el = tid % kStatsSub;   // sub-block, expert in the round
  const int64_t s0 = t0 + (int64_t)i * kStatsSub;
  const int n = (int)((t1 - s0) < kStatsSub ? (t1 - s0 > 0 ? t1 - s0 : 0) : kStatsSub);
  float l[kStatsSub];
#pragma unroll
  for (int u = 0; u < kStatsSub; ++u) l[u] = u < n ? lse[s0 + u] : 0.f;
  for (int e0 = 0; e0 < E; e0 += R * kStatsSub) {
    float h[R][kStatsSub];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = e0 + r * kStatsSub + el;
#pragma unroll
      for (int u = 0; u < kStatsSub; ++u) h[r][u] = (u < n && e < E) ? logits[(s0 + u) * E + e] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      double m = 0.0;
#pragma unroll
      for (int u = 0; u < kStatsSub; ++u)
        if (u < n) m += (double)expf(h[r][u] - l[u]);
      s_grp[r * 256 + tid] = m;
    }
    __syncthreads();
    if (tid < R * kStatsSub) {
      const int r = tid / kStatsSub, e = e0 + tid;
      if (e < E) {
        double g = 0.0;
        for (int q = 0; q < kStatsSubs; ++q) g += s_grp[r * 256 + q * kStatsSub + (tid % kStatsSub)];
        out[e] = g;
      }
    }
    __syncthreads();
  }
  // lse^2: lane el == 0 of each sub-block, then the sub-blocks in order
  double z = 0.0;
#pragma unroll
  for (int u = 0; u < kStatsSub; ++u)
    if (u < n) z += (double)l[u] * (double)l[u];
  s_red[tid] = z;
  __syncthreads();
  if (tid == 0) {
    double g = 0.0;
    for (int q = 0; q < kStatsSubs; ++q) g += s_red[q * kStatsSub];
    out[E] = g;
  }
  __syncthreads();
}

// Value of group b, column col: stored directly (nsub == 0: part is
// [ngroups][C]) or summed from its sub-partials (part is [nsub][C], the
// group's kStatsSubs rows in order).
__device__ __forceinline__ double stats_group_value(const double* __restrict__ part, int64_t b, int col,
                                                    int C, int64_t nsub) {
  if (nsub == 0) return part[b * C + col];
  const int64_t r0 = b * kStatsSubs;
  double v[kStatsSubs];
#pragma unroll
  for (int i = 0; i < kStatsSubs; ++i) v[i] = (r0 + i < nsub) ? part[(r0 + i) * C + col] : 0.0;
  // 0.0 + v[0] is v[0] (the partials are non-negative): starting from v[0]
  // also keeps the compiler from waiting on that load right where it is issued
  double g = v[0];
#pragma unroll
  for (int i = 1; i < kStatsSubs; ++i) g += v[i];
  return g;
}

// One 256-thread block, first half of the statistics finish: the sums over
// the group values (nparts groups; see stats_group_value for nsub) in a
// fixed order, all partial loads in flight together.  Expert column e is
// summed by Q = 256 / E threads, thread q taking groups q, q + Q, ... in
// order (left in s_red[q E + e]); the lse^2 column by all 256 threads
// (groups tid, tid + 256, ...) and a pairwise tree (left in s_z[0]).
// s_red, s_z: 256 doubles each.
// Every partial is a sum of non-negative terms, so adding a +0 leaves it
// unchanged: tree levels whose upper half lies past nparts are skipped, and
// with nparts <= 64 the rest runs in wave 0 with shuffles pairing the same
// entries (lane i adds lane i + w), without LDS or barriers.
__device__ __forceinline__ void stats_finish_sums(const double* __restrict__ part, int nparts, int E,
                                                  double* s_red, double* s_z, int64_t nsub = 0) {
  const int tid = threadIdx.x;
  const int C = E + 1;
  const int Q = 256 / E;
  double s = 0.0, z = 0.0;
  const int e = tid % E, q = tid / E;
  // the wave that holds the lse^2 group sums (lane i: group i)
  int zw = 0;
  if (nsub > 0 && nparts <= Q && nparts <= 64) {
    // at most one group a thread in either sum, the lse^2 groups in wave 3
    // (the expert groups fill the first waves; wave 3 has room for 64
    // groups, so more groups, possible when E <= 3, take the general path
    // below, which pairs the same entries): every sub-partial is loaded
    // before any is added up
    zw = 3;
    const bool has_e = q < nparts, has_z = tid >= 192 && tid - 192 < nparts;
    const int64_t re = (int64_t)q * kStatsSubs, rz = (int64_t)(tid - 192) * kStatsSubs;
    double ve[kStatsSubs], vz[kStatsSubs];
#pragma unroll
    for (int i = 0; i < kStatsSubs; ++i) {
      ve[i] = (has_e && re + i < nsub) ? part[(re + i) * C + e] : 0.0;
      vz[i] = (has_z && rz + i < nsub) ? part[(rz + i) * C + E] : 0.0;
    }
    double ge = ve[0], gz = vz[0];  // = 0.0 + v[0]: the partials are non-negative
#pragma unroll
    for (int i = 1; i < kStatsSubs; ++i) {
      ge += ve[i];
      gz += vz[i];
    }
    if (has_e) s += ge;
    if (has_z) z += gz;
  } else {
    if (q < Q) {
      // groups q, q + Q, ... added in that order, sixteen stored group values
      // (or four summed from sub-partials) loaded before they are added
      int b = q;
      if (nsub == 0) {
        for (; b + 15 * Q < nparts; b += 16 * Q) {
          double v[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = part[(int64_t)(b + i * Q) * C + e];
#pragma unroll
          for (int i = 0; i < 16; ++i) s += v[i];
        }
      }
      for (; b + 3 * Q < nparts; b += 4 * Q) {
        const double v0 = stats_group_value(part, b, e, C, nsub);
        const double v1 = stats_group_value(part, b + Q, e, C, nsub);
        const double v2 = stats_group_value(part, b + 2 * Q, e, C, nsub);
        const double v3 = stats_group_value(part, b + 3 * Q, e, C, nsub);
        s += v0;
        s += v1;
        s += v2;
        s += v3;
      }
      for (; b < nparts; b += Q) s += stats_group_value(part, b, e, C, nsub);
    }
    for (int b = tid; b < nparts; b += 256) z += stats_group_value(part, b, E, C, nsub);
  }
  s_red[tid] = s;
  if (nparts <= 64) {
    if ((tid >> 6) == zw) {  // uniform per wave
      // lane 0 adds lane w at each level; for the lanes i < w that feed lane
      // 0, lane i ^ w is lane i + w, so the exchange is lane ^ w (a DPP move
      // below 16 instead of an LDS round trip); levels past nparts are skipped
      if (32 < nparts) z += xor_lane_d<32>(z);
      if (16 < nparts) z += xor_lane_d<16>(z);
      if (8 < nparts) z += xor_lane_d<8>(z);
      if (4 < nparts) z += xor_lane_d<4>(z);
      if (2 < nparts) z += xor_lane_d<2>(z);
      if (1 < nparts) z += xor_lane_d<1>(z);
      if (tid == 64 * zw) s_z[0] = z;
    }
    __syncthreads();
    return;
  }
  s_z[tid] = z;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (w < nparts) {  // uniform
      if (tid < w) s_z[tid] += s_z[tid + w];
      __syncthreads();
    }
  }
}

// Second half: f, P and the losses from those sums and the pre-capacity counts.
// Thread rows q >= nparts summed no group (+0), so the expert sums stop there;
// with E <= 64 the E products are summed in order in wave 0 from its lanes.
__device__ __forceinline__ void stats_finish_write(const int32_t* count, int64_t T, int E, int k,
                                                   float alpha, float beta, float* __restrict__ f,
                                                   float* __restrict__ Pm, float* __restrict__ losses,
                                                   double* s_red, double* s_z, int nparts) {
  const int tid = threadIdx.x;
  const int Q = 256 / E;
  const int qn = nparts < Q ? nparts : Q;
  double fp_e = 0.0;
  if (tid < E) {
    double s = 0.0;
    for (int q = 0; q < qn; ++q) s += s_red[q * E + tid];
    const double pe = s / (double)T;
    const double fe = (double)count[tid] / ((double)k * (double)T);
    Pm[tid] = (float)pe;
    f[tid] = (float)fe;
    fp_e = fe * pe;
  }
  double fp = 0.0;
  if (E <= 64) {
    if (tid >= 64) return;  // wave 0 holds every product
    // lane ee's product read into scalar registers (no LDS round trip)
    const long long u = __double_as_longlong(fp_e);
    const int lo = (int)(u & 0xffffffffll), hi = (int)(u >> 32);
    for (int ee = 0; ee < E; ++ee) {
      const unsigned l = (unsigned)__builtin_amdgcn_readlane(lo, ee);
      const long long h = __builtin_amdgcn_readlane(hi, ee);
      fp += __longlong_as_double((h << 32) | l);
    }
  } else {
    __syncthreads();
    if (tid < E) s_red[tid] = fp_e;
    __syncthreads();
    if (tid == 0)
      for (int ee = 0; ee < E; ++ee) fp += s_red[ee];
  }
  if (tid == 0) {
    const double la = (double)alpha * (double)E * fp;
    const double lz = (double)beta * s_z[0] / (double)T;
    losses[0] = (float)la;
    losses[1] = (float)lz;
    losses[2] = (float)(la + lz);
  }
}

__device__ __forceinline__ void stats_finish(const double* __restrict__ part, int nparts,
                                             const int32_t* count, int64_t T, int E, int k,
                                             float alpha, float beta, float* __restrict__ f,
                                             float* __restrict__ Pm, float* __restrict__ losses,
                                             double* s_red, double* s_z, int64_t nsub = 0) {
  stats_finish_sums(part, nparts, E, s_red, s_z, nsub);
  stats_finish_write(count, T, E, k, alpha, beta, f, Pm, losses, s_red, s_z, nparts);
}

}  // namespace moe
