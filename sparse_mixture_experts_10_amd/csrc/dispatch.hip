// Token-order capacity dispatch: count -> rank + gather.
//
// Builds the dispatch of page "Appendix C -- Acronyms & Symbols" (Capacity &
// communication: capacity C = ceil(C_f k T / E), dispatch tensor D scattering
// tokens into fixed-size expert buffers) with the hard cap of page "Code
// Walkthrough -- SER" (Load balancing: overflow tokens are dropped):
//   slot(t, e) = #{t' < t : e in T_k(t')}          arrival rank at expert e
//   kept       = slot < C   (C < 0: no cap)
//   count_e    = all arrivals; kept_e = min(count_e, C)
//   offset_e   = sum_{e' < e} kept_e'               packed rows, expert-major
//   row(t, j)  = offset_e + slot, or -1 when dropped; row_token[row] = t
//   x_disp[row] = x[t]
//
// Everything is integer; LDS atomics only combine order-free integer values
// (counts, bit masks), so the result is bit-identical run to run.
//
// Chunks of 64 tokens (one wavefront) are the ranking unit; groups of four
// chunks (256 tokens) the counting unit.  Kernel 1 (one block per group)
// counts each chunk's choices per expert and the group's totals, and, in the
// fused routing pass, also the group's routing-statistics partials.  Kernel 2
// (one block per chunk) rebuilds from those counts the chunk's per-expert
// arrival bases and the packed offsets (every block redundantly: no grid-wide
// step), ranks each choice inside its chunk with a per-expert 64-bit token
// mask, and copies the token rows when the packed copy is wanted.  One more
// block writes the counts and offsets, and the statistics when asked.  Each
// kernel issues its independent loads (the choices, the statistics inputs)
// before waiting on any of them.

#include "common.h"
#include "internal.h"
#include "stats_common.h"

namespace moe {

constexpr int kGroupChunks = kStatsTokens / kDispatchChunk;  // 4
constexpr int kChoicePrefetch = 8;  // top-k choices a thread holds in registers

// One block of 256 threads per group of 256 tokens.  Wave w counts chunk
// 4 b + w.  hist[c][e], group[b][e]: counts; part[b][E + 1]: statistics
// partials (when logits != nullptr).
__global__ __launch_bounds__(256) void dispatch_count_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int E, int32_t* __restrict__ hist,
    int32_t* __restrict__ group, const float* __restrict__ logits, const float* __restrict__ lse,
    double* __restrict__ part) {
  __shared__ int cnt[kGroupChunks][kMaxExperts];
  __shared__ double s_red[256];
  __shared__ double s_grp[4 * 256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t c = (int64_t)blockIdx.x * kGroupChunks + wave;
  const int64_t t = c * kDispatchChunk + lane;
  // this token's first kChoicePrefetch choices, in flight while the
  // statistics partials load
  int ch[kChoicePrefetch];
#pragma unroll
  for (int j = 0; j < kChoicePrefetch; ++j) ch[j] = (t < T && j < k) ? idx[t * k + j] : 0;
  for (int i = tid; i < kGroupChunks * kMaxExperts; i += 256) (&cnt[0][0])[i] = 0;
  if (logits != nullptr) {
    const int64_t t0 = (int64_t)blockIdx.x * kStatsTokens;
    const int64_t t1 = (t0 + kStatsTokens < T) ? t0 + kStatsTokens : T;
    stats_block_partials(logits, lse, t0, t1, E, s_red, part + (int64_t)blockIdx.x * (E + 1), s_grp);
  }
  __syncthreads();
  if (t < T) {
#pragma unroll
    for (int j = 0; j < kChoicePrefetch; ++j)
      if (j < k) atomicAdd(&cnt[wave][ch[j]], 1);
    for (int j = kChoicePrefetch; j < k; ++j) atomicAdd(&cnt[wave][idx[t * k + j]], 1);
  }
  __syncthreads();
  const int64_t nchunks = (T + kDispatchChunk - 1) / kDispatchChunk;
  for (int e = tid; e < E; e += 256) {
    int sum = 0;
    for (int w = 0; w < kGroupChunks; ++w) {
      const int64_t cc = (int64_t)blockIdx.x * kGroupChunks + w;
      if (cc < nchunks) hist[cc * E + e] = cnt[w][e];
      sum += cnt[w][e];
    }
    group[(int64_t)blockIdx.x * E + e] = sum;
  }
}

__global__ __launch_bounds__(256) void dispatch_empty_kernel(int E, int32_t* __restrict__ count,
                                                             int32_t* __restrict__ offset) {
  for (int e = threadIdx.x; e <= E; e += 256) {
    if (e < E) count[e] = 0;
    offset[e] = 0;
  }
}

// Exclusive prefix of the per-group counts over the groups, one expert a
// column: bases[u][e] = sum_{u' < u} group[u'][e], and bases[nunits][e] the
// expert's total.  A block takes 64 experts; its four waves take a quarter of
// the groups each (sums, then the quarters' prefix, then the running bases
// written in group order).  Integer sums: exact in any order.
__global__ __launch_bounds__(256) void dispatch_scan_kernel(const int32_t* __restrict__ group, int nunits, int E,
                                                            int32_t* __restrict__ bases) {
  __shared__ int s_q[4][64];
  const int el = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + el;
  const int per = (nunits + 3) / 4;
  const int u0 = q * per < nunits ? q * per : nunits;
  const int u1 = u0 + per < nunits ? u0 + per : nunits;
  int sum = 0;
  if (e < E) {
    int u = u0;
    for (; u + 7 < u1; u += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = group[(int64_t)(u + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += v[i];
    }
    for (; u < u1; ++u) sum += group[(int64_t)u * E + e];
  }
  s_q[q][el] = sum;
  __syncthreads();
  if (e >= E) return;
  int run = 0;
  for (int qq = 0; qq < q; ++qq) run += s_q[qq][el];
  int u = u0;
  for (; u + 7 < u1; u += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = group[(int64_t)(u + i) * E + e];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bases[(int64_t)(u + i) * E + e] = run;
      run += v[i];
    }
  }
  for (; u < u1; ++u) {
    const int v = group[(int64_t)u * E + e];
    bases[(int64_t)u * E + e] = run;
    run += v;
  }
  if (q == 3) bases[(int64_t)nunits * E + e] = run;
}

// One block per chunk of 64 tokens (wave 0 ranks, all four waves copy rows),
// plus one bookkeeping block (blockIdx.x == nchunks) that writes the counts and
// offsets and, in the fused routing pass, a statistics block (nchunks + 1)
// that takes the totals again and finishes the statistics, so the counts do
// not wait behind the statistics' loads and sums.
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int E, int64_t cap,
    const int32_t* __restrict__ hist, const int32_t* __restrict__ group, const int32_t* __restrict__ bases,
    int nunits, int unit_tokens, int32_t* __restrict__ count, int32_t* __restrict__ offset, int32_t* __restrict__ slot,
    int32_t* __restrict__ row, int32_t* __restrict__ row_token, const vec16* __restrict__ x,
    int64_t vecs_per_row, vec16* __restrict__ x_disp, const double* __restrict__ part, float alpha,
    float beta, float* __restrict__ f, float* __restrict__ Pm, float* __restrict__ losses) {
  __shared__ unsigned long long mask[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wsum[4];
  __shared__ int rows_s[kDispatchChunk * kMaxTopK];
  __shared__ double s_red[256];
  __shared__ double s_z[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t c = blockIdx.x;
  const int64_t nchunks = (T + kDispatchChunk - 1) / kDispatchChunk;
  const bool books = c >= nchunks;       // uniform: a bookkeeping block (counts / statistics)
  const bool stat_blk = c == nchunks + 1;  // the statistics block
  const int64_t t = c * kDispatchChunk + lane;
  const int64_t grp = books ? nunits : c * kDispatchChunk / unit_tokens;  // units before the chunk
  const int ngroups = unit_tokens == kStatsSub ? (nunits + kStatsSubs - 1) / kStatsSubs : nunits;  // statistics groups

  for (int e = tid; e < E; e += 256) {
    s_base[e] = 0;
    s_cnt[e] = 0;
  }
  // this token's first kChoicePrefetch choices (wave 0), in flight while the
  // arrival bases load
  int ch[kChoicePrefetch];
#pragma unroll
  for (int j = 0; j < kChoicePrefetch; ++j) ch[j] = (!books && wave == 0 && t < T && j < k) ? idx[t * k + j] : 0;

  // arrival base of this chunk and totals per expert: with the scanned bases,
  // the chunk's unit base plus the per-chunk counts before it inside the unit;
  // otherwise summed from the per-unit counts (units of 256 tokens, plus the
  // per-chunk counts inside the chunk's unit; or units of 16 tokens), thread
  // (q, e) summing units q, q + Q, ... (Q = 256 / E thread rows), eight loads
  // in flight.  Integer sums, so either way gives the same result.
  if (bases != nullptr) {  // uniform
    if (stat_blk) stats_finish_sums(part, ngroups, E, s_red, s_z, unit_tokens == kStatsSub ? nunits : 0);
    if (tid < E) {
      int pre = bases[(int64_t)grp * E + tid];
      const int tot = bases[(int64_t)nunits * E + tid];
      if (!books && unit_tokens > kDispatchChunk)
        for (int64_t cc = grp * kGroupChunks; cc < c; ++cc) pre += hist[cc * E + tid];
      s_base[tid] = pre;
      s_cnt[tid] = tot;
    }
  } else {
    const int Q = 256 / E;
    const int e = tid % E, q = tid / E;
    int pre = 0, tot = 0;
    // the first eight units' counts go out before the bookkeeping block's
    // statistics loads, so the two wait together
    int v0[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v0[u] = (q < Q && q + u * Q < nunits) ? group[(int64_t)(q + u * Q) * E + e] : 0;
    if (stat_blk) stats_finish_sums(part, ngroups, E, s_red, s_z, unit_tokens == kStatsSub ? nunits : 0);
    if (q < Q) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        pre += (q + u * Q < grp) ? v0[u] : 0;
        tot += v0[u];
      }
      int b = q + 8 * Q;
      for (; b + 7 * Q < nunits; b += 8 * Q) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = group[(int64_t)(b + u * Q) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          pre += (b + u * Q < grp) ? v[u] : 0;
          tot += v[u];
        }
      }
      for (; b < nunits; b += Q) {
        const int v = group[(int64_t)b * E + e];
        pre += b < grp ? v : 0;
        tot += v;
      }
      if (q == 0 && !books && unit_tokens > kDispatchChunk)
        for (int64_t cc = grp * kGroupChunks; cc < c; ++cc) pre += hist[cc * E + e];
    }
    __syncthreads();  // the zeroed sums
    if (q < Q) {
      // integer sums: LDS atomics combine the Q thread rows in any order
      atomicAdd(&s_base[e], pre);
      atomicAdd(&s_cnt[e], tot);
    }
  }
  __syncthreads();
  if (stat_blk) {
    // statistics: the sums were taken above (group values stored for units of
    // 256, summed from the 16-token sub-partials otherwise: the same order)
    stats_finish_write(s_cnt, T, E, k, alpha, beta, f, Pm, losses, s_red, s_z, ngroups);
    return;
  }
  int kept = 0;
  if (tid < E) {
    const int tot = s_cnt[tid];
    kept = (cap < 0 || tot < cap) ? tot : (int)cap;
    mask[tid] = 0ull;
  }
  __syncthreads();
  // exclusive scan of kept over the experts: shuffle scan per wave, then
  // the wave totals
  {
    int v = kept;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(v, m, 64);
      if (lane >= m) v += o;
    }
    if (lane == 63) s_wsum[wave] = v;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_wsum[w];
    v += before;                       // inclusive prefix over all experts <= tid
    if (tid < E) s_off[tid] = v - kept;
    if (tid == E - 1) s_off[E] = v;
  }
  __syncthreads();
  if (books) {
    for (int e = tid; e < E; e += 256) count[e] = s_cnt[e];
    for (int e = tid; e <= E; e += 256) offset[e] = s_off[e];
    return;
  }

  if (wave == 0 && t < T) {
#pragma unroll
    for (int j = 0; j < kChoicePrefetch; ++j)
      if (j < k) atomicOr(&mask[ch[j]], 1ull << lane);
    for (int j = kChoicePrefetch; j < k; ++j) atomicOr(&mask[idx[t * k + j]], 1ull << lane);
  }
  __syncthreads();
  if (wave == 0) {
    const uint64_t below = lanemask_lt();
    for (int j = 0; j < k; ++j) {
      int r = -1;
      if (t < T) {
        int e = 0;
#pragma unroll
        for (int jj = 0; jj < kChoicePrefetch; ++jj)
          if (jj == j) e = ch[jj];
        if (j >= kChoicePrefetch) e = idx[t * k + j];
        const int s = s_base[e] + __popcll(mask[e] & below);
        slot[t * k + j] = s;
        if (cap < 0 || s < cap) {
          r = s_off[e] + s;
          row_token[r] = (int32_t)t;
        }
        row[t * k + j] = r;
      }
      rows_s[lane * k + j] = r;
    }
  }
  if (x_disp == nullptr) return;  // uniform: index-only dispatch
  __syncthreads();
  // copy: wave w takes tokens 16w .. 16w+15 of the chunk, lanes stride the row
  for (int i = 0; i < 16; ++i) {
    const int tl = wave * 16 + i;
    const int64_t tt = c * kDispatchChunk + tl;
    if (tt >= T) break;
    const vec16* src = x + tt * vecs_per_row;
    for (int64_t v = lane; v < vecs_per_row; v += 64) {
      const vec16 q = src[v];
      for (int j = 0; j < k; ++j) {
        const int r = rows_s[tl * k + j];
        if (r >= 0) x_disp[(int64_t)r * vecs_per_row + v] = q;
      }
    }
  }
}

hipError_t launch_dispatch(const int32_t* idx, int64_t T, int k, int E, int64_t capacity,
                           const void* x, int elem_bytes, int d, int32_t* count,
                           int32_t* offset, int32_t* slot, int32_t* row, int32_t* row_token,
                           void* x_disp, const DispatchWs& ws, const RouteStats* stats,
                           hipStream_t st) {
  const int64_t nchunks = (T + kDispatchChunk - 1) / kDispatchChunk;
  const int64_t ngroups = (T + kStatsTokens - 1) / kStatsTokens;
  if (ngroups == 0) {
    // no tokens: every expert is empty (and there are no statistics to take)
    hipLaunchKernelGGL(dispatch_empty_kernel, dim3(1), dim3(256), 0, st, E, count, offset);
    return hipGetLastError();
  }
  int unit = kStatsTokens;
  int64_t nunits = ngroups;
  if (ws.units16) {
    // the counting router wrote the per-16-token counts and sub-partials
    unit = kStatsSub;
    nunits = (T + kStatsSub - 1) / kStatsSub;
  } else {
    hipLaunchKernelGGL(dispatch_count_kernel, dim3((unsigned)ngroups), dim3(256), 0, st, idx, T, k, E,
                       ws.hist, ws.group, stats ? stats->logits : nullptr, stats ? stats->lse : nullptr,
                       ws.part);
  }
  // many units of counts: scan them once for every chunk block (linear in
  // T), instead of every chunk block summing all units (which grows as T^2)
  const int32_t* bases = nullptr;
  if (!ws.units16 && ws.bases != nullptr && nunits * E > kScanMinCounts) {
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3((unsigned)((E + 63) / 64)), dim3(256), 0, st, ws.group,
                       (int)nunits, E, ws.bases);
    bases = ws.bases;
  }
  const int64_t vpr = (int64_t)d * elem_bytes / 16;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3((unsigned)(nchunks + (stats ? 2 : 1))), dim3(256), 0, st, idx, T, k, E,
                     capacity, ws.hist, ws.group, bases, (int)nunits, unit, count, offset, slot, row, row_token,
                     (const vec16*)x, vpr, (vec16*)x_disp, ws.part, stats ? stats->alpha : 0.f,
                     stats ? stats->beta : 0.f, stats ? stats->f : nullptr, stats ? stats->P : nullptr,
                     stats ? stats->losses : nullptr);
  return hipGetLastError();
}

}  // namespace moe
