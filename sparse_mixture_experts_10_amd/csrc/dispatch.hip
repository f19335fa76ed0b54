// Token-order capacity dispatch: histogram -> scan -> rank + gather.
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
// Chunks of 64 tokens (one wavefront) are the unit: kernel 1 counts each
// chunk's choices per expert, kernel 2 (one block) turns the chunk counts into
// per-chunk bases and the packed offsets, kernel 3 ranks every choice inside
// its chunk with a per-expert 64-bit token mask and copies the token rows.

#include "common.h"
#include "internal.h"

namespace moe {

__global__ __launch_bounds__(64) void dispatch_hist_kernel(const int32_t* __restrict__ idx, int64_t T,
                                                           int k, int E, int32_t* __restrict__ hist) {
  __shared__ int cnt[kMaxExperts];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kDispatchChunk + lane;
  if (t < T)
    for (int j = 0; j < k; ++j) atomicAdd(&cnt[idx[t * k + j]], 1);
  __syncthreads();
  for (int e = lane; e < E; e += 64) hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// One block.  Thread (g, e): expert e, chunk group g (contiguous chunk range).
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ hist,
                                                             int64_t nchunks, int E, int64_t cap,
                                                             int32_t* __restrict__ base,
                                                             int32_t* __restrict__ count,
                                                             int32_t* __restrict__ offset) {
  __shared__ int64_t part[1024];
  __shared__ int64_t kept_s[kMaxExperts];
  const int ngroups = blockDim.x / E;
  const int tid = threadIdx.x;
  const int e = tid % E;
  const int g = tid / E;
  const bool active = g < ngroups;
  const int64_t per = (nchunks + ngroups - 1) / ngroups;
  const int64_t c0 = (int64_t)g * per;
  const int64_t c1 = (c0 + per < nchunks) ? c0 + per : nchunks;

  int64_t local = 0;
  if (active)
    for (int64_t c = c0; c < c1; ++c) local += hist[c * E + e];
  part[tid] = local;
  __syncthreads();
  if (active) {
    int64_t run = 0;
    for (int gg = 0; gg < g; ++gg) run += part[gg * E + e];
    for (int64_t c = c0; c < c1; ++c) {
      base[c * E + e] = (int32_t)run;
      run += hist[c * E + e];
    }
    if (g == 0) {
      int64_t tot = 0;
      for (int gg = 0; gg < ngroups; ++gg) tot += part[gg * E + e];
      count[e] = (int32_t)tot;
      kept_s[e] = (cap < 0 || tot < cap) ? tot : cap;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int64_t run = 0;
    for (int ee = 0; ee < E; ++ee) {
      offset[ee] = (int32_t)run;
      run += kept_s[ee];
    }
    offset[E] = (int32_t)run;
  }
}

// One block per chunk of 64 tokens; wave 0 ranks, all four waves copy rows.
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int E, int64_t cap,
    const int32_t* __restrict__ base, const int32_t* __restrict__ offset,
    int32_t* __restrict__ slot, int32_t* __restrict__ row, int32_t* __restrict__ row_token,
    const vec16* __restrict__ x, int64_t vecs_per_row, vec16* __restrict__ x_disp) {
  __shared__ unsigned long long mask[kMaxExperts];
  __shared__ int rows_s[kDispatchChunk * kMaxTopK];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t c = blockIdx.x;
  const int64_t t = c * kDispatchChunk + lane;

  for (int e = tid; e < E; e += blockDim.x) mask[e] = 0ull;
  __syncthreads();
  if (wave == 0 && t < T)
    for (int j = 0; j < k; ++j) atomicOr(&mask[idx[t * k + j]], 1ull << lane);
  __syncthreads();
  if (wave == 0) {
    const uint64_t below = lanemask_lt();
    for (int j = 0; j < k; ++j) {
      int r = -1;
      if (t < T) {
        const int e = idx[t * k + j];
        const int s = base[c * E + e] + __popcll(mask[e] & below);
        slot[t * k + j] = s;
        if (cap < 0 || s < cap) {
          r = offset[e] + s;
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
                           void* x_disp, int32_t* ws_hist, int32_t* ws_base, hipStream_t st) {
  const int64_t nchunks = (T + kDispatchChunk - 1) / kDispatchChunk;
  if (nchunks > 0) {
    hipLaunchKernelGGL(dispatch_hist_kernel, dim3((unsigned)nchunks), dim3(64), 0, st, idx, T, k, E,
                       ws_hist);
  }
  const int threads = (1024 / E) * E;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(threads), 0, st, ws_hist, nchunks, E,
                     capacity, ws_base, count, offset);
  if (nchunks > 0) {
    const int64_t vpr = (int64_t)d * elem_bytes / 16;
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3((unsigned)nchunks), dim3(256), 0, st, idx, T,
                       k, E, capacity, ws_base, offset, slot, row, row_token, (const vec16*)x, vpr,
                       (vec16*)x_disp);
  }
  return hipGetLastError();
}

}  // namespace moe
