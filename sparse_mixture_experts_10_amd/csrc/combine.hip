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
// fetches (row, gate) of choice j once into LDS for the whole wave; then, for
// up to 8 choices, every choice's row at two vectors a lane loads together.
// Rows of large outputs are loaded with the non-temporal hint (read once).

#include "common.h"
#include "internal.h"

namespace moe {

// 16-byte row load; NT: with the non-temporal hint.  Every expert-output
// and shared row is read once.  When the expert outputs far exceed the
// 256 MB Infinity Cache, streaming them past the caches measured 12 % faster
// (large layer: 518 -> 454 us for 2.42 GB); when they fit (the 64-expert
// layers' 16-201 MB, just written by the down pass) plain loads hit there
// and the hint cost 8-11 %.
template <bool NT>
__device__ __forceinline__ vec16 load16(const vec16* p) {
  if constexpr (NT) {
    const u32x4_t q = __builtin_nontemporal_load((const u32x4_t*)p);
    vec16 o;
    o.w[0] = q[0];
    o.w[1] = q[1];
    o.w[2] = q[2];
    o.w[3] = q[3];
    return o;
  } else {
    return *p;
  }
}

template <int EPV>
__device__ __forceinline__ void unpack_vec(const vec16& q, float (&f)[EPV]) {
  if constexpr (EPV == 8) {
    unpack_bf16x8(q, f);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) f[u] = __uint_as_float(q.w[u]);
  }
}

// KC > 0: k == KC, and every choice's row (and the shared row) is loaded
// before the first is added, so the wave waits on memory once instead of once
// a choice.  A dropped choice (row < 0) loads a kept row of the same token and
// is left out of the sum by a select; a token with no kept row loads none.
// KC == 0: any k, one choice at a time.  SH: shared_out given.
template <bool BF16, int KC, bool SH, bool NT>
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
  // KC > 0: this token's choices in registers (entries past k are never
  // read as rows: they become -1), and a kept row of the token (the same for
  // the whole wave) or -1
  constexpr int NC = KC > 0 ? KC : 1;
  int rr[NC];
  float gg[NC];
  int rkept = -1;
  if constexpr (KC > 0) {
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const int sr = s_row[w][j];
      gg[j] = s_g[w][j];
      rr[j] = j < k ? sr : -1;
    }
#pragma unroll
    for (int j = KC - 1; j >= 0; --j) rkept = rr[j] >= 0 ? rr[j] : rkept;
  }
  int64_t v0 = lane;
  if constexpr (KC > 0) {
    // two vectors a lane per round: every choice's row at both is loaded
    // before the first add (2 KC loads in flight a lane)
    for (; v0 + 64 < vpr; v0 += 128) {
      vec16 qs[2];
      if constexpr (SH) {
        qs[0] = load16<NT>(ysh + t * vpr + v0);
        qs[1] = load16<NT>(ysh + t * vpr + v0 + 64);
      }
      float acc[2][EPV];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < EPV; ++u) acc[h][u] = 0.f;
      if (rkept >= 0) {  // uniform
        vec16 q[2][KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
          const vec16* rp = yd + (int64_t)(rr[j] >= 0 ? rr[j] : rkept) * vpr + v0;
          q[0][j] = load16<NT>(rp);
          q[1][j] = load16<NT>(rp + 64);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < KC; ++j) {
            float f[EPV];
            unpack_vec<EPV>(q[h][j], f);
#pragma unroll
            for (int u = 0; u < EPV; ++u) {
              const float a = fmaf(gg[j], f[u], acc[h][u]);
              acc[h][u] = rr[j] >= 0 ? a : acc[h][u];
            }
          }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (SH) {
          float f[EPV];
          unpack_vec<EPV>(qs[h], f);
#pragma unroll
          for (int u = 0; u < EPV; ++u) acc[h][u] += f[u];
        }
        vec16 o;
        if constexpr (BF16) o = pack_bf16x8(acc[h]);
        else {
#pragma unroll
          for (int u = 0; u < 4; ++u) o.w[u] = __float_as_uint(acc[h][u]);
        }
        store16_agent(y + t * vpr + v0 + 64 * h, o);
      }
    }
  }
  for (int64_t v = v0; v < vpr; v += 64) {
    vec16 qs;
    if constexpr (SH) qs = load16<NT>(ysh + t * vpr + v);
    float acc[EPV];
#pragma unroll
    for (int u = 0; u < EPV; ++u) acc[u] = 0.f;
    if constexpr (KC > 0) {
      if (rkept >= 0) {  // uniform
        vec16 q[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) q[j] = load16<NT>(yd + (int64_t)(rr[j] >= 0 ? rr[j] : rkept) * vpr + v);
#pragma unroll
        for (int j = 0; j < KC; ++j) {
          float f[EPV];
          unpack_vec<EPV>(q[j], f);
#pragma unroll
          for (int u = 0; u < EPV; ++u) {
            const float a = fmaf(gg[j], f[u], acc[u]);
            acc[u] = rr[j] >= 0 ? a : acc[u];
          }
        }
      }
    } else {
      for (int j = 0; j < k; ++j) {
        const int r = s_row[w][j];
        const float g = s_g[w][j];
        if (r >= 0) {
          float f[EPV];
          unpack_vec<EPV>(load16<NT>(yd + (int64_t)r * vpr + v), f);
#pragma unroll
          for (int u = 0; u < EPV; ++u) acc[u] = fmaf(g, f[u], acc[u]);
        }
      }
    }
    if constexpr (SH) {
      float f[EPV];
      unpack_vec<EPV>(qs, f);
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
  const int64_t rows_bytes = T * k * vpr * 16;  // bound on the expert outputs read
  const dim3 grid((unsigned)((T + 3) / 4));
  const vec16* yd = (const vec16*)expert_out;
  const vec16* ys = (const vec16*)shared_out;
  vec16* yo = (vec16*)y;
  // expert outputs beyond the Infinity Cache: stream them
  const bool nt = rows_bytes > ((int64_t)256 << 20);
#define MOE_COMBINE(B, KC, SH)                                                                              \
  do {                                                                                                     \
    if (nt) hipLaunchKernelGGL((combine_kernel<B, KC, SH, true>), grid, dim3(256), 0, st, yd, row, gate, ys, T, k, vpr, yo); \
    else hipLaunchKernelGGL((combine_kernel<B, KC, SH, false>), grid, dim3(256), 0, st, yd, row, gate, ys, T, k, vpr, yo); \
  } while (0)
#define MOE_COMBINE_SH(B, KC)                 \
  do {                                        \
    if (shared_out != nullptr) MOE_COMBINE(B, KC, true); \
    else MOE_COMBINE(B, KC, false);           \
  } while (0)
#define MOE_COMBINE_KC(B)                     \
  switch (k) {                                \
    case 1: MOE_COMBINE_SH(B, 1); break;      \
    case 2: MOE_COMBINE_SH(B, 2); break;      \
    case 3: MOE_COMBINE_SH(B, 3); break;      \
    case 4: MOE_COMBINE_SH(B, 4); break;      \
    case 5: MOE_COMBINE_SH(B, 5); break;      \
    case 6: MOE_COMBINE_SH(B, 6); break;      \
    case 7: MOE_COMBINE_SH(B, 7); break;      \
    case 8: MOE_COMBINE_SH(B, 8); break;      \
    default: MOE_COMBINE_SH(B, 0); break;     \
  }
  if (bf16) {
    MOE_COMBINE_KC(true);
  } else {
    MOE_COMBINE_KC(false);
  }
#undef MOE_COMBINE_KC
#undef MOE_COMBINE_SH
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
