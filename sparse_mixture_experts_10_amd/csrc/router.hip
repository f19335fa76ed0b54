// Fused router: logits, log-sum-exp, greedy top-k and renormalised gates.
//
// Computes, per token t (page "Appendix C -- Acronyms & Symbols", Core MoE
// symbols; page "Code Walkthrough -- SER", the gating / routing path):
//   h[t,e]   = sum_j x[t,j] W_g[e,j] + b_g[e]
//   lse[t]   = log sum_e exp(h[t,e])
//   T_k(t)   = the k experts with the largest s = h + b_sel (ties -> lower index),
//              listed in (s desc, index asc) order
//   g[t,j]   = exp(h[t,e_j]) / sum_{j'} exp(h[t,e_j'])      (renormalised softmax)
//
// Precision: every product x*w is exact in fp64 (bf16 or fp32 times fp32) and
// the sums run in fp64, so the logits and the selection match a float64
// evaluation up to summation order; logits are rounded to fp32 once.  lse and
// the gates use fp32 exp / log on the fp64 differences h - max.
//
// Two layouts share one per-token epilogue (NXE consecutive lanes per token,
// lane eg owning experts e = eg + NXE j, so per-token reductions are shuffles):
//  * E-split (router_kernel): a block owns 64 tokens x all experts (padded to
//    EP); W_g and x stream through LDS in d-chunks; a thread owns TM tokens x
//    TE experts.
//  * K-split (router_ksplit_kernel, used when W_g fits in LDS): 16 lanes per
//    token each sum a 1/16 slice of d for every expert against W_g held whole
//    in LDS, then a recursive-halving reduce-scatter leaves lane eg with the
//    sums of its experts.  Many more tokens in flight for small E.

#include "common.h"
#include "internal.h"

namespace moe {

template <int EP>
struct RouterCfg {
  static constexpr int NT = (EP <= 16) ? 64 : 256;          // threads per block
  static constexpr int TE = (EP < 8) ? EP : 8;              // experts per thread
  static constexpr int NXE = EP / TE;                       // threads per token
  static constexpr int NXT = NT / NXE;                      // token groups
  static constexpr int TM = (64 / NXT) > 1 ? (64 / NXT) : 1;  // tokens per thread
  static constexpr int BT = NXT * TM;                       // tokens per block (64)
  static constexpr int KC = (EP >= 256) ? 32 : 64;          // d-chunk staged in LDS
};

template <int NXE>
__device__ __forceinline__ double group_max(double v) {
#pragma unroll
  for (int m = 1; m < NXE; m <<= 1) v = fmax(v, __shfl_xor(v, m, 64));
  return v;
}

template <int NXE>
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
  for (int m = 1; m < NXE; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int NXE>
__device__ __forceinline__ float group_sumf(float v) {
#pragma unroll
  for (int m = 1; m < NXE; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// (score desc, index asc) argmax across the NXE lanes of a token; carries h.
template <int NXE>
__device__ __forceinline__ void group_argmax(double& s, int& e, double& h) {
#pragma unroll
  for (int m = 1; m < NXE; m <<= 1) {
    double so = __shfl_xor(s, m, 64);
    int eo = __shfl_xor(e, m, 64);
    double ho = __shfl_xor(h, m, 64);
    bool take = (so > s) || (so == s && eo < e);
    if (take) { s = so; e = eo; h = ho; }
  }
}

// Per-token epilogue.  The NXE lanes of a token hold its fp64 dot products
// (router bias not yet added): lane eg holds experts e = eg + NXE j, j < TE.
// Writes logits, lse, top-k indices and gates for token t (when live).
template <int TE, int NXE>
__device__ __forceinline__ void token_epilogue(const double (&acc)[TE], int eg, int64_t t, bool live,
                                               int E, int k, const float* __restrict__ bg,
                                               const float* __restrict__ bsel,
                                               float* __restrict__ logits, float* __restrict__ lse_out,
                                               int32_t* __restrict__ topk_idx,
                                               float* __restrict__ topk_gate) {
  const double NEG = -__builtin_huge_val();
  double h[TE], s[TE];
  double m = NEG;
#pragma unroll
  for (int j = 0; j < TE; ++j) {
    const int e = eg + NXE * j;
    const bool ok = e < E;
    h[j] = ok ? acc[j] + (bg != nullptr ? (double)bg[e] : 0.0) : NEG;
    s[j] = ok ? h[j] + (bsel != nullptr ? (double)bsel[e] : 0.0) : NEG;
    m = fmax(m, h[j]);
  }
  m = group_max<NXE>(m);
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < TE; ++j) se += (eg + NXE * j < E) ? expf((float)(h[j] - m)) : 0.f;
  se = group_sumf<NXE>(se);
  if (live) {
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const int e = eg + NXE * j;
      if (e < E) logits[t * E + e] = (float)h[j];
    }
    if (eg == 0) lse_out[t] = (float)(m + (double)logf(se));
  }
  // two passes of k argmax rounds: the first sums the selected exp(h - m),
  // the second writes indices and gates in selection order
  float gsum = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    uint32_t taken = 0;
    for (int r = 0; r < k; ++r) {
      double bs = NEG, bh = 0.0;
      int be = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < TE; ++j) {
        const int e = eg + NXE * j;
        const bool ok = (e < E) && !((taken >> j) & 1u);
        if (ok && (s[j] > bs || (s[j] == bs && e < be))) { bs = s[j]; be = e; bh = h[j]; }
      }
      group_argmax<NXE>(bs, be, bh);
      if (be % NXE == eg) taken |= 1u << (be / NXE);
      const float ex = expf((float)(bh - m));
      if (pass == 0) {
        gsum += ex;
      } else if (live && eg == 0) {
        topk_idx[t * k + r] = be;
        topk_gate[t * k + r] = ex / gsum;
      }
    }
  }
}

template <int EP, bool XBF16>
__global__ __launch_bounds__(RouterCfg<EP>::NT) void router_kernel(
    const void* __restrict__ xv, int64_t T, int d, const float* __restrict__ Wg,
    const float* __restrict__ bg, const float* __restrict__ bsel, int E, int k,
    float* __restrict__ logits, float* __restrict__ lse_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate) {
  using C = RouterCfg<EP>;
  constexpr int NT = C::NT, TE = C::TE, NXE = C::NXE, TM = C::TM, BT = C::BT, KC = C::KC;
  constexpr int LDX = KC + 1;
  __shared__ float xs[BT * LDX];
  __shared__ float ws[EP * LDX];

  const int tid = threadIdx.x;
  const int eg = tid % NXE;
  const int tg = tid / NXE;
  const int64_t t0 = (int64_t)blockIdx.x * BT;

  double acc[TM][TE];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TE; ++j) acc[i][j] = 0.0;

  for (int k0 = 0; k0 < d; k0 += KC) {
    // stage x[t0 : t0+BT, k0 : k0+KC] as fp32
    if (XBF16) {
      const bf16_t* x = (const bf16_t*)xv;
      constexpr int VPR = KC / 8;
      for (int v = tid; v < BT * VPR; v += NT) {
        const int r = v / VPR, cv = v % VPR;
        const int64_t t = t0 + r;
        const int col = k0 + cv * 8;
        float f[8];
        if (t < T && col < d) {
          vec16 q = *(const vec16*)(x + t * (int64_t)d + col);
          unpack_bf16x8(q, f);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) f[q] = 0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) xs[r * LDX + cv * 8 + q] = f[q];
      }
    } else {
      const float* x = (const float*)xv;
      constexpr int VPR = KC / 4;
      for (int v = tid; v < BT * VPR; v += NT) {
        const int r = v / VPR, cv = v % VPR;
        const int64_t t = t0 + r;
        const int col = k0 + cv * 4;
        float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < T && col < d) q = *(const float4*)(x + t * (int64_t)d + col);
        xs[r * LDX + cv * 4 + 0] = q.x;
        xs[r * LDX + cv * 4 + 1] = q.y;
        xs[r * LDX + cv * 4 + 2] = q.z;
        xs[r * LDX + cv * 4 + 3] = q.w;
      }
    }
    // stage W_g[0:EP, k0 : k0+KC]
    {
      constexpr int VPR = KC / 4;
      for (int v = tid; v < EP * VPR; v += NT) {
        const int e = v / VPR, cv = v % VPR;
        const int col = k0 + cv * 4;
        float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e < E && col < d) q = *(const float4*)(Wg + (int64_t)e * d + col);
        ws[e * LDX + cv * 4 + 0] = q.x;
        ws[e * LDX + cv * 4 + 1] = q.y;
        ws[e * LDX + cv * 4 + 2] = q.z;
        ws[e * LDX + cv * 4 + 3] = q.w;
      }
    }
    __syncthreads();
    const int kcount = (d - k0 < KC) ? (d - k0) : KC;
    for (int kk = 0; kk < kcount; ++kk) {
      double xr[TM], wr[TE];
#pragma unroll
      for (int i = 0; i < TM; ++i) xr[i] = (double)xs[(tg * TM + i) * LDX + kk];
#pragma unroll
      for (int j = 0; j < TE; ++j) wr[j] = (double)ws[(eg + NXE * j) * LDX + kk];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TE; ++j) acc[i][j] = fma(xr[i], wr[j], acc[i][j]);
    }
    __syncthreads();
  }

  // ---- per-token epilogue ----
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t t = t0 + tg * TM + i;
    token_epilogue<TE, NXE>(acc[i], eg, t, t < T, E, k, bg, bsel, logits, lse_out, topk_idx,
                            topk_gate);
  }
}

// One recursive-halving step of a reduce-scatter over lane bit O: the lane
// keeps the half of v whose index bit O matches its own lane bit and adds the
// partner's copy of that half.
template <int N, int O>
__device__ __forceinline__ void rs_halve(const double (&v)[N], double (&w)[N / 2], int lane) {
  const bool hi = (lane & O) != 0;
#pragma unroll
  for (int q = 0; q < N / 2; ++q) {
    const int i0 = (q / O) * 2 * O + q % O;
    const double keep = hi ? v[i0 + O] : v[i0];
    const double send = hi ? v[i0] : v[i0 + O];
    w[q] = keep + __shfl_xor(send, O, 64);
  }
}

constexpr int KS_LPT = 16;    // lanes per token
constexpr int KS_TPB = 16;    // tokens per block (256 threads)

template <int EP, bool XBF16>
__global__ __launch_bounds__(256) void router_ksplit_kernel(
    const void* __restrict__ xv, int64_t T, int d, const float* __restrict__ Wg,
    const float* __restrict__ bg, const float* __restrict__ bsel, int E, int k,
    float* __restrict__ logits, float* __restrict__ lse_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate) {
  extern __shared__ float wsm[];  // W_g [E][d], fp32
  const int tid = threadIdx.x;
  const int lane = tid & (KS_LPT - 1);
  const int64_t t = (int64_t)blockIdx.x * KS_TPB + tid / KS_LPT;

  const int nv4 = E * d / 4;
  for (int v = tid; v < nv4; v += 256) ((float4*)wsm)[v] = ((const float4*)Wg)[v];
  __syncthreads();

  double acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.0;
  if (t < T) {
    if (XBF16) {
      const bf16_t* x = (const bf16_t*)xv + t * (int64_t)d;
      for (int col = lane * 8; col < d; col += KS_LPT * 8) {
        float f[8];
        unpack_bf16x8(*(const vec16*)(x + col), f);
#pragma unroll
        for (int e = 0; e < EP; ++e) {
          if (e < E) {
            const float4 w0 = *(const float4*)(wsm + e * d + col);
            const float4 w1 = *(const float4*)(wsm + e * d + col + 4);
            double a = acc[e];
            a = fma((double)f[0], (double)w0.x, a);
            a = fma((double)f[1], (double)w0.y, a);
            a = fma((double)f[2], (double)w0.z, a);
            a = fma((double)f[3], (double)w0.w, a);
            a = fma((double)f[4], (double)w1.x, a);
            a = fma((double)f[5], (double)w1.y, a);
            a = fma((double)f[6], (double)w1.z, a);
            a = fma((double)f[7], (double)w1.w, a);
            acc[e] = a;
          }
        }
      }
    } else {
      const float* x = (const float*)xv + t * (int64_t)d;
      for (int col = lane * 4; col < d; col += KS_LPT * 4) {
        const float4 q = *(const float4*)(x + col);
#pragma unroll
        for (int e = 0; e < EP; ++e) {
          if (e < E) {
            const float4 w0 = *(const float4*)(wsm + e * d + col);
            double a = acc[e];
            a = fma((double)q.x, (double)w0.x, a);
            a = fma((double)q.y, (double)w0.y, a);
            a = fma((double)q.z, (double)w0.z, a);
            a = fma((double)q.w, (double)w0.w, a);
            acc[e] = a;
          }
        }
      }
    }
  }

  // reduce-scatter over the 16 lanes: lane l ends with experts l + 16 j
  constexpr int TE = (EP >= 16) ? EP / 16 : 1;
  double r[TE];
  if constexpr (EP == 8) {
    double a4[4], a2[2];
    double full[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) full[e] = acc[e] + __shfl_xor(acc[e], 8, 64);
    rs_halve<8, 4>(full, a4, lane);
    rs_halve<4, 2>(a4, a2, lane);
    rs_halve<2, 1>(a2, r, lane);
  } else {
    double b8[EP / 2], b4[EP / 4], b2[EP / 8];
    rs_halve<EP, 8>(acc, b8, lane);
    rs_halve<EP / 2, 4>(b8, b4, lane);
    rs_halve<EP / 4, 2>(b4, b2, lane);
    rs_halve<EP / 8, 1>(b2, r, lane);
  }
  // for EP = 8, lanes 8..15 duplicate lanes 0..7; their expert ids lane >= 8 >= E are void
  token_epilogue<TE, KS_LPT>(r, lane, t, t < T, E, k, bg, bsel, logits, lse_out, topk_idx, topk_gate);
}

template <int EP>
static hipError_t launch_router_ksplit(const void* x, bool xbf16, int64_t T, int d, const float* Wg,
                                       const float* bg, const float* bsel, int E, int k,
                                       float* logits, float* lse, int32_t* idx, float* gate,
                                       hipStream_t st) {
  const dim3 grid((unsigned)((T + KS_TPB - 1) / KS_TPB));
  const size_t lds = (size_t)E * d * sizeof(float);
  if (xbf16)
    hipLaunchKernelGGL((router_ksplit_kernel<EP, true>), grid, dim3(256), lds, st, x, T, d, Wg, bg,
                       bsel, E, k, logits, lse, idx, gate);
  else
    hipLaunchKernelGGL((router_ksplit_kernel<EP, false>), grid, dim3(256), lds, st, x, T, d, Wg, bg,
                       bsel, E, k, logits, lse, idx, gate);
  return hipGetLastError();
}

template <int EP>
static hipError_t launch_router_ep(const void* x, bool xbf16, int64_t T, int d, const float* Wg,
                                   const float* bg, const float* bsel, int E, int k, float* logits,
                                   float* lse, int32_t* idx, float* gate, hipStream_t st) {
  using C = RouterCfg<EP>;
  const dim3 grid((unsigned)((T + C::BT - 1) / C::BT));
  if (xbf16)
    hipLaunchKernelGGL((router_kernel<EP, true>), grid, dim3(C::NT), 0, st, x, T, d, Wg, bg, bsel, E,
                       k, logits, lse, idx, gate);
  else
    hipLaunchKernelGGL((router_kernel<EP, false>), grid, dim3(C::NT), 0, st, x, T, d, Wg, bg, bsel,
                       E, k, logits, lse, idx, gate);
  return hipGetLastError();
}

hipError_t launch_router(const void* x, bool xbf16, int64_t T, int d, const float* Wg,
                         const float* bg, const float* bsel, int E, int k, float* logits,
                         float* lse, int32_t* idx, float* gate, hipStream_t st) {
  // K-split when W_g fits in 64 KB of LDS and E <= 64
  if ((int64_t)E * d * 4 <= 65536 && E <= 64) {
    if (E <= 8) return launch_router_ksplit<8>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
    if (E <= 16) return launch_router_ksplit<16>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
    if (E <= 32) return launch_router_ksplit<32>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
    return launch_router_ksplit<64>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  }
  if (E <= 8) return launch_router_ep<8>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  if (E <= 16) return launch_router_ep<16>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  if (E <= 32) return launch_router_ep<32>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  if (E <= 64) return launch_router_ep<64>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  if (E <= 128) return launch_router_ep<128>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  return launch_router_ep<256>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
}

}  // namespace moe
