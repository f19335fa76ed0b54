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
// the sums run in fp64, so logits, lse and the selection match a float64
// evaluation up to summation order.  Outputs are rounded to fp32 once.
//
// Layout: one block owns BT = 64 tokens and all experts (padded to EP).  A
// thread owns TM tokens x TE experts (experts strided by NXE so LDS rows are
// read conflict-free); the NXE threads that share a token are consecutive
// lanes, so the per-token softmax / top-k reductions are lane shuffles.

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
  double bgv[TE], bsv[TE];
#pragma unroll
  for (int j = 0; j < TE; ++j) {
    const int e = eg + NXE * j;
    bgv[j] = (bg != nullptr && e < E) ? (double)bg[e] : 0.0;
    bsv[j] = (bsel != nullptr && e < E) ? (double)bsel[e] : 0.0;
  }
  const double NEG = -__builtin_huge_val();

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t t = t0 + tg * TM + i;
    const bool live = t < T;  // uniform across the token's lanes
    double h[TE], s[TE];
    double m = NEG;
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const int e = eg + NXE * j;
      h[j] = (e < E) ? acc[i][j] + bgv[j] : NEG;
      s[j] = (e < E) ? h[j] + bsv[j] : NEG;
      m = fmax(m, h[j]);
    }
    m = group_max<NXE>(m);
    double se = 0.0;
#pragma unroll
    for (int j = 0; j < TE; ++j) se += (eg + NXE * j < E) ? exp(h[j] - m) : 0.0;
    se = group_sum<NXE>(se);
    if (live) {
#pragma unroll
      for (int j = 0; j < TE; ++j) {
        const int e = eg + NXE * j;
        if (e < E) logits[t * E + e] = (float)h[j];
      }
      if (eg == 0) lse_out[t] = (float)(m + log(se));
    }

    // two passes of k argmax rounds: the first sums the selected exp(h - m),
    // the second writes indices and gates in selection order
    double gsum = 0.0;
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
        const double ex = exp(bh - m);
        if (pass == 0) {
          gsum += ex;
        } else if (live && eg == 0) {
          topk_idx[t * k + r] = be;
          topk_gate[t * k + r] = (float)(ex / gsum);
        }
      }
    }
  }
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
  if (E <= 8) return launch_router_ep<8>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  if (E <= 16) return launch_router_ep<16>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  if (E <= 32) return launch_router_ep<32>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  if (E <= 64) return launch_router_ep<64>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  if (E <= 128) return launch_router_ep<128>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
  return launch_router_ep<256>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, st);
}

}  // namespace moe
