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

#include <type_traits>

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
// With noise != nullptr the logits are h + sigma * noise[t, e] (noisy top-k,
// page "Code Walkthrough -- SER", the gating / routing path: training noise is
// added to the logits before selection) and everything after uses them.
// Writes logits, lse, top-k indices and gates for token t (when live).
// With flag_rel > 0 it returns true (on every lane of the token) when two
// consecutive scores among the k + 1 highest (k when k = E) are closer than
// flag_rel * max(1, |score|): the selected set or its listed order could then
// change within the logits' rounding error.
template <int TE, int NXE>
__device__ __forceinline__ bool token_epilogue(const double (&acc)[TE], int eg, int64_t t, bool live,
                                               int E, int k, const float* __restrict__ bg,
                                               const float* __restrict__ bsel,
                                               float* __restrict__ logits, float* __restrict__ lse_out,
                                               int32_t* __restrict__ topk_idx,
                                               float* __restrict__ topk_gate,
                                               const float* __restrict__ noise, double sigma,
                                               double flag_rel = 0.0) {
  const double NEG = -__builtin_huge_val();
  double h[TE], s[TE];
  double m = NEG;
#pragma unroll
  for (int j = 0; j < TE; ++j) {
    const int e = eg + NXE * j;
    const bool ok = e < E;
    double hv = acc[j] + (bg != nullptr ? (double)bg[e] : 0.0);
    if (noise != nullptr && live && ok) hv += sigma * (double)noise[t * E + e];
    h[j] = ok ? hv : NEG;
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
  bool near = false;
  double prev = 0.0;
  for (int pass = 0; pass < 2; ++pass) {
    uint32_t taken = 0;
    const int rounds = (pass == 0 && flag_rel > 0.0 && k < E) ? k + 1 : k;
    for (int r = 0; r < rounds; ++r) {
      double bs = NEG, bh = 0.0;
      int be = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < TE; ++j) {
        const int e = eg + NXE * j;
        const bool ok = (e < E) && !((taken >> j) & 1u);
        if (ok && (s[j] > bs || (s[j] == bs && e < be))) { bs = s[j]; be = e; bh = h[j]; }
      }
      group_argmax<NXE>(bs, be, bh);
      if (pass == 0 && flag_rel > 0.0) {
        if (r > 0 && prev - bs < flag_rel * fmax(1.0, fabs(prev))) near = true;
        prev = bs;
      }
      if (r == k) break;  // the (k+1)-th score only feeds the flag
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
  return near;
}

// x element types of the E-split layout: fp32, bf16, or fp64 (the MLP gate's
// hidden layer)
enum { XT_F32 = 0, XT_BF16 = 1, XT_F64 = 2 };

template <int XT>
using XStage = typename std::conditional<XT == XT_F64, double, float>::type;

// The E-split dot products of one block: 64 tokens x EP rows of W, fp64
// accumulation; x and W stream through LDS in KC-wide chunks of d.
template <int EP, int XT>
__device__ __forceinline__ void router_block_dots(
    const void* __restrict__ xv, int64_t T, int d, const float* __restrict__ Wg, int E, int64_t t0,
    XStage<XT>* xs, float* ws, double (&acc)[RouterCfg<EP>::TM][RouterCfg<EP>::TE]) {
  using C = RouterCfg<EP>;
  constexpr int NT = C::NT, TE = C::TE, NXE = C::NXE, TM = C::TM, BT = C::BT, KC = C::KC;
  constexpr int LDX = KC + 1;
  const int tid = threadIdx.x;
  const int eg = tid % NXE;
  const int tg = tid / NXE;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TE; ++j) acc[i][j] = 0.0;

  for (int k0 = 0; k0 < d; k0 += KC) {
    // stage x[t0 : t0+BT, k0 : k0+KC]
    if constexpr (XT == XT_BF16) {
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
    } else if constexpr (XT == XT_F32) {
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
    } else {
      const double* x = (const double*)xv;
      constexpr int VPR = KC / 2;
      for (int v = tid; v < BT * VPR; v += NT) {
        const int r = v / VPR, cv = v % VPR;
        const int64_t t = t0 + r;
        const int col = k0 + cv * 2;
        double2 q = make_double2(0.0, 0.0);
        if (t < T && col < d) q = *(const double2*)(x + t * (int64_t)d + col);
        xs[r * LDX + cv * 2 + 0] = q.x;
        xs[r * LDX + cv * 2 + 1] = q.y;
      }
    }
    // stage W[0:EP, k0 : k0+KC]
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
}

template <int EP, int XT>
__global__ __launch_bounds__(RouterCfg<EP>::NT) void router_kernel(
    const void* __restrict__ xv, int64_t T, int d, const float* __restrict__ Wg,
    const float* __restrict__ bg, const float* __restrict__ bsel, int E, int k,
    float* __restrict__ logits, float* __restrict__ lse_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, const float* __restrict__ noise, double sigma) {
  using C = RouterCfg<EP>;
  constexpr int TE = C::TE, NXE = C::NXE, TM = C::TM, BT = C::BT, LDX = C::KC + 1;
  __shared__ XStage<XT> xs[BT * LDX];
  __shared__ float ws[EP * LDX];
  const int tid = threadIdx.x;
  const int eg = tid % NXE;
  const int tg = tid / NXE;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  double acc[TM][TE];
  router_block_dots<EP, XT>(xv, T, d, Wg, E, t0, xs, ws, acc);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t t = t0 + tg * TM + i;
    token_epilogue<TE, NXE>(acc[i], eg, t, t < T, E, k, bg, bsel, logits, lse_out, topk_idx,
                            topk_gate, noise, sigma);
  }
}

// MLP gate, layer 1 (page "Code Walkthrough -- SER", Configuration: an MLP
// gate of width gater_hidden_dim instead of the linear router):
//   hidden[t, h] = relu(sum_j x[t, j] gW1[h, j] + gb1[h]) in fp64
template <int HP, int XT>
__global__ __launch_bounds__(RouterCfg<HP>::NT) void mlp_gate_hidden_kernel(
    const void* __restrict__ xv, int64_t T, int d, const float* __restrict__ gW1,
    const float* __restrict__ gb1, int H, double* __restrict__ hidden) {
  using C = RouterCfg<HP>;
  constexpr int TE = C::TE, NXE = C::NXE, TM = C::TM, BT = C::BT, LDX = C::KC + 1;
  __shared__ XStage<XT> xs[BT * LDX];
  __shared__ float ws[HP * LDX];
  const int tid = threadIdx.x;
  const int eg = tid % NXE;
  const int tg = tid / NXE;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  double acc[TM][TE];
  router_block_dots<HP, XT>(xv, T, d, gW1, H, t0, xs, ws, acc);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t t = t0 + tg * TM + i;
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const int h = eg + NXE * j;
      if (t < T && h < H) {
        const double a = acc[i][j] + (gb1 != nullptr ? (double)gb1[h] : 0.0);
        hidden[t * H + h] = a > 0.0 ? a : 0.0;
      }
    }
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
constexpr int KS_XV = 16;     // x vectors per lane: d <= 16 * 16 * 8 (bf16) or 16 * 16 * 4 (fp32)

template <int EP, bool XBF16>
__global__ __launch_bounds__(256) void router_ksplit_kernel(
    const void* __restrict__ xv, int64_t T, int d, const float* __restrict__ Wg,
    const float* __restrict__ bg, const float* __restrict__ bsel, int E, int k,
    float* __restrict__ logits, float* __restrict__ lse_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, const float* __restrict__ noise, double sigma) {
  extern __shared__ float wsm[];  // W_g [E][d], fp32
  const int tid = threadIdx.x;
  const int lane = tid & (KS_LPT - 1);
  const int64_t t = (int64_t)blockIdx.x * KS_TPB + tid / KS_LPT;

  // this lane's slice of the token row, loaded before the W_g fill so both
  // loads are in flight together (d <= kKsMaxD: at most KS_XV vectors a lane)
  constexpr int XW = XBF16 ? 8 : 4;   // elements per 16-byte vector
  vec16 xr[KS_XV];
#pragma unroll
  for (int it = 0; it < KS_XV; ++it) {
    const int col = (lane + KS_LPT * it) * XW;
    if (t < T && col < d) {
      xr[it] = XBF16 ? *(const vec16*)((const bf16_t*)xv + t * (int64_t)d + col)
                     : *(const vec16*)((const float*)xv + t * (int64_t)d + col);
    }
  }

  const int nv4 = E * d / 4;
  for (int v = tid; v < nv4; v += 256) ((float4*)wsm)[v] = ((const float4*)Wg)[v];
  __syncthreads();

  double acc[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) acc[e] = 0.0;
  if (t < T) {
#pragma unroll
    for (int it = 0; it < KS_XV; ++it) {
      const int col = (lane + KS_LPT * it) * XW;
      if (col < d) {
        float f[8];
        if (XBF16) {
          unpack_bf16x8(xr[it], f);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) f[q] = __uint_as_float(xr[it].w[q]);
        }
#pragma unroll
        for (int e = 0; e < EP; ++e) {
          if (e < E) {
            const float4 w0 = *(const float4*)(wsm + e * d + col);
            double a = acc[e];
            a = fma((double)f[0], (double)w0.x, a);
            a = fma((double)f[1], (double)w0.y, a);
            a = fma((double)f[2], (double)w0.z, a);
            a = fma((double)f[3], (double)w0.w, a);
            if (XBF16) {
              const float4 w1 = *(const float4*)(wsm + e * d + col + 4);
              a = fma((double)f[4], (double)w1.x, a);
              a = fma((double)f[5], (double)w1.y, a);
              a = fma((double)f[6], (double)w1.z, a);
              a = fma((double)f[7], (double)w1.w, a);
            }
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
  token_epilogue<TE, KS_LPT>(r, lane, t, t < T, E, k, bg, bsel, logits, lse_out, topk_idx, topk_gate,
                             noise, sigma);
}

template <int EP>
static hipError_t launch_router_ksplit(const void* x, bool xbf16, int64_t T, int d, const float* Wg,
                                       const float* bg, const float* bsel, int E, int k,
                                       float* logits, float* lse, int32_t* idx, float* gate,
                                       const float* noise, double sigma, hipStream_t st) {
  const dim3 grid((unsigned)((T + KS_TPB - 1) / KS_TPB));
  const size_t lds = (size_t)E * d * sizeof(float);
  if (xbf16)
    hipLaunchKernelGGL((router_ksplit_kernel<EP, true>), grid, dim3(256), lds, st, x, T, d, Wg, bg,
                       bsel, E, k, logits, lse, idx, gate, noise, sigma);
  else
    hipLaunchKernelGGL((router_ksplit_kernel<EP, false>), grid, dim3(256), lds, st, x, T, d, Wg, bg,
                       bsel, E, k, logits, lse, idx, gate, noise, sigma);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MFMA path for bf16 x and large E * d
//
// W_g is split exactly into three bf16 parts, W = hi + mid + lo (truncations:
// hi keeps the top 8 significand bits, mid the next 8, lo the rest, which fits
// because fp32 has 24).  Every product x * part is exact in fp32, so a bf16
// MFMA GEMM of x against the stacked parts [hi; mid; lo] (N = 3E, K = d, fp32
// accumulation) gives three fp32 partial logits per (token, expert); the
// finish kernel adds them and the router bias in fp64.  The fp32
// accumulations are the only rounding; every token with two consecutive top
// scores within kRefineRel of each other is recomputed exactly in fp64.
// ---------------------------------------------------------------------------
constexpr double kRefineRel = 5e-5;

__global__ void router_split_kernel(const float* __restrict__ Wg, int E, int d,
                                    bf16_t* __restrict__ Ws, int32_t* __restrict__ count) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *count = 0;  // refine list, filled later on this stream
  const int64_t n = (int64_t)E * d;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float w = Wg[i];
    const float hi = __uint_as_float(__float_as_uint(w) & 0xffff0000u);
    const float r1 = w - hi;  // exact: the low 16 significand bits of w
    const float mid = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
    const float lo = r1 - mid;  // exact, at most 8 significand bits
    Ws[i] = (bf16_t)(__float_as_uint(hi) >> 16);
    Ws[n + i] = (bf16_t)(__float_as_uint(mid) >> 16);
    Ws[2 * n + i] = (bf16_t)(__float_as_uint(lo) >> 16);
  }
}

// Per token: logits = hi + mid + lo partials (fp64) + b_g, softmax / top-k /
// gates, near-tie flag.  NXE lanes per token, as in the other layouts.
// Flagged tokens are appended to `list` (their order there is arbitrary; each
// is recomputed on its own, so results do not depend on it).
template <int EP>
__global__ __launch_bounds__(256) void router_finish_kernel(
    const float* __restrict__ part, int64_t T, int E, int k, const float* __restrict__ bg,
    const float* __restrict__ bsel, float* __restrict__ logits, float* __restrict__ lse_out,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate, int32_t* __restrict__ count,
    int32_t* __restrict__ list, const float* __restrict__ noise, double sigma) {
  constexpr int NXE = (EP >= 256) ? 32 : 16;
  constexpr int TE = EP / NXE;
  const int tid = threadIdx.x;
  const int eg = tid % NXE;
  const int64_t t = (int64_t)blockIdx.x * (256 / NXE) + tid / NXE;
  double acc[TE];
#pragma unroll
  for (int j = 0; j < TE; ++j) {
    const int e = eg + NXE * j;
    double a = 0.0;
    if (t < T && e < E) {
      const float* p = part + t * (int64_t)(3 * E) + e;
      a = (double)p[0] + (double)p[E] + (double)p[2 * E];
    }
    acc[j] = a;
  }
  const bool near = token_epilogue<TE, NXE>(acc, eg, t, t < T, E, k, bg, bsel, logits, lse_out,
                                            topk_idx, topk_gate, noise, sigma, kRefineRel);
  if (near && t < T && eg == 0) list[atomicAdd(count, 1)] = (int32_t)t;
}

// Exact fp64 recomputation of the listed tokens, one token per block at a time.
// Wave w computes experts w, w + 8, ...: lanes stride the row in float4 chunks
// (products of bf16 and fp32 are exact in fp64) for two experts at once so
// plenty of loads are in flight, then wave 0 redoes the epilogue.
constexpr int kRefineThreads = 512;

template <int EP>
__global__ __launch_bounds__(kRefineThreads) void router_refine_kernel(
    const bf16_t* __restrict__ x, int d, const float* __restrict__ Wg, const float* __restrict__ bg,
    const float* __restrict__ bsel, int E, int k, const int32_t* __restrict__ count,
    const int32_t* __restrict__ list, float* __restrict__ logits, float* __restrict__ lse_out,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate, const float* __restrict__ noise,
    double sigma) {
  constexpr int TE = (EP + 63) / 64;
  constexpr int NWAVE = kRefineThreads / 64;
  __shared__ double s_h[EP];
  extern __shared__ float s_x[];  // one token row, fp32
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = *count;
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int64_t t = list[i];
    for (int j = tid; j < d; j += kRefineThreads) s_x[j] = bf16_to_f32(x[t * (int64_t)d + j]);
    __syncthreads();
    for (int e0 = wave; e0 < E; e0 += 2 * NWAVE) {
      const int e1 = e0 + NWAVE;
      const float4* w0 = (const float4*)(Wg + (int64_t)e0 * d);
      const float4* w1 = (const float4*)(Wg + (int64_t)(e1 < E ? e1 : e0) * d);
      double a0 = 0.0, a1 = 0.0;
#pragma unroll 4
      for (int q = lane; q < d / 4; q += 64) {
        const float4 u = w0[q], v = w1[q];
        const float4 xv = ((const float4*)s_x)[q];
        a0 = fma((double)xv.x, (double)u.x, a0); a0 = fma((double)xv.y, (double)u.y, a0);
        a0 = fma((double)xv.z, (double)u.z, a0); a0 = fma((double)xv.w, (double)u.w, a0);
        a1 = fma((double)xv.x, (double)v.x, a1); a1 = fma((double)xv.y, (double)v.y, a1);
        a1 = fma((double)xv.z, (double)v.z, a1); a1 = fma((double)xv.w, (double)v.w, a1);
      }
#pragma unroll
      for (int m = 32; m > 0; m >>= 1) {
        a0 += __shfl_xor(a0, m, 64);
        a1 += __shfl_xor(a1, m, 64);
      }
      if (lane == 0) {
        s_h[e0] = a0;
        if (e1 < E) s_h[e1] = a1;
      }
    }
    __syncthreads();
    if (wave == 0) {
      double acc[TE];
#pragma unroll
      for (int j = 0; j < TE; ++j) {
        const int e = lane + 64 * j;
        acc[j] = e < E ? s_h[e] : 0.0;
      }
      token_epilogue<TE, 64>(acc, lane, t, true, E, k, bg, bsel, logits, lse_out, topk_idx, topk_gate,
                             noise, sigma);
    }
    __syncthreads();
  }
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

size_t router_mfma_ws_bytes(int64_t T, int d, int E) {
  return align256((size_t)3 * E * d * sizeof(bf16_t)) + align256((size_t)T * 3 * E * sizeof(float)) +
         256 + align256((size_t)T * sizeof(int32_t));
}

bool router_uses_mfma(bool xbf16, int d, int E) {
  return xbf16 && E > 16 && d % 32 == 0 && !((int64_t)E * d * 4 <= 65536 && E <= 64);
}

template <int EP>
static hipError_t launch_router_mfma(const void* x, int64_t T, int d, const float* Wg,
                                     const float* bg, const float* bsel, int E, int k,
                                     float* logits, float* lse, int32_t* idx, float* gate,
                                     const float* noise, double sigma, void* ws, hipStream_t st) {
  char* w8 = (char*)ws;
  bf16_t* Ws = (bf16_t*)w8;
  w8 += align256((size_t)3 * E * d * sizeof(bf16_t));
  float* part = (float*)w8;
  w8 += align256((size_t)T * 3 * E * sizeof(float));
  int32_t* count = (int32_t*)w8;
  int32_t* list = (int32_t*)(w8 + 256);
  const int64_t n = (int64_t)E * d;
  const int64_t nb = (n + 255) / 256;
  hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)(nb < 4096 ? nb : 4096)), dim3(256), 0, st, Wg,
                     E, d, Ws, count);
  GemmArgs g{};
  g.A = x; g.group_offset = nullptr; g.G = 1; g.dense_M = T; g.max_rows = T;
  g.B = Ws; g.N = 3 * E; g.K = d; g.S = 1; g.Kseg = d; g.bias = nullptr; g.C = part;
  g.act = -1; g.sq_part = nullptr; g.out_f32 = true;
  hipError_t e = launch_gemm_bf16(g, st);
  if (e != hipSuccess) return e;
  constexpr int NXE = (EP >= 256) ? 32 : 16;
  const int64_t tpb = 256 / NXE;
  hipLaunchKernelGGL((router_finish_kernel<EP>), dim3((unsigned)((T + tpb - 1) / tpb)), dim3(256), 0, st,
                     part, T, E, k, bg, bsel, logits, lse, idx, gate, count, list, noise, sigma);
  const unsigned nref = (unsigned)(T < 1024 ? T : 1024);
  hipLaunchKernelGGL((router_refine_kernel<EP>), dim3(nref), dim3(kRefineThreads), (size_t)d * sizeof(float),
                     st, (const bf16_t*)x, d, Wg, bg, bsel, E, k, count, list, logits, lse, idx, gate,
                     noise, sigma);
  return hipGetLastError();
}

template <int EP>
static hipError_t launch_router_ep(const void* x, int xt, int64_t T, int d, const float* Wg,
                                   const float* bg, const float* bsel, int E, int k, float* logits,
                                   float* lse, int32_t* idx, float* gate, const float* noise,
                                   double sigma, hipStream_t st) {
  using C = RouterCfg<EP>;
  const dim3 grid((unsigned)((T + C::BT - 1) / C::BT));
  if (xt == XT_BF16)
    hipLaunchKernelGGL((router_kernel<EP, XT_BF16>), grid, dim3(C::NT), 0, st, x, T, d, Wg, bg, bsel, E,
                       k, logits, lse, idx, gate, noise, sigma);
  else if (xt == XT_F32)
    hipLaunchKernelGGL((router_kernel<EP, XT_F32>), grid, dim3(C::NT), 0, st, x, T, d, Wg, bg, bsel,
                       E, k, logits, lse, idx, gate, noise, sigma);
  else
    hipLaunchKernelGGL((router_kernel<EP, XT_F64>), grid, dim3(C::NT), 0, st, x, T, d, Wg, bg, bsel,
                       E, k, logits, lse, idx, gate, noise, sigma);
  return hipGetLastError();
}

static hipError_t launch_router_e_split(const void* x, int xt, int64_t T, int d, const float* Wg,
                                        const float* bg, const float* bsel, int E, int k,
                                        float* logits, float* lse, int32_t* idx, float* gate,
                                        const float* noise, double sigma, hipStream_t st) {
#define MOE_ROUTER_EP(EPV) \
  return launch_router_ep<EPV>(x, xt, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, noise, sigma, st)
  if (E <= 8) MOE_ROUTER_EP(8);
  if (E <= 16) MOE_ROUTER_EP(16);
  if (E <= 32) MOE_ROUTER_EP(32);
  if (E <= 64) MOE_ROUTER_EP(64);
  if (E <= 128) MOE_ROUTER_EP(128);
  MOE_ROUTER_EP(256);
#undef MOE_ROUTER_EP
}

hipError_t launch_router(const void* x, bool xbf16, int64_t T, int d, const float* Wg,
                         const float* bg, const float* bsel, int E, int k, float* logits,
                         float* lse, int32_t* idx, float* gate, const float* noise, double sigma,
                         void* ws, hipStream_t st) {
  if (router_uses_mfma(xbf16, d, E)) {
#define MOE_ROUTER_MFMA(EPV) \
  return launch_router_mfma<EPV>(x, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, noise, sigma, ws, st)
    if (E <= 64) MOE_ROUTER_MFMA(64);
    if (E <= 128) MOE_ROUTER_MFMA(128);
    MOE_ROUTER_MFMA(256);
#undef MOE_ROUTER_MFMA
  }
  // K-split when W_g fits in 64 KB of LDS, E <= 64 and the row fits KS_XV vectors a lane
  if ((int64_t)E * d * 4 <= 65536 && E <= 64 && d <= KS_LPT * KS_XV * (xbf16 ? 8 : 4)) {
#define MOE_ROUTER_KS(EPV) \
  return launch_router_ksplit<EPV>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, noise, sigma, st)
    if (E <= 8) MOE_ROUTER_KS(8);
    if (E <= 16) MOE_ROUTER_KS(16);
    if (E <= 32) MOE_ROUTER_KS(32);
    MOE_ROUTER_KS(64);
#undef MOE_ROUTER_KS
  }
  return launch_router_e_split(x, xbf16 ? XT_BF16 : XT_F32, T, d, Wg, bg, bsel, E, k, logits, lse, idx,
                               gate, noise, sigma, st);
}

template <int HP>
static hipError_t launch_mlp_hidden(const void* x, bool xbf16, int64_t T, int d, const float* gW1,
                                    const float* gb1, int H, double* hidden, hipStream_t st) {
  using C = RouterCfg<HP>;
  const dim3 grid((unsigned)((T + C::BT - 1) / C::BT));
  if (xbf16)
    hipLaunchKernelGGL((mlp_gate_hidden_kernel<HP, XT_BF16>), grid, dim3(C::NT), 0, st, x, T, d, gW1, gb1, H,
                       hidden);
  else
    hipLaunchKernelGGL((mlp_gate_hidden_kernel<HP, XT_F32>), grid, dim3(C::NT), 0, st, x, T, d, gW1, gb1, H,
                       hidden);
  return hipGetLastError();
}

size_t mlp_router_ws_bytes(int64_t T, int H) { return align256((size_t)T * (size_t)H * sizeof(double)); }

hipError_t launch_mlp_router(const void* x, bool xbf16, int64_t T, int d, const float* gW1,
                             const float* gb1, int H, const float* gW2, const float* gb2,
                             const float* bsel, int E, int k, float* logits, float* lse, int32_t* idx,
                             float* gate, const float* noise, double sigma, void* ws, hipStream_t st) {
  double* hidden = (double*)ws;
  hipError_t e;
  if (H <= 8) e = launch_mlp_hidden<8>(x, xbf16, T, d, gW1, gb1, H, hidden, st);
  else if (H <= 16) e = launch_mlp_hidden<16>(x, xbf16, T, d, gW1, gb1, H, hidden, st);
  else if (H <= 32) e = launch_mlp_hidden<32>(x, xbf16, T, d, gW1, gb1, H, hidden, st);
  else if (H <= 64) e = launch_mlp_hidden<64>(x, xbf16, T, d, gW1, gb1, H, hidden, st);
  else if (H <= 128) e = launch_mlp_hidden<128>(x, xbf16, T, d, gW1, gb1, H, hidden, st);
  else e = launch_mlp_hidden<256>(x, xbf16, T, d, gW1, gb1, H, hidden, st);
  if (e != hipSuccess) return e;
  return launch_router_e_split(hidden, XT_F64, T, H, gW2, gb2, bsel, E, k, logits, lse, idx, gate, noise,
                               sigma, st);
}

}  // namespace moe
