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
//    sums of its experts.  Many more tokens in flight for small E.  Small
//    batches give each of those 16 slices two lanes, one per half of the
//    experts (same products, same order, same bits), for twice the waves.

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "gemm_tiles.h"
#include "lds_ring.h"

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

template <int M>
__device__ __forceinline__ float xor_lane_f(float v) {
  return __int_as_float(xor_lane<M>(__float_as_int(v)));
}

// Reductions over NXE consecutive lanes, partners at lane ^ 1, ^ 2, ^ 4, ...
// in that order (every lane ends with the same value).
template <int NXE>
__device__ __forceinline__ double group_max(double v) {
  if constexpr (NXE > 1) v = fmax(v, xor_lane_d<1>(v));
  if constexpr (NXE > 2) v = fmax(v, xor_lane_d<2>(v));
  if constexpr (NXE > 4) v = fmax(v, xor_lane_d<4>(v));
  if constexpr (NXE > 8) v = fmax(v, xor_lane_d<8>(v));
  if constexpr (NXE > 16) v = fmax(v, xor_lane_d<16>(v));
  if constexpr (NXE > 32) v = fmax(v, xor_lane_d<32>(v));
  return v;
}

template <int NXE>
__device__ __forceinline__ float group_sumf(float v) {
  if constexpr (NXE > 1) v += xor_lane_f<1>(v);
  if constexpr (NXE > 2) v += xor_lane_f<2>(v);
  if constexpr (NXE > 4) v += xor_lane_f<4>(v);
  if constexpr (NXE > 8) v += xor_lane_f<8>(v);
  if constexpr (NXE > 16) v += xor_lane_f<16>(v);
  if constexpr (NXE > 32) v += xor_lane_f<32>(v);
  return v;
}

// One step of the (score desc, index asc) argmax across lanes; carries x.
// The comparisons are combined with bitwise operators and the results
// selected, so the step is straight-line code (with the short-circuit forms
// the compiler branched on each comparison).
template <int M>
__device__ __forceinline__ void argmax_step(double& s, int& e, float& x) {
  const double so = xor_lane_d<M>(s);
  const int eo = xor_lane<M>(e);
  const float xo = xor_lane_f<M>(x);
  const bool take = (so > s) | ((so == s) & (eo < e));
  s = take ? so : s;
  e = take ? eo : e;
  x = take ? xo : x;
}

template <int NXE>
__device__ __forceinline__ void group_argmax(double& s, int& e, float& x) {
  if constexpr (NXE > 1) argmax_step<1>(s, e, x);
  if constexpr (NXE > 2) argmax_step<2>(s, e, x);
  if constexpr (NXE > 4) argmax_step<4>(s, e, x);
  if constexpr (NXE > 8) argmax_step<8>(s, e, x);
  if constexpr (NXE > 16) argmax_step<16>(s, e, x);
  if constexpr (NXE > 32) argmax_step<32>(s, e, x);
}

// Optional per-token record of the epilogue: the softmax mass per expert and
// the lse (this token's LDS rows), and a count per selected expert (LDS
// integer atomics into the block's histogram: order-free).
struct RouterTap {
  float* p;     // [E]
  float* lse;   // [1]
  int* hist;    // [E], shared by the block
};

// Router bias b_g and selection bias b_sel of the experts lane eg holds in the
// epilogue below (0 where absent; rows past E read expert E - 1, unused).  All
// loads are issued together; a kernel may take them before its main loop so
// the epilogue does not wait on them.
template <int TE>
struct RouterBias {
  float g[TE], s[TE];
};

// Zeros read in place of an absent bias, so the loads need no branch (a
// load under a branch whose result is converted gets its wait inside it).
__device__ float kNoBias[kMaxExperts];

template <int TE, int NXE>
__device__ __forceinline__ RouterBias<TE> load_router_bias(const float* __restrict__ bg,
                                                           const float* __restrict__ bsel, int eg, int E) {
  const float* pg = bg != nullptr ? bg : kNoBias;
  const float* ps = bsel != nullptr ? bsel : kNoBias;
  RouterBias<TE> b;
#pragma unroll
  for (int j = 0; j < TE; ++j) {
    const int e = eg + NXE * j < E ? eg + NXE * j : E - 1;
    b.g[j] = pg[e];
    b.s[j] = ps[e];
  }
  return b;
}

// Per-token epilogue.  The NXE lanes of a token hold its fp64 dot products
// (router bias not yet added): lane eg holds experts e = eg + NXE j, j < TE.
// With noise != nullptr the logits are h + sigma * noise[t, e] (noisy top-k,
// page "Code Walkthrough -- SER", the gating / routing path: training noise is
// added to the logits before selection), and the gate temperature tau > 0
// (the same page's gate-forward argument) divides them: z = (h + sigma n) /
// tau in fp64.  Everything after uses z: the stored logits, lse, selection on
// z + b_sel, the gates and the statistics.  tau = 1 skips the division.
// Writes logits, lse, top-k indices and gates for token t (when live).
// With flag_rel > 0 it returns true (on every lane of the token) when two
// consecutive scores among the k + 1 highest (k when k = E) are closer than
// flag_rel * max(1, |score|): the selected set or its listed order could then
// change within the logits' rounding error.
// Every lane of the wave must be active (the cross-lane steps use DPP).
template <int TE, int NXE>
__device__ __forceinline__ bool token_epilogue(const double (&acc)[TE], int eg, int64_t t, bool live,
                                               int E, int k, const float* __restrict__ bg,
                                               const float* __restrict__ bsel,
                                               float* __restrict__ logits, float* __restrict__ lse_out,
                                               int32_t* __restrict__ topk_idx,
                                               float* __restrict__ topk_gate,
                                               const float* __restrict__ noise, double sigma, double tau,
                                               double flag_rel = 0.0, RouterTap* tap = nullptr,
                                               const RouterBias<TE>* pre = nullptr) {
  const double NEG = -__builtin_huge_val();
  // every bias and noise load is issued before the first is used (a load
  // under a per-expert branch gets a wait of its own)
  const RouterBias<TE> rb = pre != nullptr ? *pre : load_router_bias<TE, NXE>(bg, bsel, eg, E);
  float nz[TE];
#pragma unroll
  for (int j = 0; j < TE; ++j) nz[j] = 0.f;
  if (noise != nullptr) {  // uniform
    const float* pn = live ? noise + t * E : kNoBias;
#pragma unroll
    for (int j = 0; j < TE; ++j) nz[j] = pn[eg + NXE * j < E ? eg + NXE * j : E - 1];
  }
  double h[TE], s[TE];
  double m = NEG;
#pragma unroll
  for (int j = 0; j < TE; ++j) {
    const int e = eg + NXE * j;
    const bool ok = e < E;
    double hv = acc[j] + (ok ? (double)rb.g[j] : 0.0);
    if (noise != nullptr && live && ok) hv += sigma * (double)nz[j];
    h[j] = ok ? hv : NEG;
  }
  if (tau != 1.0) {  // uniform
    // a real branch: the empty asm keeps the fp64 divisions from being
    // computed (and selected away) at tau = 1.  -inf / tau stays -inf.
    asm volatile("");
#pragma unroll
    for (int j = 0; j < TE; ++j) h[j] = h[j] / tau;
  }
#pragma unroll
  for (int j = 0; j < TE; ++j) {
    s[j] = (eg + NXE * j < E) ? h[j] + (double)rb.s[j] : NEG;
    m = fmax(m, h[j]);
  }
  m = group_max<NXE>(m);
  // exp(h - m) in fp32 for every expert; the lse uses their sum, the gates
  // the selected ones
  float ex[TE];
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < TE; ++j) {
    ex[j] = (eg + NXE * j < E) ? expf((float)(h[j] - m)) : 0.f;
    se += ex[j];
  }
  se = group_sumf<NXE>(se);
  if (live) {
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const int e = eg + NXE * j;
      if (e < E) logits[t * E + e] = (float)h[j];
    }
    if (eg == 0) lse_out[t] = (float)(m + (double)logf(se));
  }
  if (tap != nullptr) {
    // the softmax mass as the statistics take it: expf(logit - lse) on the
    // stored fp32 values
    const float lse_f = (float)(m + (double)logf(se));
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const int e = eg + NXE * j;
      if (e < E) tap->p[e] = expf((float)h[j] - lse_f);
    }
    if (eg == 0) *tap->lse = lse_f;
  }
  // k argmax rounds in selection order (one more for the near-tie flag); the
  // lane owning a selected expert records its round, and once the sum of the
  // selected exp(h - m) is known writes that expert's index and gate
  float gsum = 0.f;
  bool near = false;
  double prev = 0.0;
  uint32_t taken = 0;
  int rank[TE];
#pragma unroll
  for (int j = 0; j < TE; ++j) rank[j] = 0;
  const int rounds = (flag_rel > 0.0 && k < E) ? k + 1 : k;
  for (int r = 0; r < rounds; ++r) {
    double bs = NEG;
    int be = 0x7fffffff;
    float bx = 0.f;
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const int e = eg + NXE * j;
      const bool ok = (e < E) & (((taken >> j) & 1u) == 0u);
      const bool take = ok & ((s[j] > bs) | ((s[j] == bs) & (e < be)));
      bs = take ? s[j] : bs;
      be = take ? e : be;
      bx = take ? ex[j] : bx;
    }
    group_argmax<NXE>(bs, be, bx);
    if (flag_rel > 0.0) {
      if (r > 0 && prev - bs < flag_rel * fmax(1.0, fabs(prev))) near = true;
      prev = bs;
    }
    if (r == k) break;  // the (k+1)-th score only feeds the flag
    if (be % NXE == eg) {
      const int jb = be / NXE;
      taken |= 1u << jb;
#pragma unroll
      for (int j = 0; j < TE; ++j)
        if (j == jb) rank[j] = r;
    }
    gsum += bx;
  }
  if (live) {
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      if ((taken >> j) & 1u) {
        topk_idx[t * k + rank[j]] = eg + NXE * j;
        topk_gate[t * k + rank[j]] = ex[j] / gsum;
        if (tap != nullptr) atomicAdd(&tap->hist[eg + NXE * j], 1);
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
    float* __restrict__ topk_gate, const float* __restrict__ noise, double sigma, double tau) {
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
                            topk_gate, noise, sigma, tau);
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
    w[q] = keep + xor_lane_d<O>(send);
  }
}

constexpr int KS_LPT = 16;    // column slices per token (a slice: one lane, or two splitting the experts)
constexpr int KS_TPB = 16;    // tokens per block (256 threads, 512 with split experts)
static_assert(KS_TPB == kStatsSub, "a counting router block is one statistics sub-block");
constexpr int KS_XV = 16;     // x vectors per lane: d <= 16 * 16 * 8 (bf16) or 16 * 16 * 4 (fp32)
constexpr int KS_FB = 4;      // W_g float4 loads a thread has in flight during the LDS fill

// LDS layout of W_g in the K-split kernel.  A token's 16 lanes read the row in
// chunks of CH = 16 * XW columns, lane l taking columns l * XW .. l * XW + XW - 1
// of each chunk (XW = 8 for bf16 x, 4 for fp32 x).  Inside a chunk the float4
// quarter q of lane l's columns sits at float4 index q * 16 + l, so one
// ds_read_b128 of the 16 lanes covers 256 contiguous bytes (no bank
// conflicts).  Each expert row is padded to whole chunks.
__host__ __device__ constexpr int ks_chunk_cols(bool xbf16) { return KS_LPT * (xbf16 ? 8 : 4); }

__host__ __device__ inline int ks_row_float4(int d, bool xbf16) {
  const int ch = ks_chunk_cols(xbf16);
  return (d + ch - 1) / ch * (ch / 4);
}

// Experts are padded to EP rows of zeros so the inner loop needs no expert guard.
static int ks_expert_rows(int E) { return E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64; }

static size_t ks_lds_bytes(int E, int d, bool xbf16) {
  return (size_t)ks_expert_rows(E) * ks_row_float4(d, xbf16) * sizeof(float4);
}

// SPLIT: two lanes per column slice, lane 16 h + s of a token's 32 taking
// experts h EP / 2 .. (h + 1) EP / 2 - 1 of slice s (512 threads a block).  For
// one wave a SIMD the fp64 FMA chains stall on their latency (measured on
// MI355X: 9.7 cycles per wave instruction with one wave, 5.8 with two, 4.8
// with eight); after the K loop the two halves swap their sums, so every lane
// holds what the unsplit lane holds and the reduction and epilogue are the
// same code.
template <int EP, bool XBF16, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? 512 : 256) void router_ksplit_kernel(
    const void* __restrict__ xv, int64_t T, int d, const float* __restrict__ Wg,
    const float* __restrict__ bg, const float* __restrict__ bsel, int E, int k,
    float* __restrict__ logits, float* __restrict__ lse_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, const float* __restrict__ noise, double sigma, double tau,
    int32_t* __restrict__ hist16, double* __restrict__ p16) {
  extern __shared__ float4 wsm[];  // W_g, fp32, in the chunked layout above
  // fused routing pass (hist16 != nullptr): this block's 16 tokens as one
  // counting unit and one statistics sub-partial
  __shared__ float tap_p[KS_TPB][EP];
  __shared__ float tap_lse[KS_TPB];
  __shared__ int tap_hist[EP];
  // split: the reduced sums of each token's 16 slices, handed to waves 0-3
  __shared__ double s_r[SPLIT ? KS_TPB * KS_LPT : 1][(EP >= 16) ? EP / 16 : 1];
  constexpr int XW = XBF16 ? 8 : 4;   // elements per 16-byte x vector
  constexpr int CH = KS_LPT * XW;     // columns per chunk
  constexpr int CH4 = CH / 4;         // float4 per chunk
  // chunks a 64 KB W_g copy of EP rows can hold: the most x vectors a lane needs
  constexpr int XV = (16384 / (EP * CH)) < KS_XV ? 16384 / (EP * CH) : KS_XV;
  static_assert(XV >= 1, "W_g rows do not fit the LDS budget");
  constexpr int NT = KS_TPB * KS_LPT * (SPLIT ? 2 : 1);  // threads
  constexpr int EPH = SPLIT ? EP / 2 : EP;                 // experts a lane sums
  const int tid = threadIdx.x;
  const int lane = tid & (KS_LPT - 1);
  const int half = SPLIT ? (tid >> 4) & 1 : 0;
  const int64_t t = (int64_t)blockIdx.x * KS_TPB + tid / (NT / KS_TPB);
  const int row4 = ks_row_float4(d, XBF16);
  constexpr int TE = (EP >= 16) ? EP / 16 : 1;
  const RouterBias<TE> rb = load_router_bias<TE, KS_LPT>(bg, bsel, lane, E);  // used in the epilogue

  // this lane's slice of the token row, loaded before the W_g fill so both
  // loads are in flight together (at most XV vectors a lane); columns past
  // d (and rows past T) are zero
  const int nit = (d + CH - 1) / CH;
  vec16 xr[XV];
#pragma unroll
  for (int it = 0; it < XV; ++it) {
    const int col = it * CH + lane * XW;
    xr[it] = vec16{{0u, 0u, 0u, 0u}};
    if (t < T && col < d) {
      xr[it] = XBF16 ? *(const vec16*)((const bf16_t*)xv + t * (int64_t)d + col)
                     : *(const vec16*)((const float*)xv + t * (int64_t)d + col);
    }
  }

  if (hist16 != nullptr && tid < EP) tap_hist[tid] = 0;  // ordered before use by the fill's barrier

  // W_g -> LDS, EP rows (rows past E and columns past d are zero): KS_FB loads
  // in flight per thread, then their stores
  const int nv4 = EP * row4;
  for (int v0 = 0; v0 < nv4; v0 += NT * KS_FB) {
    float4 q[KS_FB];
#pragma unroll
    for (int i = 0; i < KS_FB; ++i) {
      const int v = v0 + tid + NT * i;
      q[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (v < nv4) {
        const int e = v / row4, r = v - e * row4;
        const int c = r / CH4, w = r - c * CH4;
        const int col = c * CH + (w & 15) * XW + (w >> 4) * 4;
        if (e < E && col < d) q[i] = *(const float4*)(Wg + (int64_t)e * d + col);
      }
    }
#pragma unroll
    for (int i = 0; i < KS_FB; ++i) {
      const int v = v0 + tid + NT * i;
      if (v < nv4) wsm[v] = q[i];
    }
  }
  __syncthreads();

  // no expert or column guards: the padding is zero (nit is uniform)
  double acc[EPH];
#pragma unroll
  for (int e = 0; e < EPH; ++e) acc[e] = 0.0;
#pragma unroll
  for (int it = 0; it < XV; ++it) {
    if (it < nit) {
      double f[XW];
      if constexpr (XBF16) {
        float g[8];
        unpack_bf16x8(xr[it], g);
#pragma unroll
        for (int q = 0; q < 8; ++q) f[q] = (double)g[q];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) f[q] = (double)__uint_as_float(xr[it].w[q]);
      }
      // all of this chunk's W_g quarters first, then one column at a time
      // across the experts: EP independent fp64 chains, no load-use stall
      // per expert
      const float4* wl = wsm + it * CH4 + lane + half * EPH * row4;
      constexpr int NQ = XW / 4;
      constexpr int GE = EPH < 8 ? EPH : 8;  // experts whose quarters are read together
#pragma unroll
      for (int e0 = 0; e0 < EPH; e0 += GE) {
        float4 w[GE][NQ];
#pragma unroll
        for (int e = 0; e < GE; ++e)
#pragma unroll
          for (int h = 0; h < NQ; ++h) w[e][h] = wl[(e0 + e) * row4 + 16 * h];
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
#pragma unroll
          for (int e = 0; e < GE; ++e) acc[e0 + e] = fma(f[4 * h + 0], (double)w[e][h].x, acc[e0 + e]);
#pragma unroll
          for (int e = 0; e < GE; ++e) acc[e0 + e] = fma(f[4 * h + 1], (double)w[e][h].y, acc[e0 + e]);
#pragma unroll
          for (int e = 0; e < GE; ++e) acc[e0 + e] = fma(f[4 * h + 2], (double)w[e][h].z, acc[e0 + e]);
#pragma unroll
          for (int e = 0; e < GE; ++e) acc[e0 + e] = fma(f[4 * h + 3], (double)w[e][h].w, acc[e0 + e]);
        }
      }
    }
  }

  // split halves: swap sums so both lanes of a slice hold all EP experts
  double all[EP];
  if constexpr (SPLIT) {
#pragma unroll
    for (int j = 0; j < EPH; ++j) {
      const double other = xor_lane_d<16>(acc[j]);
      all[j] = half ? other : acc[j];
      all[EPH + j] = half ? acc[j] : other;
    }
  } else {
#pragma unroll
    for (int e = 0; e < EP; ++e) all[e] = acc[e];
  }

  // reduce-scatter over the 16 lanes: lane l ends with experts l + 16 j
  double r[TE];
  if constexpr (EP == 8) {
    double a4[4], a2[2];
    double full[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) full[e] = all[e] + xor_lane_d<8>(all[e]);
    rs_halve<8, 4>(full, a4, lane);
    rs_halve<4, 2>(a4, a2, lane);
    rs_halve<2, 1>(a2, r, lane);
  } else {
    double b8[EP / 2], b4[EP / 4], b2[EP / 8];
    rs_halve<EP, 8>(all, b8, lane);
    rs_halve<EP / 2, 4>(b8, b4, lane);
    rs_halve<EP / 4, 2>(b4, b2, lane);
    rs_halve<EP / 8, 1>(b2, r, lane);
  }
  // for EP = 8, lanes 8..15 duplicate lanes 0..7; their expert ids lane >= 8 >= E are void
  if constexpr (SPLIT) {
    // the first half's sums go through LDS to waves 0-3 (16 lanes a token,
    // as unsplit), which run the epilogue; waves 4-7 skip it
    if (half == 0) {
#pragma unroll
      for (int j = 0; j < TE; ++j) s_r[(tid >> 5) * KS_LPT + lane][j] = r[j];
    }
    __syncthreads();
    if (tid < KS_TPB * KS_LPT) {  // uniform per wave
      double rr[TE];
#pragma unroll
      for (int j = 0; j < TE; ++j) rr[j] = s_r[tid][j];
      const int tl = tid / KS_LPT;
      const int64_t tt = (int64_t)blockIdx.x * KS_TPB + tl;
      RouterTap tap{tap_p[tl], &tap_lse[tl], tap_hist};
      token_epilogue<TE, KS_LPT>(rr, lane, tt, tt < T, E, k, bg, bsel, logits, lse_out, topk_idx, topk_gate,
                                 noise, sigma, tau, 0.0, hist16 != nullptr ? &tap : nullptr, &rb);
    }
  } else {
    const int tl = tid / KS_LPT;
    RouterTap tap{tap_p[tl], &tap_lse[tl], tap_hist};
    token_epilogue<TE, KS_LPT>(r, lane, t, t < T, E, k, bg, bsel, logits, lse_out, topk_idx, topk_gate,
                               noise, sigma, tau, 0.0, hist16 != nullptr ? &tap : nullptr, &rb);
  }
  if (hist16 == nullptr) return;  // uniform
  __syncthreads();
  // per expert: choices among the block's tokens and the softmax mass summed
  // in token order; thread E: the lse^2 sum (the statistics sub-partial)
  const int64_t t0 = (int64_t)blockIdx.x * KS_TPB;
  const int nt = (int)((T - t0) < KS_TPB ? (T - t0) : KS_TPB);
  if (tid < E) {
    float v[KS_TPB];
#pragma unroll
    for (int u = 0; u < KS_TPB; ++u) v[u] = tap_p[u][tid];
    double m = 0.0;
#pragma unroll
    for (int u = 0; u < KS_TPB; ++u)
      if (u < nt) m += (double)v[u];
    hist16[blockIdx.x * (int64_t)E + tid] = tap_hist[tid];
    p16[blockIdx.x * (int64_t)(E + 1) + tid] = m;
  } else if (tid == E) {
    float v[KS_TPB];
#pragma unroll
    for (int u = 0; u < KS_TPB; ++u) v[u] = tap_lse[u];
    double z = 0.0;
#pragma unroll
    for (int u = 0; u < KS_TPB; ++u)
      if (u < nt) z += (double)v[u] * (double)v[u];
    p16[blockIdx.x * (int64_t)(E + 1) + E] = z;
  }
}

template <int EP>
static hipError_t launch_router_ksplit(const void* x, bool xbf16, int64_t T, int d, const float* Wg,
                                       const float* bg, const float* bsel, int E, int k,
                                       float* logits, float* lse, int32_t* idx, float* gate,
                                       const float* noise, double sigma, double tau, int32_t* hist16,
                                       double* p16, hipStream_t st) {
  const int64_t blocks = (T + KS_TPB - 1) / KS_TPB;
  const dim3 grid((unsigned)blocks);
  const size_t lds = ks_lds_bytes(E, d, xbf16);
  // split experts when the batch gives at most one block (four waves) a CU
  const bool split = blocks <= kCus;
#define MOE_KS_LAUNCH(XB, SP)                                                                              \
  hipLaunchKernelGGL((router_ksplit_kernel<EP, XB, SP>), grid, dim3(SP ? 512 : 256), lds, st, x, T, d, Wg, bg, \
                     bsel, E, k, logits, lse, idx, gate, noise, sigma, tau, hist16, p16)
  if (xbf16) {
    if (split) MOE_KS_LAUNCH(true, true);
    else MOE_KS_LAUNCH(true, false);
  } else {
    if (split) MOE_KS_LAUNCH(false, true);
    else MOE_KS_LAUNCH(false, false);
  }
#undef MOE_KS_LAUNCH
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


// Row order of the 3E split rows: ew = 0, [hi; mid; lo] (row p E + e holds part
// p of expert e); ew > 0, groups of ew experts, each group's hi, mid and lo
// rows together (row 3 ew g + p ew + q holds part p of expert ew g + q), so
// that a wave owning one group's 3 ew columns holds all three partials of its
// experts.
__global__ void router_split_kernel(const float* __restrict__ Wg, int E, int d, int ew,
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
    const int e = (int)(i / d);
    const int64_t col = i - (int64_t)e * d;
    const int64_t r0 = ew > 0 ? (int64_t)(e / ew) * 3 * ew + e % ew : e;  // row of part 0
    const int64_t step = ew > 0 ? ew : E;                                   // rows between parts
    Ws[r0 * d + col] = (bf16_t)(__float_as_uint(hi) >> 16);
    Ws[(r0 + step) * d + col] = (bf16_t)(__float_as_uint(mid) >> 16);
    Ws[(r0 + 2 * step) * d + col] = (bf16_t)(__float_as_uint(lo) >> 16);
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
    int32_t* __restrict__ list, const float* __restrict__ noise, double sigma, double tau) {
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
                                            topk_idx, topk_gate, noise, sigma, tau, kRefineRel);
  if (near && t < T && eg == 0) list[atomicAdd(count, 1)] = (int32_t)t;
}

// The partials and the finish in one kernel, for E = EP: a block
// takes RW = 16 NW tokens against all 3E split-weight rows, and wave w owns
// tokens 16 w .. 16 w + 15 over every column, so after the K loop each lane
// holds the hi, mid and lo partials of the same experts.  The K loop runs
// 32-wide stages through an NS-stage LDS ring with the grouped GEMM's MFMA in
// the same K order, so the fp32 partials are the ones the GEMM writes; the
// fp64 logits ((hi + mid) + lo, the finish kernel's order) go through LDS to
// the same per-token epilogue, NXE lanes a token.  The results are those of
// the split GEMM and the finish kernel, without the 3E-column partials buffer.
template <int EP, int NW, int NS>
__global__ __launch_bounds__(64 * NW) void router_mfma_kernel(
    const bf16_t* __restrict__ x, int64_t T, int d, const bf16_t* __restrict__ Ws, int k,
    const float* __restrict__ bg, const float* __restrict__ bsel, float* __restrict__ logits,
    float* __restrict__ lse_out, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    int32_t* __restrict__ count, int32_t* __restrict__ list, const float* __restrict__ noise,
    double sigma, double tau) {
  constexpr int E = EP;
  constexpr int RW = 16 * NW;          // tokens a block
  constexpr int NR = RW + 3 * E;       // stage rows: the tokens, then hi, mid, lo weight rows
  constexpr int SLAB = NR * 64;        // 32 bf16 of K a row
  constexpr int LPW = NR / (16 * NW);  // 1 KB load instructions a wave per stage (16 rows each)
  constexpr int TN = 3 * E / 16;       // MFMA column tiles a wave
  static_assert(NR % (16 * NW) == 0, "stage rows split evenly over the waves");
  static_assert(NS >= 2 && NS <= 4, "2 to 4 stages");
  __shared__ __attribute__((aligned(1024))) char st0[SLAB];
  __shared__ __attribute__((aligned(1024))) char st1[SLAB];
  __shared__ __attribute__((aligned(1024))) char st2[NS > 2 ? SLAB : 16];
  __shared__ __attribute__((aligned(1024))) char st3[NS > 3 ? SLAB : 16];
  __shared__ double s_h[RW * E];
  char* const stages[4] = {st0, st1, st2, st3};
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * RW;

  // load slots: instruction j = wave + NW i fills rows 16 j .. 16 j + 15, lane l
  // row 16 j + l / 4 at physical chunk l % 4 (token rows past T reload row T - 1)
  const bf16_t* src[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = 16 * (wave + NW * i) + lane / 4;
    const int chunk = (lane % 4) ^ swz<1>(row);
    if (row < RW) {
      const int64_t t = t0 + row < T ? t0 + row : T - 1;
      src[i] = x + t * d + chunk * 8;
    } else {
      src[i] = Ws + (int64_t)(row - RW) * d + chunk * 8;
    }
  }
  const int nk = d / 32;
  auto issue = [&](int kt, int stage) {
    const int kk = (kt < nk ? kt : nk - 1) * 32;  // past the end: harmless reload
    char* base = stages[stage];
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + kk),
                                       (lds_ptr_t)(base + 16 * (wave + NW * i) * 64), 16, 0, 0);
  };
  // operand reads: lane (fr, fc) reads row fr of a 16-row tile at logical chunk fc
  const int fr = lane & 15, fc = lane >> 4;
  int a_rd, b_rd[TN];
  {
    const int R = wave * 16 + fr;
    a_rd = R * 64 + ((fc ^ swz<1>(R)) << 4);
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int R = RW + j * 16 + fr;
    b_rd[j] = R * 64 + ((fc ^ swz<1>(R)) << 4);
  }
  f32x4_t acc[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, s);
  auto step = [&](int kt, int stage) {
    wait_vmcnt<(NS - 2) * LPW>();  // this wave's loads of stage kt have landed
    slab_barrier();                 // ... and every other wave's
    issue(kt + NS - 1, (stage + NS - 1) % NS);
    const char* base = stages[stage];
    const bf16x8_t a = *(const bf16x8_t*)(base + a_rd);
    bf16x8_t b[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = *(const bf16x8_t*)(base + b_rd[j]);
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a, acc[j], 0, 0, 0);
  };
  int kt = 0;
  for (; kt + NS <= nk; kt += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) step(kt + s, s);
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (kt + s < nk) step(kt + s, s);
  wait_vmcnt<0>();
  __syncthreads();

  // lane (fr, fc) holds token 16 wave + fr at columns 16 j + 4 fc + r: hi for
  // column e, mid for E + e, lo for 2E + e (the + 0 is the GEMM's bias add)
#pragma unroll
  for (int j = 0; j < E / 16; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const double h = (double)(acc[j][r] + 0.f) + (double)(acc[E / 16 + j][r] + 0.f) +
                       (double)(acc[2 * E / 16 + j][r] + 0.f);
      s_h[(wave * 16 + fr) * E + j * 16 + fc * 4 + r] = h;
    }
  __syncthreads();
  constexpr int NXE = 16, TE = E / NXE, TPP = 64 * NW / NXE;  // lanes a token, experts a lane, tokens a pass
  const int eg = tid % NXE;
#pragma unroll 1
  for (int p = 0; p < RW / TPP; ++p) {
    const int tl = p * TPP + tid / NXE;
    const int64_t t = t0 + tl;
    double a[TE];
#pragma unroll
    for (int j = 0; j < TE; ++j) a[j] = s_h[tl * E + eg + NXE * j];
    const bool near = token_epilogue<TE, NXE>(a, eg, t, t < T, E, k, bg, bsel, logits, lse_out,
                                              topk_idx, topk_gate, noise, sigma, tau, kRefineRel);
    if (near && t < T && eg == 0) list[atomicAdd(count, 1)] = (int32_t)t;
  }
}

// The split-weight partials and the finish in one kernel for E = EP experts
// (EP a multiple of 64) and blocks of 128 tokens: eight waves in 2 x 4, wave
// (wm, wn) owning tokens 64 wm .. 64 wm + 63 against the 3 EP / 4 split rows
// of expert group wn (hi, mid, lo of experts EP / 4 wn .. EP / 4 (wn + 1) - 1,
// in the router_split_kernel grouped order), so each lane ends with the three
// partials of the same experts.  The K loop is the grouped GEMM's (32-wide
// stages through a 4-stage LDS ring, the 16 x 16 x 32 MFMA, K in order, the
// ping-pong schedule).  The fp64 logits, (hi + mid) + lo as the finish kernel
// adds them, go through LDS (over the idle ring) to the shared per-token
// epilogue, which lists the near-ties.  Every block reads the 3 EP split rows
// once, and x once; no partials buffer.  (Measured on MI355X, 32768 tokens,
// d 4096, 128 experts: 154 us against 159 us for the split GEMM alone plus
// 39 us for the finish kernel; 64-wide stages or no ping-pong measured the
// same.)
template <int EP>
struct RouterFusedCfg {
  static constexpr int NW = 8, NT = 64 * NW, WGM = 2, WGN = 4;
  static constexpr int RW = 128;                   // tokens a block
  static constexpr int EW = EP / WGN;              // experts a wave column
  static constexpr int WM = RW / WGM, WN = 3 * EW; // wave tile: 64 tokens x 3 EW split rows
  static constexpr int TM = WM / 16, TN = WN / 16, TH = EW / 16;  // MFMA tiles; tiles per part
  static constexpr int NR = RW + 3 * EP;           // stage rows: tokens, then split rows
  static constexpr int SLAB = NR * 64;             // 32 bf16 of K a row
  static constexpr int LPW = NR / (16 * NW);       // 1 KB load instructions a wave per stage
  static constexpr int NS = 4;
  static_assert(EP % 64 == 0, "whole 16-column tiles per part and wave");
  static_assert(NR % (16 * NW) == 0, "stage rows split evenly over the waves");
  static_assert(NS * SLAB >= RW * EP * 8, "the fp64 logits fit in the idle ring");
};

template <int EP>
__global__ __launch_bounds__(512) void router_fused_kernel(
    const bf16_t* __restrict__ x, int64_t T, int d, const bf16_t* __restrict__ Ws, int k,
    const float* __restrict__ bg, const float* __restrict__ bsel, float* __restrict__ logits,
    float* __restrict__ lse_out, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    int32_t* __restrict__ count, int32_t* __restrict__ list, const float* __restrict__ noise,
    double sigma, double tau) {
  using C = RouterFusedCfg<EP>;
  constexpr int E = EP, NW = C::NW, RW = C::RW, LPW = C::LPW, TM = C::TM, TN = C::TN, TH = C::TH;
  constexpr int NS = C::NS, SLAB = C::SLAB;
  __shared__ __attribute__((aligned(1024))) char ring[NS * SLAB];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int64_t t0 = (int64_t)blockIdx.x * RW;

  // load slots: instruction j = wave + NW i fills rows 16 j .. 16 j + 15, lane l
  // row 16 j + l / 4 at physical chunk l % 4 (token rows past T reload row T - 1)
  const bf16_t* src[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = 16 * (wave + NW * i) + lane / 4;
    const int chunk = (lane % 4) ^ swz<1>(row);
    if (row < RW) {
      const int64_t t = t0 + row < T ? t0 + row : T - 1;
      src[i] = x + t * d + chunk * 8;
    } else {
      src[i] = Ws + (int64_t)(row - RW) * d + chunk * 8;
    }
  }
  const int nk = d / 32;
  auto issue = [&](int kt, int stage) {
    const int kk = (kt < nk ? kt : nk - 1) * 32;  // past the end: harmless reload
    char* base = ring + stage * SLAB;
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + kk),
                                       (lds_ptr_t)(base + 16 * (wave + NW * i) * 64), 16, 0, 0);
  };
  // operand reads: lane (fr, fc) reads row fr of a 16-row tile at logical chunk fc
  const int fr = lane & 15, fc = lane >> 4;
  int a_rd[TM], b_rd[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int R = wm * C::WM + i * 16 + fr;
    a_rd[i] = R * 64 + ((fc ^ swz<1>(R)) << 4);
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int R = RW + wn * C::WN + j * 16 + fr;
    b_rd[j] = R * 64 + ((fc ^ swz<1>(R)) << 4);
  }
  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Ping-pong: waves 0-3 (token half 0) and 4-7 (token half 1) put one wave
  // of each on every SIMD; every wave runs, per stage j, MEM(j): refill stage
  // j - 1's buffer with its share of stage j + NS - 1, read stage j, wait for
  // its share of stage j + 1; barrier; MUL(j); barrier.  Half 1 passes one
  // extra barrier first (half 0 one after), so one wave a SIMD multiplies
  // while the other loads and reads.
  const int grp = wave >> 2;
  bf16x8_t fa[TM], fb[TN];
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, s);
  wait_vmcnt<(NS - 2) * LPW>();  // stage 0
  slab_barrier();
  if (grp == 1) slab_barrier();
  auto pp_step = [&](int kt, int stage) {
    __builtin_amdgcn_sched_barrier(0);
    issue(kt + NS - 1, (stage + NS - 1) % NS);
    const char* base = ring + stage * SLAB;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = *(const bf16x8_t*)(base + a_rd[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = *(const bf16x8_t*)(base + b_rd[j]);
    wait_vmcnt<(NS - 2) * LPW>();  // this wave's share of stage kt + 1
    slab_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    slab_barrier();
  };
  int kt = 0;
  for (; kt + NS <= nk; kt += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) pp_step(kt + s, s);
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (kt + s < nk) pp_step(kt + s, s);
  if (grp == 0) slab_barrier();
  wait_vmcnt<0>();
  __syncthreads();

  // lane (fr, fc) holds token wm WM + 16 i + fr at group columns 16 j + 4 fc + r:
  // tiles 0 .. TH - 1 the hi part of experts EW wn + 16 j + 4 fc + r, then mid,
  // then lo (the + 0 is the GEMM's bias add)
  double* s_h = (double*)ring;  // [RW][E]
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TH; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double h = (double)(acc[i][j][r] + 0.f) + (double)(acc[i][TH + j][r] + 0.f) +
                         (double)(acc[i][2 * TH + j][r] + 0.f);
        s_h[(wm * C::WM + i * 16 + fr) * E + C::EW * wn + j * 16 + fc * 4 + r] = h;
      }
  __syncthreads();
  // 8 lanes a token (16 experts a lane): each selection round's cross-lane
  // argmax is 3 exchange steps after 16 local comparisons, and the 128 tokens
  // take 2 passes (16 lanes a token, 4 steps after 8 comparisons over 4
  // passes, measured 4 us slower at 32768 tokens, d 4096)
  constexpr int NXE = 8, TE = E / NXE, TPP = C::NT / NXE;  // lanes a token, experts a lane, tokens a pass
  const int eg = tid % NXE;
#pragma unroll 1
  for (int p = 0; p < RW / TPP; ++p) {
    const int tl = p * TPP + tid / NXE;
    const int64_t t = t0 + tl;
    double a[TE];
#pragma unroll
    for (int j = 0; j < TE; ++j) a[j] = s_h[tl * E + eg + NXE * j];
    const bool near = token_epilogue<TE, NXE>(a, eg, t, t < T, E, k, bg, bsel, logits, lse_out,
                                              topk_idx, topk_gate, noise, sigma, tau, kRefineRel);
    if (near && t < T && eg == 0) list[atomicAdd(count, 1)] = (int32_t)t;
  }
}

// Exact recomputation of the listed tokens, in two kernels.
//  * dots: work items (8 listed tokens, 8 experts) spread over the grid; a
//    block's thread (e, l) sums columns 4 l + 128 q of expert e for all 8
//    tokens (products of bf16 and fp32 are exact in fp64), so each W_g row
//    is read once for 8 tokens; the 32 lanes of an expert then add up in a
//    fixed order.  h[i][e] (fp64) goes to the partials buffer, which no
//    longer holds partials by then.
//  * epilogue: one wave per listed token redoes the per-token epilogue on h.
constexpr int kRefineTok = 8;  // listed tokens a work item
constexpr int kRefineExp = 8;  // experts a work item (32 lanes each)

__global__ __launch_bounds__(256) void router_refine_dots_kernel(
    const bf16_t* __restrict__ x, int d, const float* __restrict__ Wg, int E,
    const int32_t* __restrict__ count, const int32_t* __restrict__ list, double* __restrict__ h) {
  const int n = *count;
  const int parts = (E + kRefineExp - 1) / kRefineExp;
  const int chunks = (n + kRefineTok - 1) / kRefineTok;
  const int tid = threadIdx.x;
  const int l = tid & 31;
  for (int64_t w = blockIdx.x; w < (int64_t)chunks * parts; w += gridDim.x) {  // uniform
    const int i0 = (int)(w / parts) * kRefineTok;
    const int e = (int)(w % parts) * kRefineExp + tid / 32;
    const bf16_t* xr[kRefineTok];
#pragma unroll
    for (int u = 0; u < kRefineTok; ++u) xr[u] = x + (int64_t)list[i0 + u < n ? i0 + u : n - 1] * d;
    double acc[kRefineTok];
#pragma unroll
    for (int u = 0; u < kRefineTok; ++u) acc[u] = 0.0;
    if (e < E) {
      const float* wr = Wg + (int64_t)e * d;
      for (int c = 4 * l; c < d; c += 128) {
        const float4 wv = *(const float4*)(wr + c);
        uint2 xv[kRefineTok];  // four bf16 a token
#pragma unroll
        for (int u = 0; u < kRefineTok; ++u) xv[u] = *(const uint2*)(xr[u] + c);
#pragma unroll
        for (int u = 0; u < kRefineTok; ++u) {
          acc[u] = fma((double)__uint_as_float(xv[u].x << 16), (double)wv.x, acc[u]);
          acc[u] = fma((double)__uint_as_float(xv[u].x & 0xffff0000u), (double)wv.y, acc[u]);
          acc[u] = fma((double)__uint_as_float(xv[u].y << 16), (double)wv.z, acc[u]);
          acc[u] = fma((double)__uint_as_float(xv[u].y & 0xffff0000u), (double)wv.w, acc[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRefineTok; ++u) {
      double a = acc[u];
      a += xor_lane_d<1>(a);
      a += xor_lane_d<2>(a);
      a += xor_lane_d<4>(a);
      a += xor_lane_d<8>(a);
      a += xor_lane_d<16>(a);
      if (l == 0 && e < E && i0 + u < n) h[(int64_t)(i0 + u) * E + e] = a;
    }
  }
}

template <int EP>
__global__ __launch_bounds__(256) void router_refine_epilogue_kernel(
    const double* __restrict__ h, const float* __restrict__ bg, const float* __restrict__ bsel, int E,
    int k, const int32_t* __restrict__ count, const int32_t* __restrict__ list,
    float* __restrict__ logits, float* __restrict__ lse_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, const float* __restrict__ noise, double sigma, double tau) {
  constexpr int TE = (EP + 63) / 64;
  const int n = *count;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = blockIdx.x * 4 + wave; i < n; i += gridDim.x * 4) {  // uniform per wave
    const int64_t t = list[i];
    double acc[TE];
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const int e = lane + 64 * j;
      acc[j] = e < E ? h[(int64_t)i * E + e] : 0.0;
    }
    token_epilogue<TE, 64>(acc, lane, t, true, E, k, bg, bsel, logits, lse_out, topk_idx, topk_gate,
                           noise, sigma, tau);
  }
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

size_t router_mfma_ws_bytes(int64_t T, int d, int E) {
  return align256((size_t)3 * E * d * sizeof(bf16_t)) + align256((size_t)T * 3 * E * sizeof(float)) +
         256 + align256((size_t)T * sizeof(int32_t));
}

bool router_uses_mfma(bool xbf16, int d, int E) {
  return xbf16 && E > 16 && d % 32 == 0 && !(ks_lds_bytes(E, d, xbf16) <= 65536 && E <= 64);
}

template <int EP>
static hipError_t launch_router_mfma(const void* x, int64_t T, int d, const float* Wg,
                                     const float* bg, const float* bsel, int E, int k,
                                     float* logits, float* lse, int32_t* idx, float* gate,
                                     const float* noise, double sigma, double tau, void* ws, hipStream_t st) {
  char* w8 = (char*)ws;
  bf16_t* Ws = (bf16_t*)w8;
  w8 += align256((size_t)3 * E * d * sizeof(bf16_t));
  float* part = (float*)w8;
  w8 += align256((size_t)T * 3 * E * sizeof(float));
  int32_t* count = (int32_t*)w8;
  int32_t* list = (int32_t*)(w8 + 256);
  const int64_t n = (int64_t)E * d;
  const int64_t nb = (n + 255) / 256;
  // 128 experts: the fused kernel over blocks of 128 tokens (every block
  // reads the 3 MB of split rows once from L2, x once)
  const bool fused128 = EP == 128 && E == EP;
  hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)(nb < 4096 ? nb : 4096)), dim3(256), 0, st, Wg,
                     E, d, fused128 ? E / 4 : 0, Ws, count);
  bool fused = false;
  if constexpr (EP == 128) {
    if (fused128) {
      hipLaunchKernelGGL((router_fused_kernel<128>), dim3((unsigned)((T + 127) / 128)), dim3(512), 0, st,
                         (const bf16_t*)x, T, d, Ws, k, bg, bsel, logits, lse, idx, gate, count, list, noise,
                         sigma, tau);
      fused = true;
    }
  }
  if constexpr (EP == 64) {
    // partials and finish in one kernel where it measured faster: 64 experts
    // and 256 or more blocks of 64 tokens (switch layer, T 16384, d 1024:
    // routing pass 48.7 -> 46.7 us).  With fewer tokens (two-wave blocks:
    // 64 experts at T 8192, d 2048, 60.6 -> 69.5 us) the GEMM and the finish
    // kernel stay ahead.  (128 experts take router_fused_kernel above, whose
    // blocks of 128 tokens read the split rows once per 128 tokens.)
    if (E == EP && T >= 64 * 256) {
      hipLaunchKernelGGL((router_mfma_kernel<EP, 4, 4>), dim3((unsigned)((T + 63) / 64)), dim3(256), 0, st,
                         (const bf16_t*)x, T, d, Ws, k, bg, bsel, logits, lse, idx, gate, count, list,
                         noise, sigma, tau);
      fused = true;
    }
  }
  if (!fused) {
    GemmArgs g{};
    g.A = x; g.group_offset = nullptr; g.G = 1; g.dense_M = T; g.max_rows = T;
    g.B = Ws; g.N = 3 * E; g.K = d; g.S = 1; g.Kseg = d; g.bias = nullptr; g.C = part;
    g.act = -1; g.sq_part = nullptr; g.out_f32 = true;
    hipError_t e = launch_gemm_bf16(g, st);
    if (e != hipSuccess) return e;
    constexpr int NXE = (EP >= 256) ? 32 : 16;
    const int64_t tpb = 256 / NXE;
    hipLaunchKernelGGL((router_finish_kernel<EP>), dim3((unsigned)((T + tpb - 1) / tpb)), dim3(256), 0, st,
                       part, T, E, k, bg, bsel, logits, lse, idx, gate, count, list, noise, sigma, tau);
  }
  // the listed tokens' exact logits go into the consumed partials buffer
  // (T E doubles <= T 3E floats)
  double* h = (double*)part;
  hipLaunchKernelGGL(router_refine_dots_kernel, dim3(512), dim3(256), 0, st, (const bf16_t*)x, d, Wg, E,
                     count, list, h);
  hipLaunchKernelGGL((router_refine_epilogue_kernel<EP>), dim3(256), dim3(256), 0, st, h, bg, bsel, E, k,
                     count, list, logits, lse, idx, gate, noise, sigma, tau);
  return hipGetLastError();
}

template <int EP>
static hipError_t launch_router_ep(const void* x, int xt, int64_t T, int d, const float* Wg,
                                   const float* bg, const float* bsel, int E, int k, float* logits,
                                   float* lse, int32_t* idx, float* gate, const float* noise,
                                   double sigma, double tau, hipStream_t st) {
  using C = RouterCfg<EP>;
  const dim3 grid((unsigned)((T + C::BT - 1) / C::BT));
  if (xt == XT_BF16)
    hipLaunchKernelGGL((router_kernel<EP, XT_BF16>), grid, dim3(C::NT), 0, st, x, T, d, Wg, bg, bsel, E,
                       k, logits, lse, idx, gate, noise, sigma, tau);
  else if (xt == XT_F32)
    hipLaunchKernelGGL((router_kernel<EP, XT_F32>), grid, dim3(C::NT), 0, st, x, T, d, Wg, bg, bsel,
                       E, k, logits, lse, idx, gate, noise, sigma, tau);
  else
    hipLaunchKernelGGL((router_kernel<EP, XT_F64>), grid, dim3(C::NT), 0, st, x, T, d, Wg, bg, bsel,
                       E, k, logits, lse, idx, gate, noise, sigma, tau);
  return hipGetLastError();
}

static hipError_t launch_router_e_split(const void* x, int xt, int64_t T, int d, const float* Wg,
                                        const float* bg, const float* bsel, int E, int k,
                                        float* logits, float* lse, int32_t* idx, float* gate,
                                        const float* noise, double sigma, double tau, hipStream_t st) {
#define MOE_ROUTER_EP(EPV) \
  return launch_router_ep<EPV>(x, xt, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, noise, sigma, tau, st)
  if (E <= 8) MOE_ROUTER_EP(8);
  if (E <= 16) MOE_ROUTER_EP(16);
  if (E <= 32) MOE_ROUTER_EP(32);
  if (E <= 64) MOE_ROUTER_EP(64);
  if (E <= 128) MOE_ROUTER_EP(128);
  MOE_ROUTER_EP(256);
#undef MOE_ROUTER_EP
}

// K-split when W_g (EP padded rows) fits in 64 KB of LDS and E <= 64 (and the
// MFMA path does not apply); the LDS bound also keeps the chunk count within
// the kernel's x vectors
bool router_uses_ksplit(bool xbf16, int d, int E) {
  return !router_uses_mfma(xbf16, d, E) && ks_lds_bytes(E, d, xbf16) <= 65536 && E <= 64 &&
         d <= KS_XV * ks_chunk_cols(xbf16);
}

hipError_t launch_router_counting(const void* x, bool xbf16, int64_t T, int d, const float* Wg,
                                  const float* bg, const float* bsel, int E, int k, float* logits,
                                  float* lse, int32_t* idx, float* gate, const float* noise,
                                  double sigma, double tau, int32_t* hist16, double* p16, hipStream_t st) {
#define MOE_ROUTER_KSC(EPV) \
  return launch_router_ksplit<EPV>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, noise, sigma, tau, \
                                   hist16, p16, st)
  if (E <= 8) MOE_ROUTER_KSC(8);
  if (E <= 16) MOE_ROUTER_KSC(16);
  if (E <= 32) MOE_ROUTER_KSC(32);
  MOE_ROUTER_KSC(64);
#undef MOE_ROUTER_KSC
}

hipError_t launch_router(const void* x, bool xbf16, int64_t T, int d, const float* Wg,
                         const float* bg, const float* bsel, int E, int k, float* logits,
                         float* lse, int32_t* idx, float* gate, const float* noise, double sigma, double tau,
                         void* ws, hipStream_t st) {
  if (router_uses_mfma(xbf16, d, E)) {
#define MOE_ROUTER_MFMA(EPV) \
  return launch_router_mfma<EPV>(x, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, noise, sigma, tau, ws, st)
    if (E <= 64) MOE_ROUTER_MFMA(64);
    if (E <= 128) MOE_ROUTER_MFMA(128);
    MOE_ROUTER_MFMA(256);
#undef MOE_ROUTER_MFMA
  }
  if (router_uses_ksplit(xbf16, d, E)) {
#define MOE_ROUTER_KS(EPV) \
  return launch_router_ksplit<EPV>(x, xbf16, T, d, Wg, bg, bsel, E, k, logits, lse, idx, gate, noise, sigma, tau, \
                                   nullptr, nullptr, st)
    if (E <= 8) MOE_ROUTER_KS(8);
    if (E <= 16) MOE_ROUTER_KS(16);
    if (E <= 32) MOE_ROUTER_KS(32);
    MOE_ROUTER_KS(64);
#undef MOE_ROUTER_KS
  }
  return launch_router_e_split(x, xbf16 ? XT_BF16 : XT_F32, T, d, Wg, bg, bsel, E, k, logits, lse, idx,
                               gate, noise, sigma, tau, st);
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
                             float* gate, const float* noise, double sigma, double tau, void* ws, hipStream_t st) {
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
                               sigma, tau, st);
}

}  // namespace moe
