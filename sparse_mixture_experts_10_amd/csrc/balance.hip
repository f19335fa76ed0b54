// Balancing and reweighting statistics around the layer.
//
//  * coefficient-of-variation load and importance losses and their weighted
//    combination with the z-loss (page "Code Walkthrough -- SER", Load
//    balancing: balance across experts, total importance per expert, and
//    aux_loss = load_balance_coef * load_balance + z_loss_coef * z_loss):
//      load_i       = pre-capacity count_i
//      importance_i = sum over the batch of the gates routed to expert i
//      CV(v)^2      = population variance / mean^2   (0 when the mean is 0)
//      out = { CV(load)^2, CV(importance)^2, mean_t lse_t^2,
//              load_balance_coef CV(load)^2 + z_loss_coef mean_t lse_t^2 }
//  * aux-loss-free selection-bias update (page "Appendix C -- Acronyms &
//    Symbols", Balancing: per-expert selection bias b_i, update rate gamma):
//      b_i <- b_i + gamma sign(k T / E - count_i), the sign decided exactly
//      in integers
//  * EMA tracker and layer-wise DRO weights (page "Sparse MoE Expert-Credit
//    Loss Reweighting Diagram", panel (c)):
//      lhat <- decay lhat + (1 - decay) l ;  mu <- softmax(mu + eta lhat) ;
//      L_DRO = sum_i mu_i l_i
//
// Deterministic: fp64 sums in a fixed order, no floating-point atomics.

#include "common.h"
#include "internal.h"

namespace moe {

// One block of 256 threads per kStatsTokens tokens: importance partials per
// expert (thread e scans the block's choices in token order) and the lse^2
// partial.  part[b][E + 1].
__global__ __launch_bounds__(256) void balance_partial_kernel(const float* __restrict__ gate,
                                                              const int32_t* __restrict__ idx,
                                                              const float* __restrict__ lse,
                                                              int64_t T, int E, int k,
                                                              double* __restrict__ part) {
  __shared__ int s_idx[kStatsTokens * kMaxTopK];
  __shared__ float s_g[kStatsTokens * kMaxTopK];
  __shared__ double s_red[256];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kStatsTokens;
  const int64_t t1 = (t0 + kStatsTokens < T) ? t0 + kStatsTokens : T;
  const int n = (int)(t1 - t0) * k;
  for (int i = tid; i < n; i += 256) {
    s_idx[i] = idx[t0 * k + i];
    s_g[i] = gate[t0 * k + i];
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    double s = 0.0;
    for (int i = 0; i < n; ++i)
      if (s_idx[i] == e) s += (double)s_g[i];
    part[(int64_t)blockIdx.x * (E + 1) + e] = s;
  }
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
  if (tid == 0) part[(int64_t)blockIdx.x * (E + 1) + E] = s_red[0];
}

__global__ __launch_bounds__(256) void balance_final_kernel(const double* __restrict__ part,
                                                            int nparts,
                                                            const int32_t* __restrict__ count,
                                                            int64_t T, int E, float lb_coef,
                                                            float z_coef,
                                                            float* __restrict__ importance,
                                                            float* __restrict__ out) {
  __shared__ double s_imp[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) {
    double s = 0.0;
    for (int b = 0; b < nparts; ++b) s += part[(int64_t)b * (E + 1) + e];
    s_imp[e] = s;
    importance[e] = (float)s;
  }
  __syncthreads();
  if (tid == 0) {
    // CV^2 with the population variance, both vectors in fp64 in expert order
    double mc = 0.0, mi = 0.0;
    for (int e = 0; e < E; ++e) {
      mc += (double)count[e];
      mi += s_imp[e];
    }
    mc /= E;
    mi /= E;
    double vc = 0.0, vi = 0.0;
    for (int e = 0; e < E; ++e) {
      const double dc = (double)count[e] - mc, di = s_imp[e] - mi;
      vc += dc * dc;
      vi += di * di;
    }
    vc /= E;
    vi /= E;
    const double cv_load = mc != 0.0 ? vc / (mc * mc) : 0.0;
    const double cv_imp = mi != 0.0 ? vi / (mi * mi) : 0.0;
    double z = 0.0;
    for (int b = 0; b < nparts; ++b) z += part[(int64_t)b * (E + 1) + E];
    z /= (double)T;
    out[0] = (float)cv_load;
    out[1] = (float)cv_imp;
    out[2] = (float)z;
    out[3] = (float)((double)lb_coef * cv_load + (double)z_coef * z);
  }
}

hipError_t launch_balance(const float* gate, const int32_t* idx, const int32_t* count,
                          const float* lse, int64_t T, int E, int k, float lb_coef, float z_coef,
                          float* importance, float* out, double* ws_partial, hipStream_t st) {
  const int64_t nparts = (T + kStatsTokens - 1) / kStatsTokens;
  hipLaunchKernelGGL(balance_partial_kernel, dim3((unsigned)nparts), dim3(256), 0, st, gate, idx, lse,
                     T, E, k, ws_partial);
  hipLaunchKernelGGL(balance_final_kernel, dim3(1), dim3(256), 0, st, ws_partial, (int)nparts, count, T,
                     E, lb_coef, z_coef, importance, out);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ count, int E,
                                                          int k, int64_t T, float gamma,
                                                          float* __restrict__ b_sel) {
  for (int e = threadIdx.x; e < E; e += 256) {
    // sign(k T / E - count_e) = sign(k T - E count_e), exact in 64-bit integers
    const int64_t diff = (int64_t)k * T - (int64_t)E * count[e];
    const float s = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
    b_sel[e] = b_sel[e] + gamma * s;
  }
}

hipError_t launch_bias_update(const int32_t* count, int E, int k, int64_t T, float gamma,
                              float* b_sel, hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(256), 0, st, count, E, k, T, gamma, b_sel);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void dro_update_kernel(const float* __restrict__ loss, int E,
                                                         float decay, float eta,
                                                         float* __restrict__ ema,
                                                         float* __restrict__ mu,
                                                         float* __restrict__ dro_loss) {
  __shared__ double s_z[kMaxExperts];
  __shared__ double s_w[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) {
    const double l = (double)loss[e];
    const double eh = (double)decay * (double)ema[e] + (1.0 - (double)decay) * l;
    ema[e] = (float)eh;
    s_z[e] = (double)mu[e] + (double)eta * eh;
  }
  __syncthreads();
  if (tid == 0) {
    double m = s_z[0];
    for (int e = 1; e < E; ++e) m = fmax(m, s_z[e]);
    double sum = 0.0;
    for (int e = 0; e < E; ++e) {
      s_w[e] = exp(s_z[e] - m);
      sum += s_w[e];
    }
    double L = 0.0;
    for (int e = 0; e < E; ++e) {
      const double w = s_w[e] / sum;
      s_w[e] = w;
      L += w * (double)loss[e];
    }
    dro_loss[0] = (float)L;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) mu[e] = (float)s_w[e];
}

hipError_t launch_dro_update(const float* loss, int E, float decay, float eta, float* ema, float* mu,
                             float* dro_loss, hipStream_t st) {
  hipLaunchKernelGGL(dro_update_kernel, dim3(1), dim3(256), 0, st, loss, E, decay, eta, ema, mu,
                     dro_loss);
  return hipGetLastError();
}

}  // namespace moe
