// Batch routing statistics and activation-weighted expert credit.
//
// Page "Appendix C -- Acronyms & Symbols", Balancing:
//   f_e    = count_e / (k T)           (fraction of the batch's choices sent to e,
//                                       counted before the capacity cap)
//   P_e    = (1/T) sum_t softmax(h_t)_e  (average router mass)
//   L_aux  = alpha E sum_e f_e P_e       (Switch auxiliary loss)
//   L_z    = beta (1/T) sum_t lse_t^2    (router z-loss)
// Page "Sparse MoE Expert-Credit Loss Reweighting Diagram", panel (b):
//   credit[t,j]    = g[t,j] * ||a_{t,j}||_2   (a = the expert's hidden activation;
//                                             0 for a dropped choice)
//   mean_credit_e  = (1/T) sum of credit over the kept choices of expert e
//   expert_loss_e  = (1/T) sum of credit * token_loss[t] over the same choices
//                    (the expert-attributed loss, when per-token losses are given)
//
// Deterministic: no floating-point atomics.  Kernel 1 gives every block of 256
// tokens fixed-order partial sums (fp64) of softmax mass per expert and of
// lse^2, and writes the per-choice credit (also stored per packed row).  Kernel 2 sums the partials in
// block order (block 0) and, in blocks 1..E, each expert's credit over its
// packed rows in row order.  With f, P and losses NULL (the routing pass
// computed them) only the credit is formed: kernel 1 skips the partial sums
// and block 0 of kernel 2 has nothing to do.

#include "common.h"
#include "internal.h"
#include "stats_common.h"

namespace moe {

__global__ __launch_bounds__(256) void stats_partial_kernel(
    const float* __restrict__ logits, const float* __restrict__ lse, int64_t T, int E, int k,
    const float* __restrict__ gate, const float* __restrict__ sq, const int32_t* __restrict__ row,
    float* __restrict__ credit, double* __restrict__ part, float* __restrict__ credit_row,
    const float* __restrict__ token_loss, float* __restrict__ loss_row) {
  __shared__ double s_red[256];
  __shared__ double s_grp[4 * 256];
  const int64_t t0 = (int64_t)blockIdx.x * kStatsTokens;
  const int64_t t1 = (t0 + kStatsTokens < T) ? t0 + kStatsTokens : T;
  if (part != nullptr)  // uniform; nullptr: the credit alone
    stats_block_partials(logits, lse, t0, t1, E, s_red, part + (int64_t)blockIdx.x * (E + 1), s_grp);
  const int64_t t = t0 + threadIdx.x;
  if (credit != nullptr && t < t1) {
    for (int j = 0; j < k; ++j) {
      const int r = row[t * k + j];
      const float c = r >= 0 ? gate[t * k + j] * sqrtf(sq[r]) : 0.f;
      credit[t * k + j] = c;
      if (r >= 0) {
        credit_row[r] = c;
        if (token_loss != nullptr) loss_row[r] = c * token_loss[t];
      }
    }
  }
}

// block 0: f, P, losses.  block 1 + e: mean credit of expert e.
__global__ __launch_bounds__(256) void stats_final_kernel(
    const double* __restrict__ part, int nparts, const int32_t* __restrict__ count, int64_t T,
    int E, int k, float alpha, float beta, float* __restrict__ f, float* __restrict__ Pm,
    float* __restrict__ losses, const int32_t* __restrict__ offset,
    const float* __restrict__ credit_row, float* __restrict__ mean_credit,
    const float* __restrict__ loss_row, float* __restrict__ expert_loss) {
  __shared__ double s_red[256];
  __shared__ double s_z[256];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    if (f != nullptr) stats_finish(part, nparts, count, T, E, k, alpha, beta, f, Pm, losses, s_red, s_z);
    return;
  }
  const int e = blockIdx.x - 1;
  const int64_t r0 = offset[e], r1 = offset[e + 1];
  // rows of expert e in row order per thread; the credit of each kept row was
  // stored by the partial kernel
  double s = 0.0;
  int64_t r = r0 + tid;
  for (; r + 3 * 256 < r1; r += 4 * 256) {
    const float c0 = credit_row[r], c1 = credit_row[r + 256], c2 = credit_row[r + 512],
                c3 = credit_row[r + 768];
    s += (double)c0;
    s += (double)c1;
    s += (double)c2;
    s += (double)c3;
  }
  for (; r < r1; r += 256) s += (double)credit_row[r];
  s_red[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] += s_red[tid + w];
    __syncthreads();
  }
  if (tid == 0) mean_credit[e] = (float)(s_red[0] / (double)T);
  if (expert_loss == nullptr) return;  // uniform
  // expert-attributed loss: the same order over credit * token loss
  __syncthreads();
  double q = 0.0;
  for (int64_t rr = r0 + tid; rr < r1; rr += 256) q += (double)loss_row[rr];
  s_red[tid] = q;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] += s_red[tid + w];
    __syncthreads();
  }
  if (tid == 0) expert_loss[e] = (float)(s_red[0] / (double)T);
}

hipError_t launch_stats(const float* logits, const float* lse, const int32_t* idx,
                        const float* gate, const int32_t* count, int64_t T, int E, int k,
                        float alpha, float beta, float* f, float* Pm, float* losses,
                        const float* sq, const int32_t* row, const int32_t* offset,
                        const int32_t* row_token, float* credit, float* mean_credit,
                        double* ws_partial, float* credit_row, const float* token_loss,
                        float* loss_row, float* expert_loss, hipStream_t st) {
  (void)idx;
  (void)row_token;
  const int64_t nparts = (T + kStatsTokens - 1) / kStatsTokens;
  // f == nullptr: the credit alone (the statistics' partial sums are skipped)
  hipLaunchKernelGGL(stats_partial_kernel, dim3((unsigned)nparts), dim3(256), 0, st, logits, lse, T,
                     E, k, gate, sq, row, credit, f != nullptr ? ws_partial : nullptr, credit_row,
                     token_loss, loss_row);
  const unsigned nblk = mean_credit != nullptr ? (unsigned)(E + 1) : 1u;
  hipLaunchKernelGGL(stats_final_kernel, dim3(nblk), dim3(256), 0, st, ws_partial, (int)nparts, count,
                     T, E, k, alpha, beta, f, Pm, losses, offset, credit_row, mean_credit, loss_row,
                     expert_loss);
  return hipGetLastError();
}

}  // namespace moe
