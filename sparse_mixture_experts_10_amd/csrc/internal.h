// Host-side launchers shared between the kernel files and the C ABI layer.
// All of them enqueue on `st` and return the launch status; none blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gemm_args.h"

namespace moe {

constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 32;
constexpr int kDispatchChunk = 64;    // tokens per dispatch chunk (one wavefront)
constexpr int kStatsTokens = 256;     // tokens per statistics partial block
constexpr int kStatsSub = 16;         // tokens per statistics sub-partial (and router block)
constexpr int kGemmBN = 128;          // N tile of the bf16 grouped GEMM
constexpr int kGemmBM = 128;          // M tile of the bf16 grouped GEMM
constexpr int kGemmF32BN = 64;        // N tile of the fp32 grouped GEMM
constexpr int kGemmF32BM = 64;        // M tile of the fp32 grouped GEMM

// ws: MFMA-path scratch (router_mfma_ws_bytes) when router_uses_mfma(), else unused.
// noise: [T, E] standard-normal draws added as sigma * noise (or nullptr);
// tau: gate temperature dividing the (noisy) logits, 1 = none.
hipError_t launch_router(const void* x, bool xbf16, int64_t T, int d, const float* Wg,
                         const float* bg, const float* bsel, int E, int k, float* logits,
                         float* lse, int32_t* idx, float* gate, const float* noise, double sigma, double tau,
                         void* ws, hipStream_t st);
// MLP gate: hidden [T, H] fp64 in ws (mlp_router_ws_bytes), then the E-split router on it.
hipError_t launch_mlp_router(const void* x, bool xbf16, int64_t T, int d, const float* gW1,
                             const float* gb1, int H, const float* gW2, const float* gb2,
                             const float* bsel, int E, int k, float* logits, float* lse, int32_t* idx,
                             float* gate, const float* noise, double sigma, double tau, void* ws, hipStream_t st);
size_t mlp_router_ws_bytes(int64_t T, int H);
bool router_uses_mfma(bool xbf16, int d, int E);
size_t router_mfma_ws_bytes(int64_t T, int d, int E);
bool router_uses_ksplit(bool xbf16, int d, int E);
// The K-split router that also counts: per block of 16 tokens it writes the
// choices per expert, hist16 [ceil(T / 16)][E], and the statistics
// sub-partials, p16 [ceil(T / 16)][E + 1] (only when router_uses_ksplit()).
hipError_t launch_router_counting(const void* x, bool xbf16, int64_t T, int d, const float* Wg,
                                  const float* bg, const float* bsel, int E, int k, float* logits,
                                  float* lse, int32_t* idx, float* gate, const float* noise,
                                  double sigma, double tau, int32_t* hist16, double* p16, hipStream_t st);

// Dispatch scratch: per-chunk counts [nchunks][E], per-group counts
// [ngroups][E] (a group is kStatsTokens tokens), and, for the fused routing
// pass, statistics partials [ngroups][E + 1].  With units16 the counting
// router has already written per-16-token counts into group ([ceil(T/16)][E])
// and the statistics sub-partials into part ([ceil(T/16)][E + 1]); hist is
// unused and no counting kernel runs.
// bases ([ngroups + 1][E], or nullptr): the scanned group counts, used when
// there are more than kScanMinCounts of them.
constexpr int64_t kScanMinCounts = 4096;
struct DispatchWs {
  int32_t* hist;
  int32_t* group;
  double* part;
  bool units16 = false;
  int32_t* bases = nullptr;
};
// Routing statistics taken in the same pass as the dispatch (nullptr: none).
struct RouteStats {
  const float* logits;
  const float* lse;
  float alpha, beta;
  float* f;
  float* P;
  float* losses;
};
hipError_t launch_dispatch(const int32_t* idx, int64_t T, int k, int E, int64_t capacity,
                           const void* x, int elem_bytes, int d, int32_t* count,
                           int32_t* offset, int32_t* slot, int32_t* row, int32_t* row_token,
                           void* x_disp, const DispatchWs& ws, const RouteStats* stats,
                           hipStream_t st);

// The fused routing pass behind moe_route, split so that a caller can check
// the arguments and size the scratch before it picks where the scratch comes
// from.  Arguments as moe_route's (include/moe.h).
struct RouteCall {
  const void* x;
  int x_dtype;
  int64_t T;
  int32_t d;
  const float *W_g, *b_g, *b_sel;
  int32_t E, k;
  const float* noise;
  float noise_std, temperature;
  int64_t capacity;
  float alpha, beta;
  float *logits, *lse;
  int32_t* topk_idx;
  float* topk_gate;
  int32_t *expert_count, *expert_offset, *slot, *row, *row_token;
  float *f, *P, *losses;
};
// Checks every argument (nothing is enqueued); *ws_need receives the scratch
// bytes the call needs.  Returns a MOE_* status.
int route_check(const RouteCall& c, size_t* ws_need);
// Enqueues the pass; c passed route_check and ws holds ws_need bytes, 256-byte aligned.
int route_run(const RouteCall& c, void* ws, hipStream_t st);

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t st);     // picks the path below
int gemm_bf16_n_tiles(const GemmArgs& a);                           // N tiles of that choice
hipError_t launch_gemm_bf16_v1(const GemmArgs& a, hipStream_t st);  // any K % 8 == 0
bool gemm_v2_supported(const GemmArgs& a);                         // K % 32 == 0
bool gemm_v2_wide_k(const GemmArgs& a);                            // K % 64 == 0
hipError_t launch_gemm_bf16_v2(const GemmArgs& a, int tile, hipStream_t st);  // tile 64, 128, 144, 145, 257, 259, 256, 513
bool gemm_persist_supported(const GemmArgs& a);                     // one K segment, bf16 out, G <= 256
hipError_t launch_gemm_bf16_persist(const GemmArgs& a, hipStream_t st);  // persistent 256 x 256 tiles
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t st);
hipError_t launch_sq_reduce(const float* sq_part, int n_tiles, const int32_t* group_offset, int G,
                            int64_t max_rows, float* sq, hipStream_t st);

hipError_t launch_combine(const void* expert_out, const int32_t* row, const float* gate,
                          const void* shared_out, int64_t T, int k, int d_out, bool bf16,
                          void* y, hipStream_t st);

// workspace: partial [nblocks][E+1] double; credit_row [rows] and loss_row [rows] float
// (credit only; loss_row only with per-token losses)
hipError_t launch_stats(const float* logits, const float* lse, const int32_t* idx,
                        const float* gate, const int32_t* count, int64_t T, int E, int k,
                        float alpha, float beta, float* f, float* Pm, float* losses,
                        const float* sq, const int32_t* row, const int32_t* offset,
                        const int32_t* row_token, float* credit, float* mean_credit,
                        double* ws_partial, float* credit_row, const float* token_loss,
                        float* loss_row, float* expert_loss, hipStream_t st);

// workspace: partial [nblocks][E+1] double
hipError_t launch_balance(const float* gate, const int32_t* idx, const int32_t* count,
                          const float* lse, int64_t T, int E, int k, float lb_coef, float z_coef,
                          float* importance, float* out, double* ws_partial, hipStream_t st);
hipError_t launch_bias_update(const int32_t* count, int E, int k, int64_t T, float gamma,
                              float* b_sel, hipStream_t st);
hipError_t launch_dro_update(const float* loss, int E, float decay, float eta, float* ema, float* mu,
                             float* dro_loss, hipStream_t st);

}  // namespace moe
