// C ABI: argument checks, workspace sizing and kernel launches.
// Every check runs before the first launch, so a rejected call enqueues nothing.

#include "moe.h"

#include <hip/hip_runtime.h>

#include "internal.h"

using namespace moe;

namespace {

constexpr size_t kWsAlign = 256;

inline size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline bool dtype_ok(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }

inline int elem_bytes(int dt) { return dt == MOE_BF16 ? 2 : 4; }

inline bool act_ok(int a) { return a == MOE_ACT_RELU || a == MOE_ACT_GELU || a == MOE_ACT_SWISH; }

inline int check_ek(int32_t E, int32_t k) {
  if (E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// gate temperature: finite and positive
inline bool temperature_ok(float tau) { return tau > 0.f && tau <= 3.402823466e38f; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// dispatch scratch: chunk counts, group counts, scanned group counts (and
// statistics partials, last)
size_t dispatch_ws(int64_t T, int32_t E, bool with_stats = false) {
  const int64_t nchunks = (T + kDispatchChunk - 1) / kDispatchChunk;
  const int64_t ngroups = (T + kStatsTokens - 1) / kStatsTokens;
  size_t b = align_up((size_t)nchunks * (size_t)E * sizeof(int32_t)) +
             align_up((size_t)ngroups * (size_t)E * sizeof(int32_t)) +
             align_up((size_t)(ngroups + 1) * (size_t)E * sizeof(int32_t));
  if (with_stats) b += align_up((size_t)ngroups * (size_t)(E + 1) * sizeof(double));
  return b;
}

DispatchWs dispatch_ws_layout(void* ws, int64_t T, int32_t E) {
  const int64_t nchunks = (T + kDispatchChunk - 1) / kDispatchChunk;
  const int64_t ngroups = (T + kStatsTokens - 1) / kStatsTokens;
  char* p = (char*)ws;
  DispatchWs w;
  w.hist = (int32_t*)p;
  p += align_up((size_t)nchunks * (size_t)E * sizeof(int32_t));
  w.group = (int32_t*)p;
  p += align_up((size_t)ngroups * (size_t)E * sizeof(int32_t));
  w.bases = (int32_t*)p;
  p += align_up((size_t)(ngroups + 1) * (size_t)E * sizeof(int32_t));
  w.part = (double*)p;
  return w;
}

// The fused routing pass counts inside the router (no counting kernel) when
// the K-split router runs and the per-16-token counts stay few enough for
// every scatter block to sum them.
static bool route_counts_in_router(int64_t T, int32_t d, int32_t E, bool xbf16) {
  const int64_t units = (T + kStatsSub - 1) / kStatsSub;
  return router_uses_ksplit(xbf16, d, E) && units * (int64_t)E <= 8192;
}

// counting-router layout: per-16-token counts [units][E], then the statistics
// sub-partials [units][E + 1]
static DispatchWs route_units_layout(void* ws, int64_t T, int32_t E) {
  const int64_t units = (T + kStatsSub - 1) / kStatsSub;
  DispatchWs w;
  w.hist = nullptr;
  w.group = (int32_t*)ws;
  w.part = (double*)((char*)ws + align_up((size_t)units * (size_t)E * sizeof(int32_t)));
  w.units16 = true;
  return w;
}

size_t route_ws(int64_t T, int32_t d, int32_t E, bool xbf16) {
  if (route_counts_in_router(T, d, E, xbf16)) {
    // the counting router's units; sized to cover the dispatch's scratch too,
    // as the workspace query documents
    const int64_t units = (T + kStatsSub - 1) / kStatsSub;
    const size_t b = align_up((size_t)units * (size_t)E * sizeof(int32_t)) +
                     align_up((size_t)units * (size_t)(E + 1) * sizeof(double));
    const size_t dw = dispatch_ws(T, E, true);
    return b > dw ? b : dw;
  }
  const size_t r = router_uses_mfma(xbf16, d, E) ? align_up(router_mfma_ws_bytes(T, d, E)) : 0;
  return r + dispatch_ws(T, E, true);
}

size_t ffn_ws(int32_t F, int64_t max_rows) {
  // per-row, per-N-tile partial sums of squares (sized for the smaller fp32 tile)
  const int64_t tiles = (F + kGemmF32BN - 1) / kGemmF32BN;
  return align_up((size_t)max_rows * (size_t)tiles * sizeof(float));
}

// statistics scratch: block partials, then (credit only) one credit value per
// packed row
size_t stats_ws_parts(int64_t T, int32_t E) {
  const int64_t nparts = (T + kStatsTokens - 1) / kStatsTokens;
  return align_up((size_t)nparts * (size_t)(E + 1) * sizeof(double));
}

size_t stats_row_bytes(int64_t T, int32_t k) { return align_up((size_t)T * (size_t)k * sizeof(float)); }

size_t stats_ws(int64_t T, int32_t E, int32_t k, bool credit) {
  return stats_ws_parts(T, E) + (credit ? 2 * stats_row_bytes(T, k) : 0);
}

}  // namespace

namespace moe {

int route_check(const RouteCall& c, size_t* ws_need) {
  if (int rc = check_ek(c.E, c.k)) return rc;
  if (c.T < 0 || c.d < 1 || c.d % 8 != 0 || c.capacity < -1) return MOE_ERR_INVALID_ARG;
  if (!temperature_ok(c.temperature)) return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(c.x_dtype)) return MOE_ERR_UNSUPPORTED;
  if (c.T * (int64_t)c.k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (!c.expert_count || !c.expert_offset) return MOE_ERR_INVALID_ARG;
  if (c.T > 0) {
    if (!c.x || !c.W_g || !c.logits || !c.lse || !c.topk_idx || !c.topk_gate || !c.slot || !c.row ||
        !c.row_token || !c.f || !c.P || !c.losses)
      return MOE_ERR_INVALID_ARG;
    if (!aligned16(c.x) || !aligned16(c.W_g)) return MOE_ERR_INVALID_ARG;
  }
  *ws_need = route_ws(c.T, c.d, c.E, c.x_dtype == MOE_BF16);
  return MOE_OK;
}

int route_run(const RouteCall& c, void* ws, hipStream_t stream) {
  const int64_t T = c.T;
  const int32_t d = c.d, E = c.E, k = c.k;
  const bool xbf16 = c.x_dtype == MOE_BF16;
  RouteStats rs{c.logits, c.lse, c.alpha, c.beta, c.f, c.P, c.losses};
  if (T > 0 && route_counts_in_router(T, d, E, xbf16)) {
    // two kernels: the counting router, then the scatter
    const DispatchWs w = route_units_layout(ws, T, E);
    const hipError_t e = launch_router_counting(c.x, xbf16, T, d, c.W_g, c.b_g, c.b_sel, E, k, c.logits,
                                                c.lse, c.topk_idx, c.topk_gate, c.noise,
                                                (double)c.noise_std, (double)c.temperature, w.group, w.part,
                                                stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(launch_dispatch(c.topk_idx, T, k, E, c.capacity, nullptr, 2, d, c.expert_count,
                                      c.expert_offset, c.slot, c.row, c.row_token, nullptr, w, &rs, stream));
  }
  const size_t rws = router_uses_mfma(xbf16, d, E) ? align_up(router_mfma_ws_bytes(T, d, E)) : 0;
  if (T > 0) {
    const hipError_t e = launch_router(c.x, xbf16, T, d, c.W_g, c.b_g, c.b_sel, E, k, c.logits, c.lse,
                                       c.topk_idx, c.topk_gate, c.noise, (double)c.noise_std,
                                       (double)c.temperature, ws, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return hip_status(launch_dispatch(c.topk_idx, T, k, E, c.capacity, nullptr, 2, d, c.expert_count,
                                    c.expert_offset, c.slot, c.row, c.row_token, nullptr,
                                    dispatch_ws_layout((char*)ws + rws, T, E), T > 0 ? &rs : nullptr,
                                    stream));
}

}  // namespace moe

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failure";
    case MOE_ERR_SCRATCH: return "needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int moe_version(void) { return 2; }

int moe_capacity(int64_t cf_num, int64_t cf_den, int32_t k, int64_t T, int32_t E,
                 int64_t* capacity) {
  if (capacity == nullptr || cf_num < 0 || cf_den < 1 || k < 1 || T < 0 || E < 1)
    return MOE_ERR_INVALID_ARG;
  // C = ceil(cf_num * k * T / (cf_den * E)), exact in 128-bit integers
  const __int128 num = (__int128)cf_num * k * T;
  const __int128 den = (__int128)cf_den * E;
  const __int128 c = (num + den - 1) / den;
  if (c > (__int128)INT64_MAX) return MOE_ERR_INVALID_ARG;
  *capacity = (int64_t)c;
  return MOE_OK;
}

int moe_workspace_bytes(int op, int64_t T, int32_t d, int32_t E, int32_t k, int32_t F,
                        int64_t max_rows, size_t* bytes) {
  (void)d;
  (void)k;
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  switch (op) {
    case MOE_OP_ROUTER:
      if (T < 0 || E < 1 || d < 1) return MOE_ERR_INVALID_ARG;
      *bytes = router_uses_mfma(true, d, E) ? router_mfma_ws_bytes(T, d, E) : 0;
      return MOE_OK;
    case MOE_OP_COMBINE:
    case MOE_OP_SHARED_FFN:
      *bytes = 0;
      return MOE_OK;
    case MOE_OP_DISPATCH:
      if (T < 0 || E < 1) return MOE_ERR_INVALID_ARG;
      *bytes = dispatch_ws(T, E);
      return MOE_OK;
    case MOE_OP_FFN:
      if (F < 1 || max_rows < 0) return MOE_ERR_INVALID_ARG;
      *bytes = ffn_ws(F, max_rows);
      return MOE_OK;
    case MOE_OP_STATS:
      if (T < 0 || E < 1) return MOE_ERR_INVALID_ARG;
      if (k < 1) return MOE_ERR_INVALID_ARG;
      *bytes = stats_ws(T, E, k, true);
      return MOE_OK;
    case MOE_OP_MLP_ROUTER:
      if (T < 0 || F < 1) return MOE_ERR_INVALID_ARG;
      *bytes = mlp_router_ws_bytes(T, F);
      return MOE_OK;
    case MOE_OP_BALANCE:
      if (T < 0 || E < 1) return MOE_ERR_INVALID_ARG;
      *bytes = stats_ws_parts(T, E);
      return MOE_OK;
    case MOE_OP_ROUTE:
      if (T < 0 || E < 1 || d < 1) return MOE_ERR_INVALID_ARG;
      *bytes = route_ws(T, d, E, true);
      return MOE_OK;
    default:
      return MOE_ERR_INVALID_ARG;
  }
}

int moe_router_topk(const void* x, int x_dtype, int64_t T, int32_t d, const float* W_g,
                    const float* b_g, const float* b_sel, int32_t E, int32_t k, const float* noise,
                    float noise_std, float temperature, float* logits, float* lse, int32_t* topk_idx,
                    float* topk_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (int rc = check_ek(E, k)) return rc;
  if (T < 0 || d < 1 || d % 8 != 0 || !temperature_ok(temperature)) return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(x_dtype)) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !W_g || !logits || !lse || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(W_g)) return MOE_ERR_INVALID_ARG;
  if (router_uses_mfma(x_dtype == MOE_BF16, d, E)) {
    const size_t need = router_mfma_ws_bytes(T, d, E);
    if (ws == nullptr || ws_bytes < need || ((uintptr_t)ws % kWsAlign) != 0) return MOE_ERR_WORKSPACE;
  }
  return hip_status(launch_router(x, x_dtype == MOE_BF16, T, d, W_g, b_g, b_sel, E, k, logits, lse,
                                  topk_idx, topk_gate, noise, (double)noise_std, (double)temperature, ws,
                                  stream));
}

int moe_mlp_router_topk(const void* x, int x_dtype, int64_t T, int32_t d, const float* gW1,
                        const float* gb1, int32_t H, const float* gW2, const float* gb2,
                        const float* b_sel, int32_t E, int32_t k, const float* noise, float noise_std,
                        float temperature, float* logits, float* lse, int32_t* topk_idx, float* topk_gate,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  if (int rc = check_ek(E, k)) return rc;
  if (T < 0 || d < 1 || d % 8 != 0 || H < 1 || H % 8 != 0) return MOE_ERR_INVALID_ARG;
  if (!temperature_ok(temperature)) return MOE_ERR_INVALID_ARG;
  if (H > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (!dtype_ok(x_dtype)) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !gW1 || !gW2 || !logits || !lse || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(gW1) || !aligned16(gW2)) return MOE_ERR_INVALID_ARG;
  const size_t need = mlp_router_ws_bytes(T, H);
  if (ws == nullptr || ws_bytes < need || ((uintptr_t)ws % kWsAlign) != 0) return MOE_ERR_WORKSPACE;
  return hip_status(launch_mlp_router(x, x_dtype == MOE_BF16, T, d, gW1, gb1, H, gW2, gb2, b_sel, E, k,
                                      logits, lse, topk_idx, topk_gate, noise, (double)noise_std,
                                      (double)temperature, ws, stream));
}

int moe_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int64_t capacity,
                 const void* x, int x_dtype, int32_t d, int32_t* expert_count,
                 int32_t* expert_offset, int32_t* slot, int32_t* row, int32_t* row_token,
                 void* x_disp, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (int rc = check_ek(E, k)) return rc;
  if (T < 0 || capacity < -1) return MOE_ERR_INVALID_ARG;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (!expert_count || !expert_offset) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_idx || !slot || !row || !row_token)) return MOE_ERR_INVALID_ARG;
  if ((x == nullptr) != (x_disp == nullptr)) return MOE_ERR_INVALID_ARG;
  if (x_disp != nullptr) {
    if (!dtype_ok(x_dtype)) return MOE_ERR_UNSUPPORTED;
    if (d < 1 || d % 8 != 0 || !aligned16(x) || !aligned16(x_disp)) return MOE_ERR_INVALID_ARG;
  }
  const size_t need = dispatch_ws(T, E);
  if (need > 0 && (ws == nullptr || ws_bytes < need || ((uintptr_t)ws % kWsAlign) != 0))
    return MOE_ERR_WORKSPACE;
  return hip_status(launch_dispatch(topk_idx, T, k, E, capacity, x, elem_bytes(x_dtype), d,
                                    expert_count, expert_offset, slot, row, row_token, x_disp,
                                    dispatch_ws_layout(ws, T, E), nullptr, stream));
}

int moe_route(const void* x, int x_dtype, int64_t T, int32_t d, const float* W_g,
              const float* b_g, const float* b_sel, int32_t E, int32_t k, const float* noise,
              float noise_std, float temperature, int64_t capacity, float alpha, float beta,
              float* logits, float* lse, int32_t* topk_idx, float* topk_gate, int32_t* expert_count,
              int32_t* expert_offset, int32_t* slot, int32_t* row, int32_t* row_token, float* f,
              float* P, float* losses, void* ws, size_t ws_bytes, hipStream_t stream) {
  const RouteCall c{x, x_dtype, T, d, W_g, b_g, b_sel, E, k, noise, noise_std, temperature, capacity, alpha,
                    beta, logits, lse, topk_idx, topk_gate, expert_count, expert_offset, slot, row, row_token,
                    f, P, losses};
  size_t need = 0;
  if (int rc = route_check(c, &need)) return rc;
  if (need > 0 && (ws == nullptr || ws_bytes < need || ((uintptr_t)ws % kWsAlign) != 0))
    return MOE_ERR_WORKSPACE;
  return route_run(c, ws, stream);
}

static int check_ffn_common(int32_t G, int64_t max_rows, int dtype) {
  if (G < 1 || max_rows < 0) return MOE_ERR_INVALID_ARG;
  if (G > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (max_rows >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static int check_up(const void* a, const int32_t* a_rows, const int32_t* group_offset, int32_t G,
                    int64_t max_rows,
                    int32_t d, int32_t F, int dtype, int act, const void* W1, const void* b1,
                    void* hidden, float* hidden_sqnorm, void* ws, size_t ws_bytes) {
  if (int rc = check_ffn_common(G, max_rows, dtype)) return rc;
  if (d < 1 || F < 1 || d % 8 || F % 8) return MOE_ERR_INVALID_ARG;
  if (!act_ok(act)) return MOE_ERR_UNSUPPORTED;
  if (max_rows == 0) return MOE_OK;
  if (!a || !group_offset || !W1 || !b1 || !hidden) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(W1) || !aligned16(hidden)) return MOE_ERR_INVALID_ARG;
  if (hidden_sqnorm != nullptr) {
    const size_t need = ffn_ws(F, max_rows);
    if (ws == nullptr || ws_bytes < need || ((uintptr_t)ws % kWsAlign) != 0) return MOE_ERR_WORKSPACE;
  }
  return MOE_OK;
}

static int check_down(const void* hidden, const int32_t* group_offset, int32_t G, int64_t max_rows,
                      int32_t F, int32_t d_out, int dtype, const void* W2, const void* b2,
                      void* out) {
  if (int rc = check_ffn_common(G, max_rows, dtype)) return rc;
  if (F < 1 || d_out < 1 || F % 8 || d_out % 8) return MOE_ERR_INVALID_ARG;
  if (max_rows == 0) return MOE_OK;
  if (!hidden || !group_offset || !W2 || !b2 || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(hidden) || !aligned16(W2) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

static hipError_t run_up(const void* a, const int32_t* a_rows, const int32_t* group_offset, int32_t G,
                         int64_t max_rows, int32_t d, int32_t F, int dtype, int act, const void* W1,
                         const void* b1, void* hidden, float* hidden_sqnorm, void* ws,
                         hipStream_t stream) {
  const bool bf16 = dtype == MOE_BF16;
  GemmArgs g{};
  g.A = a; g.a_rows = a_rows; g.group_offset = group_offset; g.G = G; g.dense_M = 0; g.max_rows = max_rows;
  g.B = W1; g.N = F; g.K = d; g.S = 1; g.Kseg = d; g.bias = b1; g.C = hidden;
  g.act = act; g.sq_part = hidden_sqnorm ? (float*)ws : nullptr;
  hipError_t e = bf16 ? launch_gemm_bf16(g, stream) : launch_gemm_f32(g, stream);
  if (e != hipSuccess || hidden_sqnorm == nullptr) return e;
  const int tiles = bf16 ? gemm_bf16_n_tiles(g) : (F + kGemmF32BN - 1) / kGemmF32BN;
  return launch_sq_reduce((const float*)ws, tiles, group_offset, G, max_rows, hidden_sqnorm, stream);
}

static hipError_t run_down(const void* hidden, const int32_t* group_offset, int32_t G,
                           int64_t max_rows, int32_t F, int32_t d_out, int dtype, const void* W2,
                           const void* b2, void* out, hipStream_t stream) {
  GemmArgs g{};
  g.A = hidden; g.group_offset = group_offset; g.G = G; g.dense_M = 0; g.max_rows = max_rows;
  g.B = W2; g.N = d_out; g.K = F; g.S = 1; g.Kseg = F; g.bias = b2; g.C = out;
  g.act = -1; g.sq_part = nullptr;
  return dtype == MOE_BF16 ? launch_gemm_bf16(g, stream) : launch_gemm_f32(g, stream);
}

int moe_expert_up(const void* a, const int32_t* a_rows, const int32_t* group_offset, int32_t G,
                  int64_t max_rows, int32_t d, int32_t F, int dtype, int act, const void* W1,
                  const void* b1, void* hidden, float* hidden_sqnorm, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  if (int rc = check_up(a, a_rows, group_offset, G, max_rows, d, F, dtype, act, W1, b1, hidden,
                        hidden_sqnorm, ws, ws_bytes))
    return rc;
  if (max_rows == 0) return MOE_OK;
  return hip_status(run_up(a, a_rows, group_offset, G, max_rows, d, F, dtype, act, W1, b1, hidden,
                           hidden_sqnorm, ws, stream));
}

int moe_expert_down(const void* hidden, const int32_t* group_offset, int32_t G, int64_t max_rows,
                    int32_t F, int32_t d_out, int dtype, const void* W2, const void* b2, void* out,
                    hipStream_t stream) {
  if (int rc = check_down(hidden, group_offset, G, max_rows, F, d_out, dtype, W2, b2, out)) return rc;
  if (max_rows == 0) return MOE_OK;
  return hip_status(run_down(hidden, group_offset, G, max_rows, F, d_out, dtype, W2, b2, out, stream));
}

int moe_grouped_ffn(const void* a, const int32_t* a_rows, const int32_t* group_offset, int32_t G,
                    int64_t max_rows, int32_t d, int32_t F, int32_t d_out, int dtype, int act,
                    const void* W1, const void* b1, const void* W2, const void* b2, void* hidden,
                    void* out, float* hidden_sqnorm, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  if (int rc = check_up(a, a_rows, group_offset, G, max_rows, d, F, dtype, act, W1, b1, hidden,
                        hidden_sqnorm, ws, ws_bytes))
    return rc;
  if (int rc = check_down(hidden, group_offset, G, max_rows, F, d_out, dtype, W2, b2, out)) return rc;
  if (max_rows == 0) return MOE_OK;
  hipError_t e = run_up(a, a_rows, group_offset, G, max_rows, d, F, dtype, act, W1, b1, hidden,
                        hidden_sqnorm, ws, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(run_down(hidden, group_offset, G, max_rows, F, d_out, dtype, W2, b2, out, stream));
}

int moe_shared_ffn(const void* x, int64_t T, int32_t d, int32_t F, int32_t S, int32_t d_out,
                   int dtype, int act, const void* W1, const void* b1, const void* W2,
                   const void* b2, void* hidden, void* out, hipStream_t stream) {
  if (T < 0 || S < 1 || d < 1 || F < 1 || d_out < 1 || d % 8 || F % 8 || d_out % 8)
    return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || !act_ok(act)) return MOE_ERR_UNSUPPORTED;
  if (T >= ((int64_t)1 << 31) || (int64_t)S * F >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !W1 || !b1 || !W2 || !b2 || !hidden || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W2) || !aligned16(hidden) || !aligned16(out))
    return MOE_ERR_INVALID_ARG;
  const bool bf16 = dtype == MOE_BF16;
  GemmArgs g1{};
  g1.A = x; g1.group_offset = nullptr; g1.G = 1; g1.dense_M = T; g1.max_rows = T;
  g1.B = W1; g1.N = S * F; g1.K = d; g1.S = 1; g1.Kseg = d; g1.bias = b1; g1.C = hidden;
  g1.act = act; g1.sq_part = nullptr;
  GemmArgs g2 = g1;
  g2.A = hidden; g2.B = W2; g2.N = d_out; g2.K = S * F; g2.S = S; g2.Kseg = F; g2.bias = b2;
  g2.C = out; g2.act = -1;
  hipError_t e = bf16 ? launch_gemm_bf16(g1, stream) : launch_gemm_f32(g1, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = bf16 ? launch_gemm_bf16(g2, stream) : launch_gemm_f32(g2, stream);
  return hip_status(e);
}

int moe_combine(const void* expert_out, const int32_t* row, const float* topk_gate,
                const void* shared_out, int64_t T, int32_t k, int32_t d_out, int dtype, void* y,
                hipStream_t stream) {
  if (T < 0 || k < 1 || d_out < 1 || d_out % 8) return MOE_ERR_INVALID_ARG;
  if (k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!expert_out || !row || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(expert_out) || !aligned16(y) || (shared_out && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(expert_out, row, topk_gate, shared_out, T, k, d_out,
                                   dtype == MOE_BF16, y, stream));
}

int moe_route_stats(const float* logits, const float* lse, const int32_t* topk_idx,
                    const float* topk_gate, const int32_t* expert_count, int64_t T, int32_t E,
                    int32_t k, float alpha, float beta, float* f, float* P, float* losses,
                    const float* hidden_sqnorm, const int32_t* row, const int32_t* expert_offset,
                    const int32_t* row_token, float* credit, float* mean_credit,
                    const float* token_loss, float* expert_loss, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  if (int rc = check_ek(E, k)) return rc;
  if (T < 1) return MOE_ERR_INVALID_ARG;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (!logits || !lse || !topk_idx || !topk_gate || !expert_count) return MOE_ERR_INVALID_ARG;
  // f, P and losses go together; all NULL asks for the credit alone
  if ((f == nullptr) != (P == nullptr) || (f == nullptr) != (losses == nullptr)) return MOE_ERR_INVALID_ARG;
  if ((credit == nullptr) != (mean_credit == nullptr)) return MOE_ERR_INVALID_ARG;
  if (f == nullptr && credit == nullptr) return MOE_ERR_INVALID_ARG;  // nothing to compute
  if (credit && (!hidden_sqnorm || !row || !expert_offset || !row_token)) return MOE_ERR_INVALID_ARG;
  if ((token_loss == nullptr) != (expert_loss == nullptr)) return MOE_ERR_INVALID_ARG;
  if (token_loss && !credit) return MOE_ERR_INVALID_ARG;   // the loss is weighted by the credit
  const size_t need = stats_ws(T, E, k, credit != nullptr);
  if (ws == nullptr || ws_bytes < need || ((uintptr_t)ws % kWsAlign) != 0) return MOE_ERR_WORKSPACE;
  char* rows = (char*)ws + stats_ws_parts(T, E);
  float* credit_row = credit ? (float*)rows : nullptr;
  float* loss_row = token_loss ? (float*)(rows + stats_row_bytes(T, k)) : nullptr;
  return hip_status(launch_stats(logits, lse, topk_idx, topk_gate, expert_count, T, E, k, alpha,
                                 beta, f, P, losses, hidden_sqnorm, row, expert_offset, row_token,
                                 credit, mean_credit, (double*)ws, credit_row, token_loss, loss_row,
                                 expert_loss, stream));
}

int moe_balance_losses(const float* topk_gate, const int32_t* topk_idx, const int32_t* expert_count,
                       const float* lse, int64_t T, int32_t E, int32_t k, float load_balance_coef,
                       float z_loss_coef, float* importance, float* out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  if (int rc = check_ek(E, k)) return rc;
  if (T < 1) return MOE_ERR_INVALID_ARG;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (!topk_gate || !topk_idx || !expert_count || !lse || !importance || !out) return MOE_ERR_INVALID_ARG;
  const size_t need = stats_ws_parts(T, E);
  if (ws == nullptr || ws_bytes < need || ((uintptr_t)ws % kWsAlign) != 0) return MOE_ERR_WORKSPACE;
  return hip_status(launch_balance(topk_gate, topk_idx, expert_count, lse, T, E, k, load_balance_coef,
                                   z_loss_coef, importance, out, (double*)ws, stream));
}

int moe_selection_bias_update(const int32_t* expert_count, int32_t E, int32_t k, int64_t T, float gamma,
                              float* b_sel, hipStream_t stream) {
  if (int rc = check_ek(E, k)) return rc;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (!expert_count || !b_sel) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_bias_update(expert_count, E, k, T, gamma, b_sel, stream));
}

int moe_dro_update(const float* expert_loss, int32_t E, float ema_decay, float eta, float* ema,
                   float* mu, float* dro_loss, hipStream_t stream) {
  if (E < 1) return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (!expert_loss || !ema || !mu || !dro_loss) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_dro_update(expert_loss, E, ema_decay, eta, ema, mu, dro_loss, stream));
}

}  // extern "C"
