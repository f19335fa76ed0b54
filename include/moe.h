/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts forward layer.
 *
 * One MoE sub-layer forward pass, as the pages define it:
 *   router logits h = W_g x (+ router bias), softmax, greedy top-k with
 *   renormalised gate weights                         -> moe_router_topk
 *   capacity C = ceil(C_f k T / E), token-order dispatch, overflow dropped
 *                                                      -> moe_capacity, moe_dispatch
 *   per-expert two-layer FFN w1/b1 -> act -> w2/b2     -> moe_grouped_ffn
 *   always-on shared experts                           -> moe_shared_ffn
 *   gate-weighted combine                              -> moe_combine
 *   f_i, P_i, Switch aux loss, z-loss, expert credit   -> moe_route_stats
 * Sources: "Appendix C -- Acronyms & Symbols" (MoE lessons), sections Core MoE
 * symbols, Parameter accounting, Balancing, Capacity & communication;
 * "Code Walkthrough -- SER (Sparse Expert Routing)", sections The gating /
 * routing path and Load balancing; "Sparse MoE Expert-Credit Loss Reweighting
 * Diagram", panel (b).
 *
 * Conventions for every call:
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device; the caller owns all memory.  The library never
 *     allocates, frees or keeps a pointer after the call returns.
 *   - Tensors are dense row-major.  bf16 tensors hold raw bf16 bit patterns
 *     (round-to-nearest-even is used wherever the library rounds to bf16).
 *   - Rows of x, x_disp, expert weights, hidden and outputs must start on
 *     16-byte boundaries: base pointers 16-byte aligned, and d, F, d_out
 *     multiples of 8.
 *   - Arguments are checked before anything is enqueued; a failed check
 *     returns a negative status and enqueues nothing.  A launch failure returns
 *     MOE_ERR_HIP.  Faults inside kernels surface at the caller's next sync.
 *   - Work is enqueued on `stream` (0 = default stream); no call blocks the
 *     host, none calls hipMalloc or hipMemset, so calls can be captured in a
 *     HIP graph.  Results are bitwise deterministic run to run.
 *   - Limits: 1 <= E <= 256, 1 <= k <= min(E, 32), T * k < 2^31.
 *   - Workspaces (`ws`) are caller-allocated device scratch of at least
 *     moe_workspace_bytes() bytes, 256-byte aligned; they need no clearing.
 *   - Calls sharing a workspace or outputs must be ordered on one stream.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)  /* null pointer, bad size, misalignment, out-of-range value */
#define MOE_ERR_UNSUPPORTED (-2)  /* valid but outside this library's limits (dtype, E, k) */
#define MOE_ERR_WORKSPACE (-3)    /* workspace missing or smaller than moe_workspace_bytes() */
#define MOE_ERR_HIP (-4)          /* a HIP launch failed */
#define MOE_ERR_SCRATCH (-5)      /* needs more scratch than the static buffer of moe_route_noalloc holds */

/* Element types. */
#define MOE_F32 0
#define MOE_BF16 1

/* Expert activations ("Code Walkthrough -- SER": ReLU, GELU, Swish are named;
 * the library uses ReLU max(0,z), exact GELU 0.5 z (1 + erf(z / sqrt 2)),
 * Swish z * sigmoid(z)). */
#define MOE_ACT_RELU 0
#define MOE_ACT_GELU 1
#define MOE_ACT_SWISH 2

/* Operations, for moe_workspace_bytes(). */
#define MOE_OP_ROUTER 0
#define MOE_OP_DISPATCH 1
#define MOE_OP_FFN 2
#define MOE_OP_COMBINE 3
#define MOE_OP_STATS 4
#define MOE_OP_SHARED_FFN 5
#define MOE_OP_ROUTE 6
#define MOE_OP_BALANCE 7
#define MOE_OP_MLP_ROUTER 8

/* Static description of a status code (never NULL). */
const char* moe_status_string(int status);

/* ABI version, currently 2 (2 added the gate temperature to the router calls). */
int moe_version(void);

/*
 * Expert capacity C = ceil(C_f * k * T / E) with C_f = cf_num / cf_den, in exact
 * integer arithmetic ("Appendix C -- Acronyms & Symbols", Capacity &
 * communication).  Host-only; touches no device.
 *   cf_num >= 0, cf_den >= 1, k >= 1, T >= 0, E >= 1; *capacity receives C.
 * Returns MOE_ERR_INVALID_ARG on a bad argument or if C would overflow int64.
 */
int moe_capacity(int64_t cf_num, int64_t cf_den, int32_t k, int64_t T, int32_t E,
                 int64_t* capacity);

/*
 * Device workspace size in bytes needed by operation `op` for these sizes
 * (0 when the operation needs none).  Host-only.  Arguments that an operation
 * does not use are ignored: ROUTER uses T, d, E (the size assumes bf16 x;
 * fp32 x needs none); DISPATCH uses T, E; FFN uses F, max_rows; STATS uses T, E,
 * k (the size covers credit and the expert-attributed loss); ROUTE uses T, d,
 * E (as ROUTER plus DISPATCH plus the statistics partials); BALANCE uses T, E;
 * MLP_ROUTER uses T and F = the gate's hidden width H.
 */
int moe_workspace_bytes(int op, int64_t T, int32_t d, int32_t E, int32_t k, int32_t F,
                        int64_t max_rows, size_t* bytes);

/*
 * Router: logits, log-sum-exp, top-k and gates for T tokens.
 * ("Appendix C -- Acronyms & Symbols", Core MoE symbols: h = W_g x, P =
 * softmax(h), T_k(x), g_i = P_i renormalised over T_k; Balancing: per-expert
 * selection bias b_i; "Code Walkthrough -- SER", The gating / routing path:
 * linear router with bias, greedy top-k picks the highest logits.)
 *   x        [T, d] device, x_dtype MOE_F32 or MOE_BF16
 *   W_g      [E, d] fp32 device;  b_g [E] fp32 device or NULL (router bias, part of h)
 *   b_sel    [E] fp32 device or NULL: added to h for the selection only
 *   noise    [T, E] fp32 device or NULL: noisy top-k ("Code Walkthrough -- SER",
 *            The gating / routing path: training noise is added to the logits
 *            before selection).  The logits become h + noise_std * noise and
 *            everything below uses them.  noise holds standard-normal draws
 *            supplied by the caller; NULL = greedy.
 *   temperature  gate temperature tau, finite and > 0 (1 = none; "Code
 *            Walkthrough -- SER", The gating / routing path: the gate-forward
 *            call takes a temperature).  The logits are divided by it after
 *            the noise, z = (h + noise_std * noise) / tau, in fp64, and z
 *            replaces h everywhere below: the stored logits, lse, the
 *            selection on z + b_sel, the gates.  Otherwise MOE_ERR_INVALID_ARG.
 *   logits   [T, E] fp32 out: the (noisy, tempered) h, without b_sel
 *   lse      [T] fp32 out: log sum_e exp(h_e)
 *   topk_idx [T, k] int32 out: selected experts ordered by (h + b_sel desc,
 *            index asc); equal scores go to the lower index
 *   topk_gate[T, k] fp32 out: exp(h_e) / sum over the selected of exp(h_e')
 *   ws       MOE_OP_ROUTER workspace (needed only for bf16 x with E * d too
 *            large for the on-chip path; moe_workspace_bytes says how much).
 * Selection precision: small E * d, or fp32 x: products and sums in fp64
 * (exact products).  Otherwise W_g is split exactly into three bf16 parts and
 * the logits are a bf16 MFMA GEMM with fp32 accumulation; every token whose
 * k-th / (k+1)-th score gap is within 5e-5 (relative) is then recomputed in
 * fp64, so selections agree with a float64 evaluation except on gaps near
 * float64 rounding.  Logits are rounded to fp32 once.  T = 0 is a no-op.
 */
int moe_router_topk(const void* x, int x_dtype, int64_t T, int32_t d, const float* W_g,
                    const float* b_g, const float* b_sel, int32_t E, int32_t k, const float* noise,
                    float noise_std, float temperature, float* logits, float* lse, int32_t* topk_idx,
                    float* topk_gate, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Dispatch in token order under capacity `capacity` (>= 0, or -1 = no cap).
 * ("Appendix C -- Acronyms & Symbols", Capacity & communication: dispatch
 * tensor D scatters tokens into fixed-size expert buffers; "Code Walkthrough --
 * SER", Load balancing: a hard per-expert cap drops overflow tokens.)
 *   topk_idx      [T, k] int32 device, entries in [0, E), distinct per token
 *   x             [T, d] device (x_dtype) or NULL together with x_disp = NULL
 *   expert_count  [E] int32 out: choices per expert before the cap
 *   expert_offset [E+1] int32 out: exclusive prefix of min(count, C); the kept
 *                 rows of expert e are expert_offset[e] .. expert_offset[e+1]-1
 *   slot          [T, k] int32 out: arrival rank of choice (t, j) at its expert
 *                 (number of earlier tokens that chose it)
 *   row           [T, k] int32 out: expert_offset[e] + slot if slot < C, else -1
 *   row_token     [rows] int32 out: token of each kept row (token order inside
 *                 an expert); needs room for min(T k, E C) entries
 *   x_disp        [rows, d] out (x_dtype) or NULL: x_disp[row] = x[token]; needs
 *                 room for min(T k, E C) rows.  Rows past expert_offset[E] and
 *                 entries past it in row_token are left untouched.
 *   ws            MOE_OP_DISPATCH workspace.
 * T = 0 writes zero counts and offsets.
 */
int moe_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int64_t capacity,
                 const void* x, int x_dtype, int32_t d, int32_t* expert_count,
                 int32_t* expert_offset, int32_t* slot, int32_t* row, int32_t* row_token,
                 void* x_disp, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Router with the optional MLP gate ("Code Walkthrough -- SER", Configuration:
 * use_mlp_gater with gater_hidden_dim; The gating / routing path: the logits
 * come from the linear router or the MLP gate):
 *   h = gW2 relu(gW1 x + gb1) + gb2   (hidden width H, evaluated in fp64)
 * then softmax, lse, top-k and gates exactly as moe_router_topk (b_sel, noise
 * and temperature likewise).
 *   gW1 [H, d], gb1 [H] or NULL, gW2 [E, H], gb2 [E] or NULL: fp32 device
 *   H % 8 == 0, H <= 256
 *   ws  MOE_OP_MLP_ROUTER workspace (the fp64 hidden layer, T x H).
 * T = 0 is a no-op.
 */
int moe_mlp_router_topk(const void* x, int x_dtype, int64_t T, int32_t d, const float* gW1,
                        const float* gb1, int32_t H, const float* gW2, const float* gb2,
                        const float* b_sel, int32_t E, int32_t k, const float* noise, float noise_std,
                        float temperature, float* logits, float* lse, int32_t* topk_idx, float* topk_gate,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The whole routing half of the layer in one call: moe_router_topk, then an
 * index-only moe_dispatch, then the statistics f, P and losses of
 * moe_route_stats (without credit), in three kernels.  Outputs are bit-identical
 * to those three calls.  ("Appendix C -- Acronyms & Symbols", Core MoE symbols,
 * Balancing, Capacity & communication; "Code Walkthrough -- SER", The gating /
 * routing path and Load balancing.)
 *   x, W_g, b_g, b_sel, noise, noise_std, temperature, logits, lse, topk_idx,
 *        topk_gate: as moe_router_topk
 *   capacity, expert_count, expert_offset, slot, row, row_token: as moe_dispatch
 *   alpha, beta, f, P, losses: as moe_route_stats
 *   ws   MOE_OP_ROUTE workspace (256-byte aligned).
 * T = 0 writes zero counts and offsets and nothing else.
 */
int moe_route(const void* x, int x_dtype, int64_t T, int32_t d, const float* W_g,
              const float* b_g, const float* b_sel, int32_t E, int32_t k, const float* noise,
              float noise_std, float temperature, int64_t capacity, float alpha, float beta,
              float* logits, float* lse, int32_t* topk_idx, float* topk_gate, int32_t* expert_count,
              int32_t* expert_offset, int32_t* slot, int32_t* row, int32_t* row_token, float* f,
              float* P, float* losses, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_route without a workspace, for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The same pass, kernels and bit-identical results as moe_route, with the
 * scratch in a static device array of MOE_ROUTE_NOALLOC_MAX_BYTES that the
 * library holds on every GPU it runs on until the process ends; the call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   Arguments: as moe_route, without ws and ws_bytes.
 *   Returns MOE_ERR_SCRATCH, enqueuing nothing, when the call would need more
 *   scratch than the array holds (moe_workspace_bytes(MOE_OP_ROUTE, ...) gives
 *   the need for bf16 x); other checks as moe_route.
 *   Every call on one GPU shares that GPU's array and leaves its contents
 *   behind (the pass needs no cleared scratch): calls that overlap on one GPU
 *   race, so order them on one stream.
 */
#define MOE_ROUTE_NOALLOC_MAX_BYTES ((size_t)64 << 20)

int moe_route_noalloc(const void* x, int x_dtype, int64_t T, int32_t d, const float* W_g,
                      const float* b_g, const float* b_sel, int32_t E, int32_t k, const float* noise,
                      float noise_std, float temperature, int64_t capacity, float alpha, float beta,
                      float* logits, float* lse, int32_t* topk_idx, float* topk_gate,
                      int32_t* expert_count, int32_t* expert_offset, int32_t* slot, int32_t* row,
                      int32_t* row_token, float* f, float* P, float* losses, hipStream_t stream);

/*
 * Grouped expert FFN over packed rows: for every group g and every row r in
 * group_offset[g] .. group_offset[g+1]-1, with A(r) = a[r] (a_rows == NULL) or
 * A(r) = a[a_rows[r]] (rows gathered on the fly, e.g. a = x, a_rows = row_token
 * from an index-only moe_dispatch):
 *   hidden[r] = act(W1[g] A(r) + b1[g]),   out[r] = W2[g] hidden[r] + b2[g]
 * ("Code Walkthrough -- SER", The gating / routing path: each expert runs its
 * two-layer MLP w1/b1 -> activation -> w2/b2.)
 *   a            [max_rows, d] device (dtype), or any [n, d] when a_rows != NULL
 *   a_rows       [max_rows] int32 device or NULL: source row of each packed row;
 *                entries below group_offset[G] must lie in [0, n)
 *   group_offset [G+1] int32 device, non-decreasing, group_offset[0] = 0
 *   max_rows     host upper bound on group_offset[G]; rows at or past max_rows
 *                are neither read nor written
 *   W1 [G, F, d], b1 [G, F], W2 [G, d_out, F], b2 [G, d_out] device (dtype)
 *   hidden       [max_rows, F] out (dtype): the activation, rounded once
 *   out          [max_rows, d_out] out (dtype)
 *   hidden_sqnorm [max_rows] fp32 out or NULL: sum over F of the activation
 *                squared, from the fp32 values before rounding
 *   dtype MOE_BF16 (MFMA, fp32 accumulate) or MOE_F32; act MOE_ACT_*.
 *   ws           MOE_OP_FFN workspace (used only when hidden_sqnorm != NULL).
 * max_rows = 0 is a successful no-op.
 */
int moe_grouped_ffn(const void* a, const int32_t* a_rows, const int32_t* group_offset, int32_t G,
                    int64_t max_rows, int32_t d, int32_t F, int32_t d_out, int dtype, int act,
                    const void* W1, const void* b1, const void* W2, const void* b2, void* hidden,
                    void* out, float* hidden_sqnorm, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/*
 * The two passes of moe_grouped_ffn as separate calls (same kernels, same
 * results), for callers that schedule or time them apart:
 *   moe_expert_up:   hidden[r] = act(W1[g] a[r] + b1[g])   (+ hidden_sqnorm[r])
 *   moe_expert_down: out[r]    = W2[g] hidden[r] + b2[g]
 * Arguments as in moe_grouped_ffn; moe_expert_up takes the MOE_OP_FFN
 * workspace when hidden_sqnorm != NULL.  max_rows = 0 is a successful no-op.
 */
int moe_expert_up(const void* a, const int32_t* a_rows, const int32_t* group_offset, int32_t G,
                  int64_t max_rows, int32_t d, int32_t F, int dtype, int act, const void* W1,
                  const void* b1, void* hidden, float* hidden_sqnorm, void* ws, size_t ws_bytes,
                  hipStream_t stream);

int moe_expert_down(const void* hidden, const int32_t* group_offset, int32_t G, int64_t max_rows,
                    int32_t F, int32_t d_out, int dtype, const void* W2, const void* b2, void* out,
                    hipStream_t stream);

/*
 * Sum of S always-on shared experts applied to every token:
 *   out[t] = sum_s ( W2[s] act(W1[s] x[t] + b1[s]) + b2[s] )
 * ("Appendix C -- Acronyms & Symbols", Parameter accounting: the set of
 * shared, always-on experts.)  Evaluated as one FFN of width S F: W1 [S, F, d]
 * is read as [S F, d], and the second layer runs over the S F hidden columns
 * segment by segment with the S output biases summed in fp32.
 *   x [T, d], W1 [S, F, d], b1 [S, F], W2 [S, d_out, F], b2 [S, d_out] device (dtype)
 *   hidden [T, S F] out (dtype, scratch), out [T, d_out] out (dtype)
 * T = 0 is a successful no-op.
 */
int moe_shared_ffn(const void* x, int64_t T, int32_t d, int32_t F, int32_t S, int32_t d_out,
                   int dtype, int act, const void* W1, const void* b1, const void* W2,
                   const void* b2, void* hidden, void* out, hipStream_t stream);

/*
 * Gate-weighted combine:
 *   y[t] = sum_{j : row[t,j] >= 0} topk_gate[t,j] * expert_out[row[t,j]]  (+ shared_out[t])
 * ("Code Walkthrough -- SER", The gating / routing path: outputs combined,
 * weighted by the gate weights; "Appendix C -- Acronyms & Symbols", Capacity &
 * communication: combine tensor = gate-weighted un-scatter.)  Dropped choices
 * contribute nothing; surviving gates are not renormalised.  fp32 accumulation
 * in j order, then the shared term, then one rounding to dtype.
 *   expert_out [rows, d_out] device (dtype); row [T, k] int32 device (from
 *   moe_dispatch); topk_gate [T, k] fp32 device; shared_out [T, d_out] or NULL;
 *   y [T, d_out] out (dtype).  T = 0 is a successful no-op.
 */
int moe_combine(const void* expert_out, const int32_t* row, const float* topk_gate,
                const void* shared_out, int64_t T, int32_t k, int32_t d_out, int dtype, void* y,
                hipStream_t stream);

/*
 * Routing statistics ("Appendix C -- Acronyms & Symbols", Balancing) and the
 * activation-weighted expert credit ("Sparse MoE Expert-Credit Loss
 * Reweighting Diagram", panel (b)):
 *   f[e]      = expert_count[e] / (k T)
 *   P[e]      = (1/T) sum_t exp(logits[t,e] - lse[t])
 *   losses[0] = alpha E sum_e f[e] P[e]   (Switch aux loss)
 *   losses[1] = beta (1/T) sum_t lse[t]^2  (z-loss)
 *   losses[2] = losses[0] + losses[1]
 *   credit[t,j]    = topk_gate[t,j] * sqrt(hidden_sqnorm[row[t,j]]), 0 when row = -1
 *   mean_credit[e] = (1/T) sum of credit over the kept choices of expert e
 *   expert_loss[e] = (1/T) sum of credit * token_loss[t] over the same choices
 *                    (the expert-attributed loss of panel (b), N = T)
 * Inputs: logits [T,E], lse [T], topk_idx [T,k], topk_gate [T,k], expert_count
 * [E] (device, from moe_router_topk / moe_dispatch).  Outputs f [E], P [E],
 * losses [3] fp32 device; all three may be NULL together when credit is
 * requested (the credit alone, e.g. after moe_route computed the statistics),
 * not one without the others.  Credit is computed when credit and mean_credit are
 * both non-NULL; it then needs hidden_sqnorm [rows], row [T,k], expert_offset
 * [E+1] and row_token [rows] (device).  The expert-attributed loss is computed
 * when token_loss [T] fp32 and expert_loss [E] fp32 (device) are both non-NULL,
 * and needs the credit.  Sums run in fp64 in a fixed order.
 *   ws  MOE_OP_STATS workspace.  T must be >= 1.
 */
int moe_route_stats(const float* logits, const float* lse, const int32_t* topk_idx,
                    const float* topk_gate, const int32_t* expert_count, int64_t T, int32_t E,
                    int32_t k, float alpha, float beta, float* f, float* P, float* losses,
                    const float* hidden_sqnorm, const int32_t* row, const int32_t* expert_offset,
                    const int32_t* row_token, float* credit, float* mean_credit,
                    const float* token_loss, float* expert_loss, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/*
 * Coefficient-of-variation balance losses ("Code Walkthrough -- SER", Load
 * balancing: balance across experts, total importance per expert, and the
 * aux loss combining load_balance_coef * load_balance + z_loss_coef * z_loss):
 *   importance[e] = sum over the batch of topk_gate[t,j] with topk_idx[t,j] = e
 *   out[0] = CV(expert_count)^2, out[1] = CV(importance)^2  (CV^2 = population
 *            variance / mean^2, 0 when the mean is 0)
 *   out[2] = (1/T) sum_t lse[t]^2
 *   out[3] = load_balance_coef * out[0] + z_loss_coef * out[2]
 * Inputs topk_gate, topk_idx [T,k], expert_count [E] (pre-capacity), lse [T]
 * device; outputs importance [E] and out [4] fp32 device.  Sums in fp64 in a
 * fixed order.  ws: MOE_OP_BALANCE workspace.  T must be >= 1.
 */
int moe_balance_losses(const float* topk_gate, const int32_t* topk_idx, const int32_t* expert_count,
                       const float* lse, int64_t T, int32_t E, int32_t k, float load_balance_coef,
                       float z_loss_coef, float* importance, float* out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * Aux-loss-free balancing ("Appendix C -- Acronyms & Symbols", Balancing:
 * per-expert selection bias b_i and its update rate gamma): every expert whose
 * pre-capacity load is below the mean load k T / E raises its bias by gamma,
 * above it lowers it by gamma, equal keeps it:
 *   b_sel[e] += gamma * sign(k T - E expert_count[e])   (sign exact in integers)
 * expert_count [E] int32 device; b_sel [E] fp32 device, updated in place.
 */
int moe_selection_bias_update(const int32_t* expert_count, int32_t E, int32_t k, int64_t T, float gamma,
                              float* b_sel, hipStream_t stream);

/*
 * One step of the EMA tracker and the layer-wise DRO weights ("Sparse MoE
 * Expert-Credit Loss Reweighting Diagram", panel (c)), in this order:
 *   ema[e] <- ema_decay * ema[e] + (1 - ema_decay) * expert_loss[e]
 *   mu     <- softmax(mu + eta * ema)
 *   dro_loss[0] = sum_e mu[e] * expert_loss[e]      (with the updated mu)
 * expert_loss [E] fp32 device (e.g. from moe_route_stats); ema, mu [E] fp32
 * device, updated in place; dro_loss [1] fp32 device.  fp64 arithmetic,
 * fixed order.
 */
int moe_dro_update(const float* expert_loss, int32_t E, float ema_decay, float eta, float* ema,
                   float* mu, float* dro_loss, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
