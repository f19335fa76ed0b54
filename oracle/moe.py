"""Loop-form float64 oracle of the sparse-MoE sub-layer forward pass.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pass, step by step, with the passage each step follows:
  1. router logits h = W_g x (+ router bias)       [Appendix C, Core MoE symbols; SER, gating path]
     or the optional MLP gate, plus the optional training noise of noisy top-k
                                                    [SER, Configuration; gating path]
     and the gate temperature tau, which divides those logits
                                                    [SER, gating path: gate_forward takes a temperature]
  2. P = softmax(h), lse = log sum_i e^{h_i}       [Appendix C, Core MoE symbols; Balancing (z-loss)]
  3. T_k(x) = the k experts with the highest scores, score = h + b_sel
                                                    [Appendix C, Core MoE symbols and Balancing (b_i);
                                                     SER, gating path: greedy picks the highest logits]
  4. g_i = P_i renormalised over T_k(x)            [Appendix C, Core MoE symbols]
  5. capacity C = ceil(C_f k T / E), dispatch in token order, overflow dropped
                                                    [Appendix C, Capacity & communication;
                                                     SER, Load balancing: capacity cap]
  6. each kept (token, expert) runs E_i(x) = W2 act(W1 x + b1) + b2
                                                    [SER, gating path: two-layer MLP w1/b1 -> act -> w2/b2]
  7. y = sum_i g_i E_i(x) + sum_{s in shared} E_s(x)
                                                    [SER, gating path: combined weighted by gate_weights;
                                                     Appendix C, Parameter accounting (shared experts)]
  8. f_i, P_i, L_aux = alpha E sum f_i P_i, L_z = beta mean (log sum e^h)^2
                                                    [Appendix C, Balancing]
  9. credit c = p ||h||_2 over the expert hidden state, and its per-expert mean
                                                    [Credit, panel (b)]

Readings where the pages leave a step open are listed with each function.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from fractions import Fraction
from typing import Dict, Optional, Sequence

import numpy as np
from scipy import special

from synth import Inputs, widen


# ----------------------------------------------------------------------------
# activations [SER, gating path: ReLU, GELU, Swish are named, not defined]
# Readings: ReLU max(0, z); GELU the exact form z * Phi(z) = 0.5 z (1 + erf(z / sqrt 2));
# Swish z * sigmoid(z) (beta = 1).
# ----------------------------------------------------------------------------
def _relu(z):
    return np.maximum(z, 0.0)


def _gelu(z):
    return 0.5 * z * (1.0 + special.erf(z / math.sqrt(2.0)))


def _swish(z):
    return z / (1.0 + np.exp(-z))


ACTIVATIONS = {"relu": _relu, "gelu": _gelu, "swish": _swish}


def activation(name: str, z: np.ndarray) -> np.ndarray:
    return ACTIVATIONS[name](z)


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------
def router_logits(x: np.ndarray, W_g: np.ndarray, b_g: Optional[np.ndarray]) -> np.ndarray:
    """h = W_g x (+ b_g) for every token row of x.

    [Appendix C, Core MoE symbols] h = W_g x with W_g in R^{E x d};
    [SER, gating path] the router is a linear layer with a bias (router_bias).
    Reading: the bias is added when the workload has one, else it is zero.
    """
    h = np.asarray(x, np.float64) @ np.asarray(W_g, np.float64).T
    if b_g is not None:
        h = h + np.asarray(b_g, np.float64)[None, :]
    return h


def mlp_gate_logits(x: np.ndarray, gW1: np.ndarray, gb1: np.ndarray, gW2: np.ndarray,
                    gb2: np.ndarray) -> np.ndarray:
    """h = gW2 relu(gW1 x + gb1) + gb2 for every token row of x.

    [SER, Configuration: use_mlp_gater, gater_hidden_dim; gating path: logits
    come from the linear router or the optional MLP gate]  Readings: a
    two-layer MLP with biases, hidden width gater_hidden_dim, ReLU between.
    """
    a = np.asarray(x, np.float64) @ np.asarray(gW1, np.float64).T + np.asarray(gb1, np.float64)[None, :]
    return np.maximum(a, 0.0) @ np.asarray(gW2, np.float64).T + np.asarray(gb2, np.float64)[None, :]


def noisy_logits(h: np.ndarray, noise: np.ndarray, sigma: float) -> np.ndarray:
    """h + sigma * eps with eps the supplied standard-normal draws [T, E].

    [SER, gating path: noisy top-k adds training noise to the logits before
    selection]  Readings: Gaussian noise of a fixed std sigma; the noisy
    logits replace the logits for everything after them (softmax, lse,
    selection, gates, statistics).
    """
    return np.asarray(h, np.float64) + float(sigma) * np.asarray(noise, np.float64)


def tempered_logits(h: np.ndarray, tau: float) -> np.ndarray:
    """h / tau: the gate's logits at temperature tau > 0.

    [SER, gating path: the gate-forward call takes a temperature argument
    and applies a softmax to the gate logits]  The page names the argument
    only.  Readings: the usual softmax temperature, dividing the logits (after
    any training noise) by tau; the tempered logits replace the logits for
    everything after them (the logits output, softmax, lse and z-loss,
    selection with the selection bias added to them, gates, statistics).
    tau = 1 leaves the pass unchanged.
    """
    tau = float(tau)
    if not (tau > 0.0 and math.isfinite(tau)):
        raise ValueError("temperature must be a finite positive number")
    return np.asarray(h, np.float64) / tau


def softmax_lse(h: np.ndarray):
    """P = softmax(h) and lse = log sum_i e^{h_i}, per token.

    [Appendix C, Core MoE symbols] P = softmax(h);
    [Appendix C, Balancing] the z-loss uses log sum_i e^{h_i}.
    Written as the definition (no max shift); the logits here stay far from
    float64 overflow.
    """
    eh = np.exp(h)
    s = eh.sum(axis=1, keepdims=True)
    return eh / s, np.log(s[:, 0])


def topk(h: np.ndarray, k: int, b_sel: Optional[np.ndarray] = None) -> np.ndarray:
    """T_k: indices of the k highest scores per token, score = h + b_sel.

    [Appendix C, Core MoE symbols] T_k(x) is the set of top-k indices;
    [SER, gating path] greedy top-k picks the highest logits;
    [Appendix C, Balancing] b_i is a per-expert selection bias.
    Readings: scores are logits, not probabilities (same order); equal scores
    go to the lower expert index; output order is (score desc, index asc).
    A stable sort on -score is exactly that order.
    """
    s = np.asarray(h, np.float64)
    if b_sel is not None:
        s = s + np.asarray(b_sel, np.float64)[None, :]
    order = np.argsort(-s, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def near_tie_gap(h: np.ndarray, k: int, b_sel: Optional[np.ndarray] = None) -> np.ndarray:
    """Per token, the smallest gap between consecutive scores among the k + 1
    highest (k when k = E; +inf when k = 1 = E).

    Comparator support, not part of the layer: the selected set depends on the
    k-th vs (k+1)-th gap and the listed order on the gaps inside the top k, so a
    token is a documented near-tie when any of these is tiny.
    """
    s = np.asarray(h, np.float64)
    if b_sel is not None:
        s = s + np.asarray(b_sel, np.float64)[None, :]
    E = s.shape[1]
    m = min(k + 1, E)
    if m < 2:
        return np.full(s.shape[0], np.inf)
    srt = -np.sort(-s, axis=1)[:, :m]
    return (srt[:, :-1] - srt[:, 1:]).min(axis=1)


def gates(P: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g_i = P_i / sum_{j in T_k} P_j for the selected experts, in idx order.

    [Appendix C, Core MoE symbols] gate weight = renormalised probability of the
    selected expert.  Reading: P is the softmax of the logits without the
    selection bias (the bias only picks the set).
    """
    sel = np.take_along_axis(P, idx, axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def capacity(capacity_factor: Optional[Fraction], k: int, T: int, E: int) -> Optional[int]:
    """C = ceil(C_f k T / E) evaluated exactly; None when dropless.

    [Appendix C, Capacity & communication] expert capacity, a fixed buffer size
    per expert.  C_f is taken as an exact rational (its decimal value).
    """
    if capacity_factor is None:
        return None
    q = Fraction(capacity_factor) * k * T / E
    return math.ceil(q)


@dataclass
class Dispatch:
    count: np.ndarray       # [E] assignments per expert, before capacity
    kept: np.ndarray        # [E] min(count, C)
    offset: np.ndarray      # [E+1] exclusive prefix of kept
    slot: np.ndarray        # [T, k] arrival rank of (t, j) at its expert
    row: np.ndarray         # [T, k] packed row, -1 when dropped
    row_token: np.ndarray   # [offset[E]] token of each packed row
    row_choice: np.ndarray  # [offset[E]] j of each packed row


def dispatch(idx: np.ndarray, E: int, C: Optional[int]) -> Dispatch:
    """Token-order dispatch under capacity C (None = no cap).

    [Appendix C, Capacity & communication] the dispatch tensor scatters tokens
    into fixed-size expert buffers; [SER, Load balancing] the capacity cap drops
    overflow tokens.  Readings: a token's arrival rank at expert e is the number
    of earlier tokens that chose e (a token's k choices are distinct experts);
    the first C arrivals are kept, later ones dropped and contribute nothing;
    kept rows are packed expert-major, token order inside an expert.
    """
    T, k = idx.shape
    n = [0] * E
    slot = np.zeros((T, k), np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            slot[t, j] = n[e]
            n[e] += 1
    count = np.array(n, np.int64)
    kept = count.copy() if C is None else np.minimum(count, C)
    offset = np.zeros(E + 1, np.int64)
    offset[1:] = np.cumsum(kept)
    row = np.full((T, k), -1, np.int64)
    row_token = np.zeros(int(offset[E]), np.int64)
    row_choice = np.zeros(int(offset[E]), np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if C is None or slot[t, j] < C:
                r = int(offset[e] + slot[t, j])
                row[t, j] = r
                row_token[r] = t
                row_choice[r] = j
    return Dispatch(count, kept, offset, slot, row, row_token, row_choice)


# ----------------------------------------------------------------------------
# experts and combine
# ----------------------------------------------------------------------------
def expert_ffn(xrows: np.ndarray, W1: np.ndarray, b1: np.ndarray, W2: np.ndarray,
               b2: np.ndarray, act: str):
    """E(x) = W2 act(W1 x + b1) + b2 for each row; also returns the hidden act(.).

    [SER, gating path] each expert is a two-layer MLP w1/b1 -> activation -> w2/b2;
    [Appendix C, Core MoE symbols] an expert is an FFN with its own weights.
    Layout: W1 [F, d], W2 [d_out, F] (out x in).
    """
    a = activation(act, xrows @ W1.T + b1[None, :])
    return a @ W2.T + b2[None, :], a


def combine(T: int, d_out: int, idx_gate: np.ndarray, row: np.ndarray,
            expert_out: Dict[int, np.ndarray], shared: Optional[np.ndarray],
            tokens: Sequence[int]) -> np.ndarray:
    """y_t = sum_j g_{t,j} E_{e_j}(x_t) over kept choices (+ shared experts, weight 1).

    [SER, gating path] expert outputs are combined, weighted by gate_weights;
    [Appendix C, Capacity & communication] the combine tensor is the
    gate-weighted un-scatter; [Appendix C, Parameter accounting] shared experts
    are always on.  Readings: dropped choices contribute zero and the kept
    gates are not renormalised again; shared experts are added ungated.
    """
    y = np.zeros((len(tokens), d_out))
    for i, t in enumerate(tokens):
        for j in range(row.shape[1]):
            r = int(row[t, j])
            if r >= 0:
                y[i] += idx_gate[t, j] * expert_out[r]
        if shared is not None:
            y[i] += shared[i]
    return y


# ----------------------------------------------------------------------------
# statistics
# ----------------------------------------------------------------------------
def route_stats(P: np.ndarray, lse: np.ndarray, count: np.ndarray, k: int,
                alpha: float, beta: float):
    """f_i, P_i, L_aux = alpha E sum_i f_i P_i and L_z = beta mean_t lse_t^2.

    [Appendix C, Balancing].  Readings: f_i = count_i / (k T), counted before
    the capacity cap (so sum f = 1); P_i is the batch mean of the full softmax
    of h; the overline of the z-loss is the mean over the T tokens.
    """
    T, E = P.shape
    f = count.astype(np.float64) / (k * T)
    Pbar = P.mean(axis=0)
    L_aux = alpha * E * float((f * Pbar).sum())
    L_z = beta * float((lse * lse).mean())
    return f, Pbar, L_aux, L_z


def credit(g: np.ndarray, row: np.ndarray, idx: np.ndarray, sqnorm_of_row: Dict[int, float],
           E: int, T: int, tokens: Sequence[int]):
    """c_{t,j} = g_{t,j} ||a_{t,j}||_2 and mean_credit_e = (1/T) sum over kept (t, j) with e_j = e.

    [Credit, panel (b)] activation-weighted credit sg(p ||h||_2); the
    stop-gradient is the identity in a forward pass.  Readings: p is the
    renormalised gate, h the expert's post-activation hidden state; the
    EMA-free mean takes the expert-attributed loss with every per-token loss
    equal to 1 and N = T; dropped choices have credit 0.
    """
    c = np.zeros((len(tokens), row.shape[1]))
    mean_c = np.zeros(E)
    for i, t in enumerate(tokens):
        for j in range(row.shape[1]):
            r = int(row[t, j])
            if r >= 0:
                c[i, j] = g[t, j] * math.sqrt(sqnorm_of_row[r])
                mean_c[int(idx[t, j])] += c[i, j]
    return c, mean_c / T


# ----------------------------------------------------------------------------
# whole pass
# ----------------------------------------------------------------------------
@dataclass
class OracleResult:
    logits: np.ndarray
    lse: np.ndarray
    P: np.ndarray
    topk_idx: np.ndarray
    topk_gate: np.ndarray
    gap: np.ndarray
    C: Optional[int]
    disp: Dispatch
    tokens: np.ndarray                      # tokens whose y / credit were evaluated
    y: np.ndarray                           # [len(tokens), d]
    expert_out: Dict[int, np.ndarray]       # packed row -> expert output (evaluated rows)
    sqnorm: Dict[int, float]                # packed row -> ||hidden||^2 (evaluated rows)
    shared_out: Optional[np.ndarray]        # [len(tokens), d] or None
    f: np.ndarray
    Pbar: np.ndarray
    L_aux: float
    L_z: float
    credit: Optional[np.ndarray] = None     # [len(tokens), k]
    mean_credit: Optional[np.ndarray] = None  # [E] (complete only when tokens = all)
    extra: Dict[str, object] = field(default_factory=dict)


def forward(inp: Inputs, tokens: Optional[Sequence[int]] = None,
            topk_override: Optional[np.ndarray] = None) -> OracleResult:
    """Run the whole pass on ``inp``.

    ``tokens`` limits the expert FFNs, the combine and the credit to those
    tokens (routing, dispatch and statistics always cover the whole batch).
    ``topk_override`` replaces the selected experts (used to re-evaluate the
    rest of the pass on another selection, e.g. a documented near-tie flip).
    """
    w = inp.workload
    dt = w.dtype
    T, E, k = w.T, w.E, w.k
    x = widen(inp.x, dt)
    if w.mlp_gate:
        h = mlp_gate_logits(x, inp.gW1, inp.gb1, inp.gW2, inp.gb2)
    else:
        h = router_logits(x, inp.W_g, inp.b_g)
    if w.router_noise is not None:
        h = noisy_logits(h, inp.noise, w.router_noise)
    if w.temperature != 1.0:
        h = tempered_logits(h, w.temperature)
    P, lse = softmax_lse(h)
    idx = topk(h, k, inp.b_sel) if topk_override is None else np.asarray(topk_override, np.int64)
    gap = near_tie_gap(h, k, inp.b_sel)
    g = gates(P, idx)
    C = capacity(w.capacity_factor, k, T, E)
    disp = dispatch(idx, E, C)

    tok = np.arange(T) if tokens is None else np.asarray(sorted(set(int(t) for t in tokens)), dtype=np.int64)
    want = np.zeros(T, bool)
    want[tok] = True
    expert_out: Dict[int, np.ndarray] = {}
    sqn: Dict[int, float] = {}
    for e in range(E):
        r0, r1 = int(disp.offset[e]), int(disp.offset[e + 1])
        rows = [r for r in range(r0, r1) if want[disp.row_token[r]]]
        if not rows:
            continue
        xr = x[disp.row_token[rows]]
        out, a = expert_ffn(xr, widen(inp.W1[e], dt), widen(inp.b1[e], dt),
                            widen(inp.W2[e], dt), widen(inp.b2[e], dt), w.act)
        for i, r in enumerate(rows):
            expert_out[r] = out[i]
            sqn[r] = float((a[i] * a[i]).sum())

    shared = None
    if w.n_shared:
        shared = np.zeros((len(tok), w.d))
        for s in range(w.n_shared):
            out, _ = expert_ffn(x[tok], widen(inp.sW1[s], dt), widen(inp.sb1[s], dt),
                                widen(inp.sW2[s], dt), widen(inp.sb2[s], dt), w.act)
            shared += out

    y = combine(T, w.d, g, disp.row, expert_out, shared, tok)
    f, Pbar, L_aux, L_z = route_stats(P, lse, disp.count, k, w.alpha, w.beta)
    res = OracleResult(h, lse, P, idx, g, gap, C, disp, tok, y, expert_out, sqn, shared,
                       f, Pbar, L_aux, L_z)
    if w.credit:
        res.credit, res.mean_credit = credit(g, disp.row, idx, sqn, E, T, tok)
    return res


def expert_rows(inp: Inputs, res: OracleResult, e: int, token_loss: Optional[np.ndarray] = None):
    """Every kept row of expert e in full: the expert outputs and ||hidden||^2 of
    its packed rows, its mean credit and (with per-token losses) its
    expert-attributed loss.

    The same steps as ``forward`` restricted to one expert, for batches too
    large to evaluate whole: [SER, gating path] the two-layer expert on the
    rows dispatched to it; [Credit, panel (b)] credit g ||a||_2 per kept
    choice and the per-expert sums (1/N) sum c (and (1/N) sum c l_j), N = T.
    ``res`` supplies the routing and dispatch (e.g. forward(inp, tokens=[])).
    Returns (rows, out [n, d], sqnorm [n], mean_credit_e, expert_loss_e or None).
    """
    w = inp.workload
    dt = w.dtype
    r0, r1 = int(res.disp.offset[e]), int(res.disp.offset[e + 1])
    rows = np.arange(r0, r1)
    tok = res.disp.row_token[r0:r1]
    ch = res.disp.row_choice[r0:r1]
    xr = widen(inp.x, dt)[tok]
    out, a = expert_ffn(xr, widen(inp.W1[e], dt), widen(inp.b1[e], dt),
                        widen(inp.W2[e], dt), widen(inp.b2[e], dt), w.act)
    sq = (a * a).sum(axis=1)
    c = res.topk_gate[tok, ch] * np.sqrt(sq)
    mean_c = float(c.sum()) / w.T
    loss = None if token_loss is None else float((c * np.asarray(token_loss, np.float64)[tok]).sum()) / w.T
    return rows, out, sq, mean_c, loss
