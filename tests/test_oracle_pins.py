"""Pins for the CPU oracle: worked examples derived by hand, closed forms,
invariants, textbook routines and brute force.  CPU only.

Each test names the passage it checks:
  [Appendix C]  "Appendix C -- Acronyms & Symbols"
  [SER]         "Code Walkthrough -- SER (Sparse Expert Routing)"
  [Credit]      "Sparse MoE Expert-Credit Loss Reweighting Diagram", panel (b)
"""
import math
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy import special, stats

import oracle
import synth
from oracle.moe import dispatch, expert_ffn, gates, route_stats, softmax_lse, topk


def _inputs_from_arrays(x, W_g, b_g, experts, k, act="relu", cf=None, b_sel=None,
                        shared=None, credit=False, alpha=0.01, beta=1e-3):
    """Wrap hand-made float arrays as fp32 synth.Inputs (values chosen exactly representable)."""
    T, d = x.shape
    E = W_g.shape[0]
    F = experts[0][0].shape[0]
    w = synth.Workload(name="hand", tag=0, T=T, d=d, E=E, k=k, F=F, act=act, dtype="f32",
                       capacity_factor=cf, n_shared=0 if shared is None else len(shared),
                       alpha=alpha, beta=beta, credit=credit)
    f32 = lambda a: np.asarray(a, np.float64)  # keep float64 so hand values are exact
    inp = synth.Inputs(w, f32(x), f32(W_g), None if b_g is None else f32(b_g),
                       None if b_sel is None else f32(b_sel),
                       np.stack([f32(e[0]) for e in experts]), np.stack([f32(e[1]) for e in experts]),
                       np.stack([f32(e[2]) for e in experts]), np.stack([f32(e[3]) for e in experts]))
    if shared is not None:
        inp.sW1 = np.stack([f32(e[0]) for e in shared]); inp.sb1 = np.stack([f32(e[1]) for e in shared])
        inp.sW2 = np.stack([f32(e[2]) for e in shared]); inp.sb2 = np.stack([f32(e[3]) for e in shared])
    return inp


# ---------------------------------------------------------------------------
# Hand-derived worked example (T=2, d=3, E=3, k=2)
#   x0 = (1,0,0), x1 = (0,1,0); W_g rows (ln3,0,0), (0,ln5,0), (ln2,ln5,0), no bias.
#   token 0: e^h = (3,1,2), P = (1/2, 1/6, 1/3), top-2 = (0, 2), gates (3/5, 2/5), lse = ln 6
#   token 1: e^h = (1,5,5), P = (1/11, 5/11, 5/11), tie at ln5 -> lower index first:
#            top-2 = (1, 2), gates (1/2, 1/2), lse = ln 11
#   counts (1,1,2) -> f = (1/4, 1/4, 1/2)
#   Pbar = (13/44, 41/132, 13/33); L_aux = alpha * 3 * sum f*Pbar = alpha * 23/22
#   L_z = beta * ((ln 6)^2 + (ln 11)^2) / 2
#   experts: W1 = I, b1 = 0, ReLU, W2 = c_e I, b2 = 0 with c = (1,2,3):
#     y0 = (3/5*1 + 2/5*3) x0 = (9/5, 0, 0); y1 = (1/2*2 + 1/2*3) x1 = (0, 5/2, 0)
#   credit = g * ||relu(x)|| = g; mean credit = ((3/5)/2, (1/2)/2, (2/5+1/2)/2) = (3/10, 1/4, 9/20)
# ---------------------------------------------------------------------------
def _hand_example(cf=None, credit=True):
    L3, L5, L2 = math.log(3), math.log(5), math.log(2)
    x = np.array([[1.0, 0, 0], [0, 1.0, 0]])
    W_g = np.array([[L3, 0, 0], [0, L5, 0], [L2, L5, 0]])
    I = np.eye(3)
    experts = [(I, np.zeros(3), c * I, np.zeros(3)) for c in (1.0, 2.0, 3.0)]
    return _inputs_from_arrays(x, W_g, None, experts, k=2, cf=cf, credit=credit)


def test_hand_example_routing():
    """[Appendix C, Core MoE symbols] h, P, T_k, g; [SER, gating path] greedy top-k."""
    r = oracle.forward(_hand_example())
    np.testing.assert_allclose(r.P, [[1 / 2, 1 / 6, 1 / 3], [1 / 11, 5 / 11, 5 / 11]], atol=1e-15)
    np.testing.assert_allclose(r.lse, [math.log(6), math.log(11)], atol=1e-15)
    assert r.topk_idx.tolist() == [[0, 2], [1, 2]]
    np.testing.assert_allclose(r.topk_gate, [[3 / 5, 2 / 5], [1 / 2, 1 / 2]], atol=1e-15)


def test_hand_example_stats():
    """[Appendix C, Balancing] f_i, P_i, L_aux = alpha E sum f P, L_z = beta mean lse^2."""
    r = oracle.forward(_hand_example())
    assert r.disp.count.tolist() == [1, 1, 2]
    np.testing.assert_allclose(r.f, [0.25, 0.25, 0.5], atol=0)
    np.testing.assert_allclose(r.Pbar, [13 / 44, 41 / 132, 13 / 33], atol=1e-15)
    assert r.L_aux == pytest.approx(0.01 * 23 / 22, rel=1e-14)
    assert r.L_z == pytest.approx(1e-3 * (math.log(6) ** 2 + math.log(11) ** 2) / 2, rel=1e-14)


def test_hand_example_output_and_credit():
    """[SER, gating path] gate-weighted combine of two-layer experts; [Credit, panel (b)]."""
    r = oracle.forward(_hand_example())
    np.testing.assert_allclose(r.y, [[9 / 5, 0, 0], [0, 5 / 2, 0]], atol=1e-14)
    np.testing.assert_allclose(r.credit, [[3 / 5, 2 / 5], [1 / 2, 1 / 2]], atol=1e-15)
    np.testing.assert_allclose(r.mean_credit, [3 / 10, 1 / 4, 9 / 20], atol=1e-15)


def test_hand_example_selection_bias():
    """[Appendix C, Balancing] b_i enters the selection only.  b_sel = (0, 1, 0):
    token 0 scores (ln3, 1, ln2) -> top-2 (0, 1); gates from the unbiased P = (1/2, 1/6, 1/3):
    (3/4, 1/4) (the biased softmax would give 3/(3+e), e/(3+e)).
    token 1 scores (0, ln5+1, ln5) -> top-2 (1, 2); gates (1/2, 1/2)."""
    inp = _hand_example()
    inp.b_sel = np.array([0.0, 1.0, 0.0])
    r = oracle.forward(inp)
    assert r.topk_idx.tolist() == [[0, 1], [1, 2]]
    np.testing.assert_allclose(r.topk_gate, [[3 / 4, 1 / 4], [1 / 2, 1 / 2]], atol=1e-15)
    np.testing.assert_allclose(r.P[0], [1 / 2, 1 / 6, 1 / 3], atol=1e-15)


def test_hand_credit_norm():
    """[Credit, panel (b)] c = g ||h||_2 with a hidden of norm 5: x0 = (3, 4, 0) routed
    alone (E=1, k=1, g=1), W1 = I, b1 = 0, ReLU -> h = (3, 4, 0), ||h|| = 5, credit 5;
    mean credit over T=2 tokens (x1 = (0, 0, 1) -> ||h|| = 1) = (5 + 1) / 2 = 3."""
    x = np.array([[3.0, 4.0, 0.0], [0.0, 0.0, 1.0]])
    I = np.eye(3)
    inp = _inputs_from_arrays(x, np.zeros((1, 3)), None, [(I, np.zeros(3), I, np.zeros(3))],
                              k=1, credit=True)
    r = oracle.forward(inp)
    np.testing.assert_allclose(r.credit, [[5.0], [1.0]], atol=1e-15)
    np.testing.assert_allclose(r.mean_credit, [3.0], atol=1e-15)
    np.testing.assert_allclose(r.y, x, atol=0)


def test_hand_example_capacity_drop():
    """[Appendix C, Capacity & communication] C = ceil(C_f k T / E) = ceil(1/2*2*2/3) = 1;
    [SER, Load balancing] overflow dropped: token 1's choice of expert 2 arrives second and
    is dropped; its gate is not renormalised (y1 = 1/2 * 2 * x1)."""
    r = oracle.forward(_hand_example(cf=Fraction(1, 2)))
    assert r.C == 1
    assert r.disp.slot.tolist() == [[0, 0], [0, 1]]
    assert r.disp.row.tolist() == [[0, 2], [1, -1]]
    assert r.disp.offset.tolist() == [0, 1, 2, 3]
    assert r.disp.row_token.tolist() == [0, 1, 0]
    np.testing.assert_allclose(r.y, [[9 / 5, 0, 0], [0, 1, 0]], atol=1e-14)
    # f is counted before the cap (sum f = 1), so the stats do not change with C
    np.testing.assert_allclose(r.f, [0.25, 0.25, 0.5], atol=0)
    np.testing.assert_allclose(r.credit, [[3 / 5, 2 / 5], [1 / 2, 0]], atol=1e-15)


def test_hand_expert_ffn():
    """[SER, gating path] w1/b1 -> act -> w2/b2 with a non-square W1 (F=3, d=2):
    x=(1,-2), W1=[[1,0],[0,1],[1,1]], b1=(0,0,.5) -> z=(1,-2,-.5) -> relu (1,0,0);
    W2=[[2,0,1],[0,3,1]], b2=(.25,0) -> out=(2.25, 0); ||a||^2 = 1."""
    W1 = np.array([[1.0, 0], [0, 1], [1, 1]])
    W2 = np.array([[2.0, 0, 1], [0, 3, 1]])
    out, a = expert_ffn(np.array([[1.0, -2.0]]), W1, np.array([0, 0, 0.5]), W2, np.array([0.25, 0]), "relu")
    np.testing.assert_allclose(out, [[2.25, 0.0]], atol=0)
    np.testing.assert_allclose(a, [[1.0, 0, 0]], atol=0)


# ---------------------------------------------------------------------------
# activations against textbook values and other library routines
# ---------------------------------------------------------------------------
def test_activations_textbook():
    """[SER, gating path] ReLU / GELU / Swish.  GELU(z) = z Phi(z) with Phi(1) = 0.8413447460685429
    (standard normal table); Swish(1) = 1/(1+e^-1) = 0.7310585786300049."""
    assert oracle.activation("gelu", np.array([1.0]))[0] == pytest.approx(0.8413447460685429, abs=1e-15)
    assert oracle.activation("gelu", np.array([-1.0]))[0] == pytest.approx(-0.15865525393145707, abs=1e-15)
    assert oracle.activation("swish", np.array([1.0]))[0] == pytest.approx(0.7310585786300049, abs=1e-15)
    z = np.linspace(-8, 8, 1001)
    np.testing.assert_allclose(oracle.activation("gelu", z), z * stats.norm.cdf(z), atol=1e-15)
    np.testing.assert_allclose(oracle.activation("swish", z), z * special.expit(z), atol=1e-15)
    np.testing.assert_array_equal(oracle.activation("relu", z), np.where(z > 0, z, 0.0))


def test_softmax_lse_library():
    """[Appendix C, Core MoE symbols / Balancing] softmax and log-sum-exp vs scipy."""
    h = np.random.default_rng(0).normal(size=(50, 17)) * 3
    P, lse = softmax_lse(h)
    np.testing.assert_allclose(P, special.softmax(h, axis=1), rtol=1e-13)
    np.testing.assert_allclose(lse, special.logsumexp(h, axis=1), rtol=1e-14)


def test_router_logits_exact_sum():
    """[Appendix C, Core MoE symbols] h = W_g x (+ bias): each logit against an exactly
    rounded sum (math.fsum) of the products."""
    rng = np.random.default_rng(1)
    x = rng.normal(size=(7, 13)); W = rng.normal(size=(5, 13)); b = rng.normal(size=5)
    h = oracle.router_logits(x, W, b)
    for t in range(7):
        for e in range(5):
            ref = math.fsum([x[t, j] * W[e, j] for j in range(13)] + [b[e]])
            assert h[t, e] == pytest.approx(ref, abs=1e-14)


# ---------------------------------------------------------------------------
# capacity and dispatch
# ---------------------------------------------------------------------------
def test_capacity_values():
    """[Appendix C, Capacity & communication] C = ceil(C_f k T / E), exact rational arithmetic:
    4*2*16/4 = 32; 1.25*2*4096/8 = 1280; 1*1*16384/64 = 256; 1.25*1*10/3 = 4.1666 -> 5;
    dropless -> None."""
    assert oracle.capacity(synth.TINY.capacity_factor, 2, 16, 4) == 32
    assert oracle.capacity(synth.DEFAULT.capacity_factor, 2, 4096, 8) == 1280
    assert oracle.capacity(synth.SWITCH_ZIPF.capacity_factor, 1, 16384, 64) == 256
    assert oracle.capacity(Fraction(5, 4), 1, 10, 3) == 5
    assert oracle.capacity(Fraction(1), 2, 6, 4) == 3          # exactly integral: no round-up
    assert oracle.capacity(Fraction(0), 2, 6, 4) == 0
    assert oracle.capacity(None, 2, 6, 4) is None


def test_dispatch_hand():
    """[SER, Load balancing] capacity cap in token order, E=2, k=1, C=2:
    choices 0,0,1,0,0,1,1,1 -> arrival ranks 0,1,0,2,3,1,2,3; the first two arrivals
    of each expert are kept: rows t0->0, t1->1, t2->2, t5->3, the rest dropped."""
    idx = np.array([[0], [0], [1], [0], [0], [1], [1], [1]])
    d = dispatch(idx, 2, 2)
    assert d.slot[:, 0].tolist() == [0, 1, 0, 2, 3, 1, 2, 3]
    assert d.count.tolist() == [4, 4]
    assert d.kept.tolist() == [2, 2]
    assert d.offset.tolist() == [0, 2, 4]
    assert d.row[:, 0].tolist() == [0, 1, 2, -1, -1, 3, -1, -1]
    assert d.row_token.tolist() == [0, 1, 2, 5]


def test_dispatch_multi_choice_order():
    """Arrival order is token order across choices j: token 1's first choice of expert 1
    comes after token 0's second choice of expert 1.  idx = [[0,1],[1,2],[2,0]], C=1:
    ranks [[0,0],[1,0],[1,1]] -> kept (0,0)(0,1)(1,1): rows [[0,1],[-1,2],[-1,-1]]."""
    d = dispatch(np.array([[0, 1], [1, 2], [2, 0]]), 3, 1)
    assert d.slot.tolist() == [[0, 0], [1, 0], [1, 1]]
    assert d.row.tolist() == [[0, 1], [-1, 2], [-1, -1]]
    assert d.count.tolist() == [2, 2, 2]


@settings(max_examples=60, deadline=None)
@given(T=st.integers(1, 40), E=st.integers(1, 9), data=st.data())
def test_dispatch_invariants(T, E, data):
    """[Appendix C, Capacity & communication] kept_e = min(count_e, C); kept set = first C
    arrivals; sum kept + dropped = kT; C >= T => no drops; rows packed expert-major."""
    k = data.draw(st.integers(1, E))
    C = data.draw(st.one_of(st.none(), st.integers(0, T + 2)))
    rng = np.random.default_rng(data.draw(st.integers(0, 2**31)))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    d = dispatch(idx, E, C)
    assert d.count.sum() == T * k
    assert (d.kept == (d.count if C is None else np.minimum(d.count, C))).all()
    assert (d.row >= 0).sum() == d.kept.sum()
    if C is not None and C >= T:
        assert (d.row >= 0).all()
    for e in range(E):
        sel = (idx == e)
        ranks = np.sort(d.slot[sel])
        assert ranks.tolist() == list(range(int(d.count[e])))
        rows = d.row[sel & (d.row >= 0)]
        assert sorted(rows.tolist()) == list(range(int(d.offset[e]), int(d.offset[e + 1])))
    toks = d.row_token
    for e in range(E):   # token order inside an expert
        seg = toks[d.offset[e]:d.offset[e + 1]]
        assert (np.diff(seg) > 0).all()


# ---------------------------------------------------------------------------
# top-k against brute force; gates
# ---------------------------------------------------------------------------
@settings(max_examples=200, deadline=None)
@given(E=st.integers(1, 6), data=st.data())
def test_topk_brute_force(E, data):
    """[Appendix C, Core MoE symbols] T_k by enumeration of all k-subsets; integer-valued
    scores make exact ties frequent (lowest index wins)."""
    k = data.draw(st.integers(1, E))
    T = data.draw(st.integers(1, 8))
    ints = data.draw(st.booleans())
    rng = np.random.default_rng(data.draw(st.integers(0, 2**31)))
    h = rng.integers(-2, 3, size=(T, E)).astype(float) if ints else rng.normal(size=(T, E))
    idx = topk(h, k)
    for t in range(T):
        assert tuple(idx[t].tolist()) == oracle.brute_topk(h[t], k)


def test_near_tie_gap_hand():
    """Smallest consecutive gap among the k+1 top scores: scores (5, 1, 3, 3.25, 0),
    k=2 -> sorted 5, 3.25, 3 -> gaps 1.75, 0.25 -> 0.25; k=1 -> 5 vs 3.25 -> 1.75;
    k=5=E -> min over all consecutive gaps of 5, 3.25, 3, 1, 0 -> 0.25; E=k=1 -> inf."""
    h = np.array([[5.0, 1.0, 3.0, 3.25, 0.0]])
    assert oracle.near_tie_gap(h, 2)[0] == 0.25
    assert oracle.near_tie_gap(h, 1)[0] == 1.75
    assert oracle.near_tie_gap(h, 5)[0] == 0.25
    assert oracle.near_tie_gap(np.array([[2.0]]), 1)[0] == np.inf


def test_topk_selection_bias_separation():
    """[Appendix C, Balancing] b_i changes only the selection: gates are unchanged by a
    b_sel that keeps T_k; b_sel = 0 equals no bias; a large b_sel changes the set but
    the gates stay the renormalised P of the unbiased logits."""
    rng = np.random.default_rng(3)
    h = rng.normal(size=(64, 8))
    P, _ = softmax_lse(h)
    i0 = topk(h, 3)
    assert (topk(h, 3, np.zeros(8)) == i0).all()
    shift = np.full(8, 0.7)                      # same shift for all: same order
    i1 = topk(h, 3, shift)
    assert (i1 == i0).all()
    np.testing.assert_array_equal(gates(P, i1), gates(P, i0))
    big = np.zeros(8); big[7] = 100.0            # forces expert 7 first
    i2 = topk(h, 3, big)
    assert (i2[:, 0] == 7).all()
    g2 = gates(P, i2)
    np.testing.assert_allclose(g2[:, 0], P[:, 7] / np.take_along_axis(P, i2, 1).sum(1), rtol=1e-15)


@settings(max_examples=50, deadline=None)
@given(T=st.integers(1, 30), E=st.integers(1, 10), data=st.data())
def test_gates_sum_to_one(T, E, data):
    """[Appendix C, Core MoE symbols] renormalised gates of the selected experts sum to 1."""
    k = data.draw(st.integers(1, E))
    h = np.random.default_rng(data.draw(st.integers(0, 2**31))).normal(size=(T, E)) * 4
    P, _ = softmax_lse(h)
    g = gates(P, topk(h, k))
    np.testing.assert_allclose(g.sum(axis=1), 1.0, atol=1e-12)
    assert (g > 0).all()
    assert (np.diff(g, axis=1) <= 1e-15).all()   # no selection bias: gates descend with scores


# ---------------------------------------------------------------------------
# whole-pass properties
# ---------------------------------------------------------------------------
def _small(w, **kw):
    return synth.draw(w.with_(**kw))


def _experts64(inp):
    dt = inp.dtype
    return [(synth.widen(inp.W1[e], dt), synth.widen(inp.b1[e], dt), synth.widen(inp.W2[e], dt),
             synth.widen(inp.b2[e], dt)) for e in range(inp.workload.E)]


def test_k_equals_E_is_dense_softmax_mixture():
    """k = E and no drops: top-k routing is the dense softmax-gated mixture
    y = sum_e softmax(h)_e E_e(x) ([Appendix C, Core MoE symbols] with T_k = all experts)."""
    for act in ("relu", "gelu", "swish"):
        inp = _small(synth.TINY, k=4, act=act)
        r = oracle.forward(inp)
        x = synth.widen(inp.x, inp.dtype)
        y = oracle.dense_softmax_mixture(x, r.logits, _experts64(inp), act)
        np.testing.assert_allclose(r.y, y, atol=1e-12)


@pytest.mark.parametrize("cf", [None, Fraction(1, 4), Fraction(1, 2), Fraction(1), Fraction(4)])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_dense_form_equals_loop_form(cf, k):
    """[Appendix C, Capacity & communication] dense D / D~ einsum form vs the loop form:
    same counts, same arrival ranks, same kept set and output, with and without drops."""
    inp = _small(synth.TINY, T=24, E=5, k=k, capacity_factor=cf, act="gelu")
    r = oracle.forward(inp)
    x = synth.widen(inp.x, inp.dtype)
    y, D, count = oracle.dense_dispatch_combine(x, r.topk_idx, r.topk_gate, 5, r.C, _experts64(inp), "gelu")
    assert (count == r.disp.count).all()
    np.testing.assert_allclose(y, r.y, atol=1e-12)
    kept = D.sum(axis=2)
    for t in range(inp.workload.T):
        for j in range(k):
            e = r.topk_idx[t, j]
            assert kept[t, e] == (1.0 if r.disp.row[t, j] >= 0 else 0.0)
            if r.disp.row[t, j] >= 0:
                assert D[t, e, r.disp.slot[t, j]] == 1.0


def test_uniform_router_closed_forms():
    """[Appendix C, Balancing] W_g = 0: P = 1/E exactly, T_k = {0..k-1} (lowest index),
    L_aux = alpha exactly (for k a power of two; any capacity), L_z = beta (ln E)^2."""
    for E, k, cf in [(8, 2, Fraction(5, 4)), (4, 1, Fraction(1, 2)), (16, 4, None), (8, 8, None)]:
        inp = _small(synth.TINY, E=E, k=k, capacity_factor=cf, router_bias=None)
        inp.W_g = np.zeros_like(inp.W_g)
        r = oracle.forward(inp)
        assert (r.P == 1.0 / E).all()
        assert (r.topk_idx == np.arange(k)[None, :]).all()
        assert r.L_aux == 0.01
        assert r.L_z == pytest.approx(1e-3 * math.log(E) ** 2, rel=1e-15)
        np.testing.assert_array_equal(r.topk_gate, 1.0 / k)


@pytest.mark.parametrize("w", [synth.TINY, synth.DEFAULT.with_(T=256), synth.SWITCH_ZIPF.with_(T=512, d=64, F=64),
                               synth.FINE_SHARED.with_(T=128, d=64, F=64),
                               synth.LARGE_CREDIT.with_(T=64, d=64, F=32)], ids=lambda w: w.name[:12])
def test_statistic_invariants(w):
    """[Appendix C, Balancing] sum f = 1 exactly, sum P_i = 1; [Credit, panel (b)]
    T * sum_e mean_credit_e = sum_{t,j} credit_{t,j}; credit >= 0."""
    inp = synth.draw(w)
    r = oracle.forward(inp)
    assert float(Fraction(int(r.disp.count.sum()), w.k * w.T)) == 1.0
    assert r.f.sum() == pytest.approx(1.0, abs=1e-15)
    assert r.Pbar.sum() == pytest.approx(1.0, abs=1e-12)
    if w.credit:
        assert w.T * r.mean_credit.sum() == pytest.approx(r.credit.sum(), rel=1e-12)
        assert (r.credit >= 0).all()


def test_relu_credit_zero_when_hidden_is_dead():
    """[Credit, panel (b)] ReLU expert whose pre-activations are all <= 0 has ||h|| = 0."""
    inp = _small(synth.TINY, credit=True)
    inp.b1 = np.full_like(inp.b1, -1e3)
    r = oracle.forward(inp)
    assert (r.credit == 0).all()
    assert (r.mean_credit == 0).all()


def test_shared_experts_identity():
    """[Appendix C, Parameter accounting] shared experts are always on: with routed
    W2 = 0, b2 = 0 the output is sum_s E_s(x), evaluated here expert by expert."""
    inp = _small(synth.FINE_SHARED, T=32, d=16, F=24, E=8, k=2)
    inp.W2 = np.zeros_like(inp.W2); inp.b2 = np.zeros_like(inp.b2)
    r = oracle.forward(inp)
    x = synth.widen(inp.x, "bf16")
    ref = 0
    for s in range(2):
        z = x @ synth.widen(inp.sW1[s], "bf16").T + synth.widen(inp.sb1[s], "bf16")
        ref = ref + (z * special.expit(z)) @ synth.widen(inp.sW2[s], "bf16").T + synth.widen(inp.sb2[s], "bf16")
    np.testing.assert_allclose(r.y, ref, atol=1e-12)


def test_token_subset_matches_full():
    """Evaluating the FFN/combine on a token subset gives the same rows as the full pass."""
    inp = _small(synth.DEFAULT, T=96, d=32, F=48)
    full = oracle.forward(inp)
    sub = oracle.forward(inp, tokens=[5, 17, 90])
    np.testing.assert_allclose(sub.y, full.y[[5, 17, 90]], atol=0)


def test_topk_override_rewires_dispatch():
    """A substituted selection flows through dispatch and combine."""
    inp = _small(synth.TINY)
    r = oracle.forward(inp)
    idx = r.topk_idx.copy()
    idx[0] = idx[0][::-1]
    r2 = oracle.forward(inp, topk_override=idx)
    assert (r2.topk_idx == idx).all()
    np.testing.assert_allclose(r2.topk_gate[0], r.topk_gate[0][::-1], atol=1e-15)
    np.testing.assert_allclose(r2.y, r.y, atol=1e-13)   # same set: same output


def test_expert_rows_hand_example():
    """The per-expert evaluation on the hand example: expert 2 holds token 0
    (choice 1, gate 2/5) and token 1 (choice 1, gate 1/2); with W1 = I, ReLU,
    W2 = 3 I its rows are 3 x_t, ||a||^2 = 1, mean credit (2/5 + 1/2) / 2 =
    9/20, and with per-token losses (2, 4) the expert loss (2/5 * 2 + 1/2 * 4) / 2
    = 7/5 [Credit, panel (b)]."""
    inp = _hand_example()
    res = oracle.forward(inp, tokens=[])
    rows, out, sq, mc, loss = oracle.expert_rows(inp, res, 2, token_loss=np.array([2.0, 4.0]))
    assert rows.tolist() == [2, 3]
    np.testing.assert_allclose(out, [[3, 0, 0], [0, 3, 0]], atol=1e-15)
    np.testing.assert_allclose(sq, [1.0, 1.0], atol=1e-15)
    assert mc == pytest.approx(9 / 20, rel=1e-14)
    assert loss == pytest.approx(7 / 5, rel=1e-14)


@pytest.mark.parametrize("w", [synth.LARGE_CREDIT.with_(T=96, d=32, F=48, E=6, k=3),
                               synth.SWITCH_ZIPF.with_(T=200, d=32, F=24, E=8, k=1, credit=True)])
def test_expert_rows_matches_whole_pass(w):
    """Expert by expert, the restricted evaluation reproduces the whole pass's
    expert outputs, ||hidden||^2, mean credit and expert-attributed loss."""
    inp = synth.draw(w)
    full = oracle.forward(inp)
    tl = synth.token_losses(w).astype(np.float64)
    want_loss = oracle.expert_attributed_loss(full.credit, full.topk_idx, tl, w.E)
    res = oracle.forward(inp, tokens=[])
    for e in range(w.E):
        rows, out, sq, mc, loss = oracle.expert_rows(inp, res, e, token_loss=tl)
        for i, r in enumerate(rows):
            np.testing.assert_allclose(out[i], full.expert_out[r], rtol=1e-13, atol=1e-13)
            assert sq[i] == pytest.approx(full.sqnorm[r], rel=1e-13)
        assert mc == pytest.approx(full.mean_credit[e], rel=1e-12, abs=1e-300)
        assert loss == pytest.approx(want_loss[e], rel=1e-12, abs=1e-300)
