"""Pins of the router variants in the oracle: the MLP gate and noisy top-k."""
import numpy as np
from scipy import special, stats

import oracle
import synth


def test_mlp_gate_hand_example():
    gW1 = np.array([[1.0, -1.0], [0.5, 0.5]])
    gb1 = np.array([0.0, -1.0])
    gW2 = np.array([[1.0, 2.0], [-1.0, 0.0]])
    gb2 = np.array([0.5, 0.0])
    x = np.array([[3.0, 1.0], [1.0, 3.0]])
    # token 0: pre-activation (2, 1) -> h = (2 + 2 + 0.5, -2); token 1: (-2, 1) -> relu (0, 1) -> (2.5, 0)
    np.testing.assert_array_equal(oracle.mlp_gate_logits(x, gW1, gb1, gW2, gb2), [[4.5, -2.0], [2.5, 0.0]])


def test_mlp_gate_reduces_to_linear_router():
    """gW1 = I with a bias that keeps every pre-activation positive: the gate is
    the linear router with W_g = gW2 and b_g = gW2 c + gb2."""
    rng = np.random.default_rng(1)
    d, E, T = 6, 5, 20
    x = rng.standard_normal((T, d))
    c = np.full(d, 50.0)
    gW2, gb2 = rng.standard_normal((E, d)), rng.standard_normal(E)
    got = oracle.mlp_gate_logits(x, np.eye(d), c, gW2, gb2)
    np.testing.assert_allclose(got, oracle.router_logits(x, gW2, gW2 @ c + gb2), rtol=1e-12, atol=1e-12)


def test_mlp_gate_dead_hidden_gives_bias():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 4))
    gb2 = np.array([0.3, -0.1, 0.2])
    h = oracle.mlp_gate_logits(x, rng.standard_normal((8, 4)), np.full(8, -1e6), rng.standard_normal((3, 8)), gb2)
    np.testing.assert_array_equal(h, np.tile(gb2, (7, 1)))


def _tiny_noisy(sigma):
    return synth.TINY.with_(router_noise=sigma)


def test_zero_noise_is_greedy():
    a = oracle.forward(synth.draw(_tiny_noisy(0.0)))
    b = oracle.forward(synth.draw(synth.TINY))
    np.testing.assert_array_equal(a.topk_idx, b.topk_idx)
    np.testing.assert_array_equal(a.y, b.y)
    assert a.L_aux == b.L_aux and a.L_z == b.L_z


def test_noise_enters_selection_softmax_and_lse():
    w = _tiny_noisy(0.7)
    inp = synth.draw(w)
    ref = oracle.forward(inp)
    clean = oracle.router_logits(synth.widen(inp.x, w.dtype), inp.W_g, inp.b_g)
    noisy = clean + 0.7 * inp.noise.astype(np.float64)
    np.testing.assert_allclose(ref.lse, special.logsumexp(noisy, axis=1), rtol=1e-13)
    for t in range(w.T):
        assert tuple(ref.topk_idx[t]) == oracle.brute_topk(noisy[t].tolist(), w.k)
    g = special.softmax(noisy, axis=1)
    sel = np.take_along_axis(g, ref.topk_idx, 1)
    np.testing.assert_allclose(ref.topk_gate, sel / sel.sum(1, keepdims=True), rtol=1e-13)


def test_large_noise_spreads_choices_uniformly():
    """With noise far above the logit scale every expert is picked k/E of the
    time; the counts pass a chi-square test of uniformity."""
    w = synth.DEFAULT.with_(T=4096, d=16, F=16, E=8, k=1, dtype="f32", router_noise=100.0, capacity_factor=None)
    ref = oracle.forward(synth.draw(w), tokens=[])
    counts = ref.disp.count
    assert stats.chisquare(counts).pvalue > 1e-4, counts


# ---------------------------------------------------------------------------
# Gate temperature [SER, gating path: the gate-forward call takes a
# temperature].  Reading: the gate's logits (after any noise) are divided by
# tau and replace the logits everywhere after; b_sel is added to the tempered
# logits for the selection.
# ---------------------------------------------------------------------------
def _hand_tempered(tau, b_sel=None, temperature=None):
    """The hand example of test_oracle_pins (T=2, d=3, E=3, k=2) with every
    router row multiplied by tau: at temperature tau its tempered logits are
    the hand example's logits (ln 3, 0, ln 2) and (0, ln 5, ln 5) exactly
    (division by a power of two is exact)."""
    import math
    L3, L5, L2 = math.log(3), math.log(5), math.log(2)
    x = np.array([[1.0, 0, 0], [0, 1.0, 0]])
    W_g = tau * np.array([[L3, 0, 0], [0, L5, 0], [L2, L5, 0]])
    w = synth.Workload(name="hand_tau", tag=0, T=2, d=3, E=3, k=2, F=3, act="relu", dtype="f32",
                       capacity_factor=None, credit=True,
                       temperature=tau if temperature is None else temperature)
    I = np.eye(3)
    return synth.Inputs(w, x, W_g, None, None if b_sel is None else np.asarray(b_sel, np.float64),
                        np.stack([I] * 3), np.zeros((3, 3)), np.stack([c * I for c in (1.0, 2.0, 3.0)]),
                        np.zeros((3, 3)))


def test_temperature_hand_example():
    """tau = 2 on doubled router rows gives the hand example's routing: P =
    (1/2, 1/6, 1/3) and (1/11, 5/11, 5/11), lse = ln 6 and ln 11, top-2 (0, 2)
    and (1, 2) (a tie at ln 5, lower index first), gates (3/5, 2/5) and
    (1/2, 1/2), L_z = beta ((ln 6)^2 + (ln 11)^2) / 2.  Without the division
    the same rows would give P proportional to (9, 1, 4): gates (9/13, 4/13)."""
    import math
    r = oracle.forward(_hand_tempered(2.0))
    np.testing.assert_allclose(r.logits, [[math.log(3), 0, math.log(2)], [0, math.log(5), math.log(5)]],
                               atol=0)
    np.testing.assert_allclose(r.P, [[1 / 2, 1 / 6, 1 / 3], [1 / 11, 5 / 11, 5 / 11]], atol=1e-15)
    np.testing.assert_allclose(r.lse, [math.log(6), math.log(11)], atol=1e-15)
    assert r.topk_idx.tolist() == [[0, 2], [1, 2]]
    np.testing.assert_allclose(r.topk_gate, [[3 / 5, 2 / 5], [1 / 2, 1 / 2]], atol=1e-15)
    assert abs(r.L_z - 1e-3 * (math.log(6) ** 2 + math.log(11) ** 2) / 2) < 1e-17
    untempered = oracle.forward(_hand_tempered(2.0, temperature=1.0))
    np.testing.assert_allclose(untempered.topk_gate[0], [9 / 13, 4 / 13], atol=1e-15)


def test_temperature_selection_bias_adds_to_tempered_logits():
    """Token 0 with b_sel = (0, 1, 0): tempered scores (ln 3, 1, ln 2) pick
    (0, 1); untempered scores (2 ln 3, 1, 2 ln 2) would pick (0, 2).  The gates
    are the tempered P = (1/2, 1/6, 1/3) renormalised over {0, 1}: (3/4, 1/4)."""
    r = oracle.forward(_hand_tempered(2.0, b_sel=[0.0, 1.0, 0.0]))
    assert r.topk_idx[0].tolist() == [0, 1]
    np.testing.assert_allclose(r.topk_gate[0], [3 / 4, 1 / 4], atol=1e-15)


def test_temperature_one_is_identity():
    a = oracle.forward(synth.draw(synth.TINY.with_(temperature=1.0)))
    b = oracle.forward(synth.draw(synth.TINY))
    np.testing.assert_array_equal(a.logits, b.logits)
    np.testing.assert_array_equal(a.y, b.y)


def test_temperature_keeps_selection_and_powers_gates():
    """Without selection bias or noise dividing by tau > 0 keeps the order of
    the logits, so the selected experts do not change, and each gate becomes
    the untempered gate to the power 1/tau, renormalised."""
    w = synth.DEFAULT.with_(T=200, d=32, F=16, E=12, k=3, dtype="f32", capacity_factor=None)
    base = oracle.forward(synth.draw(w), tokens=[])
    for tau in (0.25, 3.0):
        r = oracle.forward(synth.draw(w.with_(temperature=tau)), tokens=[])
        np.testing.assert_array_equal(r.topk_idx, base.topk_idx)
        p = base.topk_gate ** (1.0 / tau)
        np.testing.assert_allclose(r.topk_gate, p / p.sum(1, keepdims=True), rtol=1e-12)
        np.testing.assert_allclose(r.lse, special.logsumexp(base.logits / tau, axis=1), rtol=1e-13)


def test_temperature_after_noise_and_uniform_limit():
    """The noise is added before the division: lse = logsumexp((h + sigma n) /
    tau).  A very high temperature flattens the softmax: P -> 1/E, lse ->
    ln E, and the Switch loss -> alpha (the uniform-router closed form)."""
    w = _tiny_noisy(0.7).with_(temperature=3.0)
    inp = synth.draw(w)
    r = oracle.forward(inp)
    clean = oracle.router_logits(synth.widen(inp.x, w.dtype), inp.W_g, inp.b_g)
    z = (clean + 0.7 * inp.noise.astype(np.float64)) / 3.0
    np.testing.assert_allclose(r.lse, special.logsumexp(z, axis=1), rtol=1e-13)
    flat = oracle.forward(synth.draw(synth.TINY.with_(temperature=1e12)))
    np.testing.assert_allclose(flat.P, 1.0 / 4, rtol=1e-10)
    np.testing.assert_allclose(flat.lse, np.log(4.0), rtol=1e-10)
    assert abs(flat.L_aux - 0.01) < 1e-11


def test_temperature_must_be_positive():
    import pytest
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            oracle.tempered_logits(np.zeros((1, 2)), bad)
