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
