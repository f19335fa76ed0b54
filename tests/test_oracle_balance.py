"""Pins of the balancing / reweighting oracle (oracle/balance.py) against hand
examples, closed forms, invariants and library routines."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy import stats

import oracle
import synth


# ---------------------------------------------------------------- expert-attributed loss
def test_expert_loss_hand_example():
    # 2 tokens, k = 2, E = 3: l_0 = 0.5*2/2, l_1 = 2*4/2, l_2 = (0.25*2 + 1*4)/2
    idx = np.array([[0, 2], [2, 1]])
    credit = np.array([[0.5, 0.25], [1.0, 2.0]])
    loss = np.array([2.0, 4.0])
    np.testing.assert_allclose(oracle.expert_attributed_loss(credit, idx, loss, 3), [0.5, 4.0, 2.25],
                               rtol=0, atol=1e-15)


def test_expert_loss_unit_losses_is_mean_credit():
    """With every per-token loss 1 the expert-attributed loss is the mean credit."""
    w = synth.TINY.with_(credit=True, capacity_factor=None)
    inp = synth.draw(w)
    ref = oracle.forward(inp)
    got = oracle.expert_attributed_loss(ref.credit, ref.topk_idx, np.ones(w.T), w.E)
    np.testing.assert_allclose(got, ref.mean_credit, rtol=1e-13, atol=1e-15)


def test_expert_loss_dropped_choice_contributes_nothing():
    idx = np.array([[0, 1]])
    credit = np.array([[0.0, 3.0]])          # choice 0 dropped: credit 0
    got = oracle.expert_attributed_loss(credit, idx, np.array([5.0]), 2)
    assert got[0] == 0.0 and got[1] == 15.0


@settings(max_examples=40, deadline=None)
@given(T=st.integers(1, 12), E=st.integers(2, 6), data=st.data())
def test_expert_loss_linear_in_losses(T, E, data):
    k = data.draw(st.integers(1, E))
    rng = np.random.default_rng(data.draw(st.integers(0, 10**6)))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    credit = rng.random((T, k))
    l1, l2 = rng.random(T), rng.random(T)
    a = oracle.expert_attributed_loss(credit, idx, 2.0 * l1 + 3.0 * l2, E)
    b = 2.0 * oracle.expert_attributed_loss(credit, idx, l1, E) + 3.0 * oracle.expert_attributed_loss(credit, idx, l2, E)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- EMA + DRO weights
def test_dro_hand_example():
    mu0 = np.full(3, 1 / 3)
    ema, mu, L = oracle.dro_update(np.array([1.0, 2.0, 3.0]), np.zeros(3), mu0, 0.5, 2.0)
    np.testing.assert_allclose(ema, [0.5, 1.0, 1.5])
    e = np.exp([0.0, 1.0, 2.0])                       # softmax(1/3 + 2 * ema) = softmax([1, 2, 3] + 1/3)
    np.testing.assert_allclose(mu, e / e.sum(), rtol=1e-14)
    assert abs(L - float((e / e.sum() * [1, 2, 3]).sum())) < 1e-14


def test_dro_two_experts_logistic():
    mu0, ema0, l = np.array([0.7, 0.3]), np.array([0.2, 0.9]), np.array([1.5, 0.5])
    ema, mu, _ = oracle.dro_update(l, ema0, mu0, 0.9, 0.3)
    z0 = mu0[0] + 0.3 * (0.9 * 0.2 + 0.1 * 1.5)
    z1 = mu0[1] + 0.3 * (0.9 * 0.9 + 0.1 * 0.5)
    assert abs(mu[0] - 1.0 / (1.0 + math.exp(z1 - z0))) < 1e-15


def test_dro_uniform_fixed_point_and_shift_invariance():
    E = 8
    rng = np.random.default_rng(3)
    l, ema0 = rng.random(E), rng.random(E)
    _, mu, _ = oracle.dro_update(l, ema0, np.full(E, 1 / E), 0.9, 0.0)
    np.testing.assert_allclose(mu, 1 / E, rtol=1e-14)                  # eta = 0 keeps uniform weights
    mu0 = rng.dirichlet(np.ones(E))
    e1, m1, L1 = oracle.dro_update(l, ema0, mu0, 0.8, 0.7)
    e2, m2, L2 = oracle.dro_update(l + 5.0, ema0 + 5.0, mu0, 0.8, 0.7)
    np.testing.assert_allclose(e2, e1 + 5.0, rtol=1e-14)
    np.testing.assert_allclose(m2, m1, rtol=1e-12)                      # softmax shift invariance
    assert abs(L2 - (L1 + 5.0)) < 1e-12 and abs(m1.sum() - 1) < 1e-15


def test_ema_closed_form():
    """n steps with a constant loss: lhat_n = l + decay^n (lhat_0 - l)."""
    l, ema, mu = np.array([2.0, -1.0]), np.array([0.5, 0.5]), np.array([0.5, 0.5])
    for _ in range(7):
        ema, mu, _ = oracle.dro_update(l, ema, mu, 0.75, 0.1)
    np.testing.assert_allclose(ema, l + 0.75 ** 7 * (np.array([0.5, 0.5]) - l), rtol=1e-14)


# ---------------------------------------------------------------- selection-bias update
def test_bias_update_hand_examples():
    b = np.array([0.1, -0.2, 0.0, 0.3])
    # E = 4, k = 1, T = 8: mean load 2
    np.testing.assert_allclose(oracle.selection_bias_update(b, np.array([4, 2, 1, 1]), 1, 8, 0.01),
                               b + 0.01 * np.array([-1, 0, 1, 1]), rtol=0, atol=1e-17)
    # E = 3, k = 2, T = 4: mean 8/3, never equal to an integer count
    np.testing.assert_allclose(oracle.selection_bias_update(np.zeros(3), np.array([4, 3, 1]), 2, 4, 0.5),
                               [-0.5, -0.5, 0.5])


def test_bias_update_balanced_is_identity():
    b = np.linspace(-1, 1, 16)
    np.testing.assert_array_equal(oracle.selection_bias_update(b, np.full(16, 6), 3, 32, 0.1), b)


# ---------------------------------------------------------------- CV / importance losses
def test_cv_squared_closed_forms_and_library():
    assert oracle.cv_squared(np.full(7, 3.0)) == 0.0
    assert oracle.cv_squared(np.zeros(5)) == 0.0
    for E in (2, 5, 64):
        v = np.zeros(E)
        v[0] = 11.0
        assert abs(oracle.cv_squared(v) - (E - 1)) < 1e-12                 # one expert takes everything
    rng = np.random.default_rng(9)
    v = rng.random(40) + 0.1
    assert abs(oracle.cv_squared(v) - stats.variation(v) ** 2) < 1e-13   # population coefficient of variation


def test_importance_sums_to_tokens_and_uniform_router():
    w = synth.DEFAULT.with_(T=64, d=16, F=16, E=8, k=2, dtype="f32")
    inp = synth.draw(w)
    ref = oracle.forward(inp, tokens=[])
    imp = oracle.importance(ref.topk_gate, ref.topk_idx, w.E)
    assert abs(imp.sum() - w.T) < 1e-12                                 # the gates of a token sum to 1
    # one-hot routing form
    onehot = np.zeros((w.T, w.E))
    for j in range(w.k):
        onehot[np.arange(w.T), ref.topk_idx[:, j]] += ref.topk_gate[:, j]
    np.testing.assert_allclose(imp, onehot.sum(0), rtol=1e-13)
    # uniform router: experts 0..k-1 take every token with gate 1/k
    inp.W_g = np.zeros_like(inp.W_g)
    inp.b_g = None
    u = oracle.forward(inp, tokens=[])
    imp_u, cv_load, cv_imp, z, aux = oracle.balance_losses(u.topk_gate, u.topk_idx, u.disp.count, u.lse,
                                                           w.E, 0.01, 1e-3)
    np.testing.assert_allclose(imp_u, [w.T / w.k] * w.k + [0] * (w.E - w.k), rtol=1e-14)
    assert abs(cv_load - (w.E / w.k - 1)) < 1e-12 and abs(cv_imp - (w.E / w.k - 1)) < 1e-12
    assert abs(z - math.log(w.E) ** 2) < 1e-12
    assert abs(aux - (0.01 * (w.E / w.k - 1) + 1e-3 * math.log(w.E) ** 2)) < 1e-12


def test_balance_losses_hand_example():
    """T = 2, E = 3, k = 2, unequal gates: the load and importance terms differ."""
    idx = np.array([[0, 1], [0, 2]])
    gate = np.array([[0.75, 0.25], [0.6, 0.4]])
    count = np.array([2, 1, 1])
    lse = np.array([1.0, 3.0])
    imp, cv_load, cv_imp, z, aux = oracle.balance_losses(gate, idx, count, lse, 3, 0.5, 0.25)
    np.testing.assert_allclose(imp, [1.35, 0.25, 0.4], rtol=1e-15)
    assert abs(cv_load - 0.125) < 1e-15                       # var (2/9) / mean^2 (16/9)
    m = 2.0 / 3.0
    want_imp = ((1.35 - m) ** 2 + (0.25 - m) ** 2 + (0.4 - m) ** 2) / 3 / (m * m)
    assert abs(cv_imp - want_imp) < 1e-14 and abs(cv_imp - 0.53375) < 1e-12
    assert z == 5.0                                           # (1 + 9) / 2
    assert abs(aux - (0.5 * 0.125 + 0.25 * 5.0)) < 1e-15
