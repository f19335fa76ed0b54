"""Float64 oracle of the balancing and reweighting statistics around the layer.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

  1. expert-attributed loss  l_i = (1/N) sum_j c_i(x_j) l_j 1[i in T_k(x_j)]
                                         [Credit, panel (b)]
  2. EMA tracker and layer-wise DRO weights
        lhat_i <- b lhat_i + (1 - b) l_i ;  mu <- softmax(mu + eta lhat) ;
        L_DRO = sum_i mu_i l_i           [Credit, panel (c)]
  3. aux-loss-free selection-bias update with rate gamma
                                         [Appendix C, Balancing: b_i, gamma]
  4. coefficient-of-variation balance and importance losses and their
     weighted combination with the z-loss
                                         [SER, Load balancing: load_balance,
                                          importance and aux losses]

Readings (the pages name these quantities without printing every formula):
  * 1: c is the activation-weighted credit of panel (b) (renormalised gate
    times the norm of the expert's hidden activation; 0 for a dropped
    choice), N = T, and l_j is a per-token loss supplied by the caller (no
    model exists here, so the tests draw synthetic ones).
  * 2: the printed update is taken literally: the softmax is applied to
    mu + eta lhat with mu the current weights (not log mu), the EMA is
    updated first, then mu, and L_DRO uses the updated mu with the step's
    l_i.  The stop-gradients are the identity in a forward pass.
  * 3: the plainest rule the symbols support: every expert whose load is
    below the mean load moves its bias up by gamma, above the mean down by
    gamma, equal: unchanged, i.e. b_i <- b_i + gamma sign(mean - load_i),
    with load_i the pre-capacity count and mean = k T / E.
  * 4: CV(v)^2 = var(v) / mean(v)^2 with the population variance (0 when the
    mean is 0); load_i = pre-capacity count_i; importance_i = the sum over the
    batch of the renormalised gates routed to i; the combination is
    load_balance_coef * CV(load)^2 + z_loss_coef * mean_t lse_t^2.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np


def expert_attributed_loss(credit: np.ndarray, idx: np.ndarray, token_loss: np.ndarray,
                           E: int) -> np.ndarray:
    """l_i = (1/N) sum_j c_{j,i} l_j over the choices (j, i) of the batch.

    credit [T, k] (0 for dropped choices), idx [T, k], token_loss [T].
    [Credit, panel (b)]
    """
    T, k = idx.shape
    out = np.zeros(E)
    for t in range(T):
        for j in range(k):
            out[int(idx[t, j])] += float(credit[t, j]) * float(token_loss[t])
    return out / T


def dro_update(expert_loss: np.ndarray, ema: np.ndarray, mu: np.ndarray, decay: float,
               eta: float) -> Tuple[np.ndarray, np.ndarray, float]:
    """One step of the EMA tracker and the DRO weights, and the DRO objective.

    lhat <- decay lhat + (1 - decay) l;  mu <- softmax(mu + eta lhat);
    L_DRO = sum_i mu_i l_i.   [Credit, panel (c)]
    """
    ema_new = decay * np.asarray(ema, np.float64) + (1.0 - decay) * np.asarray(expert_loss, np.float64)
    z = np.asarray(mu, np.float64) + eta * ema_new
    w = np.exp(z - z.max())
    mu_new = w / w.sum()
    return ema_new, mu_new, float((mu_new * expert_loss).sum())


def selection_bias_update(b_sel: np.ndarray, count: np.ndarray, k: int, T: int,
                          gamma: float) -> np.ndarray:
    """b_i <- b_i + gamma sign(k T / E - count_i), the sign taken exactly.

    [Appendix C, Balancing: per-expert selection bias b_i, update rate gamma]
    """
    E = len(count)
    out = np.asarray(b_sel, np.float64).copy()
    for i in range(E):
        diff = k * T - E * int(count[i])          # E (mean - count_i), an exact integer
        out[i] += gamma * (1 if diff > 0 else -1 if diff < 0 else 0)
    return out


def importance(gate: np.ndarray, idx: np.ndarray, E: int) -> np.ndarray:
    """importance_i = sum over the batch of the gates routed to expert i."""
    out = np.zeros(E)
    T, k = idx.shape
    for t in range(T):
        for j in range(k):
            out[int(idx[t, j])] += float(gate[t, j])
    return out


def cv_squared(v: np.ndarray) -> float:
    """CV(v)^2 = population variance / mean^2 (0 when the mean is 0)."""
    v = np.asarray(v, np.float64)
    m = float(v.mean())
    if m == 0.0:
        return 0.0
    return float(((v - m) ** 2).mean()) / (m * m)


def balance_losses(gate: np.ndarray, idx: np.ndarray, count: np.ndarray, lse: np.ndarray, E: int,
                   load_balance_coef: float, z_loss_coef: float):
    """(importance [E], CV(load)^2, CV(importance)^2, mean lse^2, combined aux loss).

    [SER, Load balancing: coefficient-of-variation balance, importance balance,
    z-loss, and aux_loss = load_balance_coef * load_balance + z_loss_coef * z_loss]
    """
    imp = importance(gate, idx, E)
    cv_load = cv_squared(count)
    cv_imp = cv_squared(imp)
    z = float(math.fsum(float(l) * float(l) for l in lse)) / len(lse)
    return imp, cv_load, cv_imp, z, load_balance_coef * cv_load + z_loss_coef * z
