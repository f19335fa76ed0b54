"""Second, independent oracle form: dense dispatch / combine tensors.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[Appendix C, Capacity & communication] defines the dispatch tensor D, which
scatters tokens into fixed-size expert buffers, and the combine tensor D~, the
gate-weighted un-scatter.  Here D in {0,1}^{T x E x C} is built from a
cumulative sum of the routing mask (no per-token counters as in the loop form)
and the layer output is y = D~ . E(D . x) with dense einsums.  Only for small
T * E * C.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np
from scipy import special

from .moe import activation


def dense_dispatch_combine(x: np.ndarray, idx: np.ndarray, g: np.ndarray, E: int,
                           C: Optional[int], experts: List[Tuple[np.ndarray, ...]], act: str):
    """Returns (y [T, d_out], D [T, E, C], count [E]).

    experts[e] = (W1 [F, d], b1 [F], W2 [d_out, F], b2 [d_out]) in float64.
    C = None means no cap (buffers of size T).
    """
    T, k = idx.shape
    M = np.zeros((T, E))
    G = np.zeros((T, E))
    np.put_along_axis(M, idx, 1.0, axis=1)
    np.put_along_axis(G, idx, g, axis=1)
    pos = np.cumsum(M, axis=0) - 1.0           # arrival rank of token t at expert e
    cap = T if C is None else C
    D = np.zeros((T, E, max(cap, 1)))
    tt, ee = np.nonzero((M > 0) & (pos < cap))
    D[tt, ee, pos[tt, ee].astype(np.int64)] = 1.0
    Dt = D * G[:, :, None]
    X = np.einsum("tec,td->ecd", D, x)          # expert buffers
    Y = np.stack([
        activation(act, X[e] @ W1.T + b1[None, :]) @ W2.T + b2[None, :]
        for e, (W1, b1, W2, b2) in enumerate(experts)
    ])
    y = np.einsum("tec,ecd->td", Dt, Y)
    return y, D, M.sum(axis=0).astype(np.int64)


def dense_softmax_mixture(x: np.ndarray, h: np.ndarray, experts: List[Tuple[np.ndarray, ...]],
                          act: str) -> np.ndarray:
    """y = sum_e softmax(h)_e E_e(x) over all experts: the dense softmax-gated
    mixture that top-k routing reduces to when k = E and nothing is dropped."""
    P = special.softmax(h, axis=1)
    y = 0.0
    for e, (W1, b1, W2, b2) in enumerate(experts):
        y = y + P[:, e:e + 1] * (activation(act, x @ W1.T + b1[None, :]) @ W2.T + b2[None, :])
    return y
