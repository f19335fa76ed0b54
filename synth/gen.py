"""Seeded input draws for a Workload.

Every tensor comes from its own counter-free stream,
``numpy.random.Generator(PCG64(SeedSequence([seed, workload.tag, tensor_id, part])))``,
drawn in float32 and stored either as fp32 or as bf16 bit patterns (uint16,
round-to-nearest-even from the fp32 draw).  Large per-expert tensors use one
stream per expert (``part`` = expert index) so they can be drawn in parallel
and bit-identically regardless of thread count.

"N(0, v)" always means variance v (so N(0, 1/fan_in) has std 1/sqrt(fan_in)).

The one piece of numerics here is the Zipf router-bias calibration, which works
on a Gaussian model of the logits (never on the batch itself): see
``zipf_router_bias``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
from scipy import special

from .workloads import SEED, Workload

TENSOR_IDS = {
    "x": 0, "W_g": 1, "b_g": 2, "b_sel": 3,
    "W1": 4, "b1": 5, "W2": 6, "b2": 7,
    "sW1": 8, "sb1": 9, "sW2": 10, "sb2": 11,
    "token_loss": 12,
    "noise": 13, "gW1": 14, "gb1": 15, "gW2": 16, "gb2": 17,
}


def _rng(seed: int, tag: int, name: str, part: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, TENSOR_IDS[name], part])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    return ((u + (((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values as float64 (bf16 bit patterns are decoded first). Exact."""
    if dtype == "bf16" and a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


def _normal(rng: np.random.Generator, shape, var: float) -> np.ndarray:
    out = rng.standard_normal(shape, dtype=np.float32)
    out *= np.float32(np.sqrt(var))
    return out


def _parse(spec: str):
    kind, _, val = spec.partition(":")
    return kind, (float(val) if val else None)


def zipf_router_bias(row_std: np.ndarray, s: float, iters: int = 300, tol: float = 1e-10) -> np.ndarray:
    """Router bias b so that argmax_e(h_e + b_e) hits expert e with Zipf(s)
    probability p_e = (e+1)^-s / H, under the model h_e ~ N(0, row_std_e^2)
    independent across experts (x ~ N(0, I) makes h_e Gaussian with variance
    ||W_g[e]||^2; the small cross-expert correlations are ignored).

    P(argmax = e) = int phi_e(u) prod_{e' != e} Phi((u - b_e') / sd_e') du is
    evaluated by the trapezoid rule on a fixed grid and b is moved by damped
    fixed-point steps b += 0.5 (ln p - ln P).  The batch is never looked at.
    """
    E = row_std.shape[0]
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    sd = row_std.astype(np.float64)
    b = np.log(p) - np.log(p).mean()
    for _ in range(iters):
        u = np.linspace(b.min() - 9 * sd.max(), b.max() + 9 * sd.max(), 3001)
        z = (u[None, :] - b[:, None]) / sd[:, None]            # [E, U]
        logcdf = special.log_ndtr(z)
        total = logcdf.sum(axis=0)                              # log prod over all experts
        logpdf = -0.5 * z * z - 0.5 * np.log(2 * np.pi) - np.log(sd)[:, None]
        integrand = np.exp(logpdf + total[None, :] - logcdf)
        P = np.trapezoid(integrand, u, axis=1)
        P = np.maximum(P / P.sum(), 1e-300)
        step = 0.5 * (np.log(p) - np.log(P))
        b = b + step
        b -= b.mean()
        if np.abs(step).max() < tol:
            break
    return b


@dataclass
class Inputs:
    workload: Workload
    x: np.ndarray                    # [T, d]   fp32 or bf16 bits
    W_g: np.ndarray                  # [E, d]   fp32
    b_g: Optional[np.ndarray]        # [E]      fp32 or None
    b_sel: Optional[np.ndarray]      # [E]      fp32 or None (selection only)
    W1: np.ndarray                   # [E, F, d]
    b1: np.ndarray                   # [E, F]
    W2: np.ndarray                   # [E, d, F]
    b2: np.ndarray                   # [E, d]
    sW1: Optional[np.ndarray] = None  # [S, F, d] shared experts
    sb1: Optional[np.ndarray] = None  # [S, F]
    sW2: Optional[np.ndarray] = None  # [S, d, F]
    sb2: Optional[np.ndarray] = None  # [S, d]
    noise: Optional[np.ndarray] = None  # [T, E] fp32 standard-normal draws (noisy top-k)
    gW1: Optional[np.ndarray] = None    # [H, d] fp32 MLP gate
    gb1: Optional[np.ndarray] = None    # [H]
    gW2: Optional[np.ndarray] = None    # [E, H]
    gb2: Optional[np.ndarray] = None    # [E]
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def dtype(self) -> str:
        return self.workload.dtype


def _per_expert(seed, w, name, n, shape, var, dtype, threads):
    out = np.empty((n,) + tuple(shape), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(e):
        out[e] = _store(_normal(_rng(seed, w.tag, name, e), shape, var), dtype)

    if threads > 1 and n > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n)))
    else:
        for e in range(n):
            one(e)
    return out


def draw(w: Workload, seed: int = SEED, threads: Optional[int] = None) -> Inputs:
    """Draw all inputs of workload ``w``. Same (w, seed) -> same bits."""
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    T, d, E, F, dt = w.T, w.d, w.E, w.F, w.dtype

    x = _store(_normal(_rng(seed, w.tag, "x"), (T, d), 1.0), dt)

    kind, val = _parse(w.router_init)
    if kind == "fan_in":
        W_g = _normal(_rng(seed, w.tag, "W_g"), (E, d), 1.0 / d)
    elif kind == "var":
        W_g = _normal(_rng(seed, w.tag, "W_g"), (E, d), val)
    elif kind == "unit_rows":
        W_g = _normal(_rng(seed, w.tag, "W_g"), (E, d), 1.0 / d).astype(np.float64)
        W_g /= np.sqrt((W_g * W_g).sum(axis=1, keepdims=True))
        W_g = W_g.astype(np.float32)
    else:
        raise ValueError(w.router_init)

    b_g = None
    if w.router_bias is not None:
        kind, val = _parse(w.router_bias)
        if kind == "var":
            b_g = _normal(_rng(seed, w.tag, "b_g"), (E,), val)
        elif kind == "zipf":
            row_std = np.sqrt((W_g.astype(np.float64) ** 2).sum(axis=1))
            b_g = zipf_router_bias(row_std, val).astype(np.float32)
        else:
            raise ValueError(w.router_bias)

    b_sel = None
    if w.sel_bias is not None:
        kind, val = _parse(w.sel_bias)
        if kind != "uniform":
            raise ValueError(w.sel_bias)
        b_sel = _rng(seed, w.tag, "b_sel").uniform(-val, val, size=E).astype(np.float32)

    W1 = _per_expert(seed, w, "W1", E, (F, d), 1.0 / d, dt, threads)
    b1 = _store(_normal(_rng(seed, w.tag, "b1"), (E, F), 0.01), dt)
    W2 = _per_expert(seed, w, "W2", E, (d, F), 1.0 / F, dt, threads)
    b2 = _store(_normal(_rng(seed, w.tag, "b2"), (E, d), 0.01), dt)

    inp = Inputs(w, x, W_g.astype(np.float32), b_g, b_sel, W1, b1, W2, b2)
    S = w.n_shared
    if S:
        inp.sW1 = _per_expert(seed, w, "sW1", S, (F, d), 1.0 / d, dt, threads)
        inp.sb1 = _store(_normal(_rng(seed, w.tag, "sb1"), (S, F), 0.01), dt)
        inp.sW2 = _per_expert(seed, w, "sW2", S, (d, F), 1.0 / F, dt, threads)
        inp.sb2 = _store(_normal(_rng(seed, w.tag, "sb2"), (S, d), 0.01), dt)
    if w.router_noise is not None:
        inp.noise = _normal(_rng(seed, w.tag, "noise"), (T, E), 1.0)
    H = w.mlp_gate
    if H:
        inp.gW1 = _normal(_rng(seed, w.tag, "gW1"), (H, d), 1.0 / d)
        inp.gb1 = _normal(_rng(seed, w.tag, "gb1"), (H,), 0.01)
        inp.gW2 = _normal(_rng(seed, w.tag, "gW2"), (E, H), 1.0 / H)
        inp.gb2 = _normal(_rng(seed, w.tag, "gb2"), (E,), 0.01)
    return inp


def token_losses(w: Workload, seed: int = SEED) -> np.ndarray:
    """Synthetic per-token losses [T] float32 for the credit reweighting (no
    model exists to produce real ones): 1 + Exp(1), positive with mean 2, the
    scale of a language model's per-token cross-entropy."""
    rng = _rng(seed, w.tag, "token_loss")
    return (1.0 + rng.standard_exponential(w.T, dtype=np.float32)).astype(np.float32)
