"""Python binding of the C ABI, one function per entry point, same names.

Argument marshalling only: tensors become device pointers plus the sizes read
from their shapes, and the stream is torch's current HIP stream unless given.
Every step of the layer runs in the HIP library; a non-zero status raises
``MoEError``.  torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._native import load

MOE_F32, MOE_BF16 = 0, 1
ACT = {"relu": 0, "gelu": 1, "swish": 2}
(OP_ROUTER, OP_DISPATCH, OP_FFN, OP_COMBINE, OP_STATS, OP_SHARED_FFN, OP_ROUTE, OP_BALANCE,
 OP_MLP_ROUTER) = range(9)


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().moe_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status} ({msg})")
        self.status = status


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MoEError(fn, rc)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _s(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(stream)


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    return _p(ws), ws.numel() * ws.element_size()


def moe_version() -> int:
    return load().moe_version()


def moe_capacity(cf_num: int, cf_den: int, k: int, T: int, E: int) -> int:
    out = ctypes.c_int64(0)
    _check("moe_capacity", load().moe_capacity(cf_num, cf_den, k, T, E, ctypes.byref(out)))
    return out.value


def moe_workspace_bytes(op: int, T: int = 0, d: int = 0, E: int = 1, k: int = 1, F: int = 1,
                        max_rows: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check("moe_workspace_bytes", load().moe_workspace_bytes(op, T, d, E, k, F, max_rows, ctypes.byref(out)))
    return out.value


def moe_router_topk(x, W_g, b_g, b_sel, k, logits, lse, topk_idx, topk_gate, ws=None, stream=None,
                    noise=None, noise_std=0.0, temperature=1.0):
    T, d = x.shape
    E = W_g.shape[0]
    wp, wn = _ws(ws)
    _check("moe_router_topk", load().moe_router_topk(
        _p(x), _dt(x), T, d, _p(W_g), _p(b_g), _p(b_sel), E, k, _p(noise), noise_std, temperature,
        _p(logits), _p(lse), _p(topk_idx), _p(topk_gate), wp, wn, _s(stream)))


def moe_mlp_router_topk(x, gW1, gb1, gW2, gb2, b_sel, k, logits, lse, topk_idx, topk_gate, ws, stream=None,
                        noise=None, noise_std=0.0, temperature=1.0):
    T, d = x.shape
    H = gW1.shape[0]
    E = gW2.shape[0]
    wp, wn = _ws(ws)
    _check("moe_mlp_router_topk", load().moe_mlp_router_topk(
        _p(x), _dt(x), T, d, _p(gW1), _p(gb1), H, _p(gW2), _p(gb2), _p(b_sel), E, k, _p(noise), noise_std,
        temperature, _p(logits), _p(lse), _p(topk_idx), _p(topk_gate), wp, wn, _s(stream)))


def moe_dispatch(topk_idx, E, capacity, x, expert_count, expert_offset, slot, row, row_token,
                 x_disp, ws, stream=None):
    T, k = topk_idx.shape
    d = x.shape[1] if x is not None else 0
    dt = _dt(x) if x is not None else MOE_BF16   # index-only dispatch: x and x_disp both None
    wp, wn = _ws(ws)
    _check("moe_dispatch", load().moe_dispatch(
        _p(topk_idx), T, k, E, capacity, _p(x), dt, d, _p(expert_count), _p(expert_offset),
        _p(slot), _p(row), _p(row_token), _p(x_disp), wp, wn, _s(stream)))


def moe_route(x, W_g, b_g, b_sel, k, capacity, alpha, beta, logits, lse, topk_idx, topk_gate,
              expert_count, expert_offset, slot, row, row_token, f, P, losses, ws, stream=None, noise=None,
              noise_std=0.0, temperature=1.0):
    T, d = x.shape
    E = W_g.shape[0]
    wp, wn = _ws(ws)
    _check("moe_route", load().moe_route(
        _p(x), _dt(x), T, d, _p(W_g), _p(b_g), _p(b_sel), E, k, _p(noise), noise_std, temperature, capacity,
        alpha, beta,
        _p(logits),
        _p(lse), _p(topk_idx), _p(topk_gate), _p(expert_count), _p(expert_offset), _p(slot), _p(row),
        _p(row_token), _p(f), _p(P), _p(losses), wp, wn, _s(stream)))


def moe_route_noalloc(x, W_g, b_g, b_sel, k, capacity, alpha, beta, logits, lse, topk_idx, topk_gate,
                      expert_count, expert_offset, slot, row, row_token, f, P, losses, stream=None, noise=None,
                      noise_std=0.0, temperature=1.0):
    """moe_route with its scratch in the library's static device array (no workspace)."""
    T, d = x.shape
    E = W_g.shape[0]
    _check("moe_route_noalloc", load().moe_route_noalloc(
        _p(x), _dt(x), T, d, _p(W_g), _p(b_g), _p(b_sel), E, k, _p(noise), noise_std, temperature, capacity,
        alpha, beta, _p(logits), _p(lse), _p(topk_idx), _p(topk_gate), _p(expert_count), _p(expert_offset),
        _p(slot), _p(row), _p(row_token), _p(f), _p(P), _p(losses), _s(stream)))


def moe_grouped_ffn(a, group_offset, max_rows, W1, b1, W2, b2, act, hidden, out,
                    hidden_sqnorm=None, ws=None, a_rows=None, stream=None):
    G, F, d = W1.shape
    d_out = W2.shape[1]
    wp, wn = _ws(ws)
    _check("moe_grouped_ffn", load().moe_grouped_ffn(
        _p(a), _p(a_rows), _p(group_offset), G, max_rows, d, F, d_out, _dt(a),
        ACT[act] if isinstance(act, str) else act, _p(W1), _p(b1), _p(W2), _p(b2), _p(hidden), _p(out),
        _p(hidden_sqnorm), wp, wn, _s(stream)))


def moe_expert_up(a, group_offset, max_rows, W1, b1, act, hidden, hidden_sqnorm=None, ws=None,
                  a_rows=None, stream=None):
    G, F, d = W1.shape
    wp, wn = _ws(ws)
    _check("moe_expert_up", load().moe_expert_up(
        _p(a), _p(a_rows), _p(group_offset), G, max_rows, d, F, _dt(a),
        ACT[act] if isinstance(act, str) else act, _p(W1), _p(b1), _p(hidden), _p(hidden_sqnorm), wp, wn,
        _s(stream)))


def moe_expert_down(hidden, group_offset, max_rows, W2, b2, out, stream=None):
    G, d_out, F = W2.shape
    _check("moe_expert_down", load().moe_expert_down(
        _p(hidden), _p(group_offset), G, max_rows, F, d_out, _dt(hidden), _p(W2), _p(b2), _p(out),
        _s(stream)))


def moe_shared_ffn(x, W1, b1, W2, b2, act, hidden, out, stream=None):
    T, d = x.shape
    S, F, _ = W1.shape
    d_out = W2.shape[1]
    _check("moe_shared_ffn", load().moe_shared_ffn(
        _p(x), T, d, F, S, d_out, _dt(x), ACT[act] if isinstance(act, str) else act, _p(W1), _p(b1),
        _p(W2), _p(b2), _p(hidden), _p(out), _s(stream)))


def moe_combine(expert_out, row, topk_gate, shared_out, y, stream=None):
    T, k = row.shape
    d_out = y.shape[1]
    _check("moe_combine", load().moe_combine(
        _p(expert_out), _p(row), _p(topk_gate), _p(shared_out), T, k, d_out, _dt(y), _p(y),
        _s(stream)))


def moe_route_stats(logits, lse, topk_idx, topk_gate, expert_count, alpha, beta, f, P, losses,
                    hidden_sqnorm=None, row=None, expert_offset=None, row_token=None, credit=None,
                    mean_credit=None, ws=None, stream=None, token_loss=None, expert_loss=None):
    T, E = logits.shape
    k = topk_idx.shape[1]
    wp, wn = _ws(ws)
    _check("moe_route_stats", load().moe_route_stats(
        _p(logits), _p(lse), _p(topk_idx), _p(topk_gate), _p(expert_count), T, E, k, alpha, beta,
        _p(f), _p(P), _p(losses), _p(hidden_sqnorm), _p(row), _p(expert_offset), _p(row_token),
        _p(credit), _p(mean_credit), _p(token_loss), _p(expert_loss), wp, wn, _s(stream)))


def moe_balance_losses(topk_gate, topk_idx, expert_count, lse, load_balance_coef, z_loss_coef, importance,
                       out, ws, stream=None):
    T, k = topk_idx.shape
    E = expert_count.shape[0]
    wp, wn = _ws(ws)
    _check("moe_balance_losses", load().moe_balance_losses(
        _p(topk_gate), _p(topk_idx), _p(expert_count), _p(lse), T, E, k, load_balance_coef, z_loss_coef,
        _p(importance), _p(out), wp, wn, _s(stream)))


def moe_selection_bias_update(expert_count, k, T, gamma, b_sel, stream=None):
    _check("moe_selection_bias_update", load().moe_selection_bias_update(
        _p(expert_count), expert_count.shape[0], k, T, gamma, _p(b_sel), _s(stream)))


def moe_dro_update(expert_loss, ema_decay, eta, ema, mu, dro_loss, stream=None):
    _check("moe_dro_update", load().moe_dro_update(
        _p(expert_loss), expert_loss.shape[0], ema_decay, eta, _p(ema), _p(mu), _p(dro_loss), _s(stream)))


# measurement support (include/moe_calib.h): not part of the layer
def moe_calib_copy(src, dst, nbytes, stream=None):
    _check("moe_calib_copy", load().moe_calib_copy(_p(src), _p(dst), nbytes, _s(stream)))


def moe_calib_read(src, nbytes, sink, stream=None):
    _check("moe_calib_read", load().moe_calib_read(_p(src), nbytes, _p(sink), _s(stream)))


def moe_calib_mfma(blocks, iters, sink, stream=None) -> float:
    """Enqueue the MFMA loop; returns the dense bf16 flops it performs."""
    fl = ctypes.c_double(0)
    _check("moe_calib_mfma", load().moe_calib_mfma(blocks, iters, _p(sink), ctypes.byref(fl), _s(stream)))
    return fl.value
