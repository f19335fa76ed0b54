"""One sparse-MoE sub-layer forward pass as a sequence of C-ABI calls.

    router_topk -> dispatch -> expert_up -> expert_down (-> shared_ffn) -> combine -> route_stats

This is the forward entry of page "Code Walkthrough -- SER" (the layer's
forward runs gate, route, the selected experts and the gate-weighted combine),
with the statistics of page "Appendix C -- Acronyms & Symbols" (Balancing) and
the credit of the expert-credit diagram page, panel (b).  Python only
allocates buffers (torch) and passes pointers; every step runs in HIP.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from typing import Optional, Tuple

import torch

from . import api


@dataclass
class MoEOutputs:
    T: int
    capacity: int               # -1 = no cap
    max_rows: int
    logits: torch.Tensor        # [T, E] fp32
    lse: torch.Tensor           # [T] fp32
    topk_idx: torch.Tensor      # [T, k] int32
    topk_gate: torch.Tensor     # [T, k] fp32
    expert_count: torch.Tensor  # [E] int32
    expert_offset: torch.Tensor  # [E+1] int32
    slot: torch.Tensor          # [T, k] int32
    row: torch.Tensor           # [T, k] int32
    row_token: torch.Tensor     # [rows] int32
    x_disp: Optional[torch.Tensor]  # [rows, d]; None when rows are gathered in the up pass
    hidden: torch.Tensor        # [rows, F]
    y_disp: torch.Tensor        # [rows, d]
    sqnorm: Optional[torch.Tensor]
    shared_hidden: Optional[torch.Tensor]
    shared_out: Optional[torch.Tensor]
    y: torch.Tensor             # [T, d]
    f: torch.Tensor             # [E]
    P: torch.Tensor             # [E]
    losses: torch.Tensor        # [3] = L_aux, L_z, sum
    credit: Optional[torch.Tensor]
    mean_credit: Optional[torch.Tensor]
    ws_router: torch.Tensor
    ws_dispatch: torch.Tensor
    ws_ffn: Optional[torch.Tensor]
    ws_stats: torch.Tensor
    ws_route: Optional[torch.Tensor] = None
    x: Optional[torch.Tensor] = None  # input of the last dispatch (rows gathered from it)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


class MoELayer:
    """Parameters on the device plus the calls of one forward pass.

    W_g [E, d] fp32, b_g / b_sel [E] fp32 or None; W1 [E, F, d], b1 [E, F],
    W2 [E, d, F], b2 [E, d] in the layer dtype (bf16 or fp32); shared =
    (W1 [S, F, d], b1 [S, F], W2 [S, d, F], b2 [S, d]) or None.
    capacity_factor: a Fraction (or anything Fraction accepts), None = no cap.
    gather_rows: True (default) dispatches indices only and the expert-up pass
    reads token rows of x through row_token; False materialises x_disp first.
    fused_route: True (default, with gather_rows) takes router, dispatch and
    statistics in one moe_route call; False makes the three calls separately.
    noise, noise_std: noisy top-k, noise [T, E] fp32 standard-normal draws.
    temperature: gate temperature tau > 0 dividing the (noisy) logits (1 = none).
    mlp_gate: (gW1 [H, d], gb1 [H], gW2 [E, H], gb2 [E]) fp32 to route with the
    MLP gate instead of W_g / b_g (always the separate calls).
    overlap_shared: run the shared experts on a side stream, forked after the
    routing pass, concurrently with the expert passes (forward only; calls()
    lists every call in order).
    overlap_stats: run the statistics call (with credit, or after the separate
    router and dispatch calls) on a second side stream beside the down pass
    and the combine (forward only).  Off by default: the persistent down-pass
    GEMM holds every CU, so the statistics kernels wait for its tail anyway,
    and the fork and join cost more than they hide (large workload step
    6742-6756 us on the main stream, 6761-6771 us on the side stream).
    """

    def __init__(self, W_g, W1, b1, W2, b2, *, k: int, act: str, capacity_factor=None,
                 b_g=None, b_sel=None, shared: Optional[Tuple[torch.Tensor, ...]] = None,
                 alpha: float = 0.01, beta: float = 1e-3, credit: bool = False,
                 gather_rows: bool = True, fused_route: bool = True, noise=None, noise_std: float = 0.0,
                 temperature: float = 1.0, mlp_gate: Optional[Tuple[torch.Tensor, ...]] = None, overlap_shared: bool = True,
                 overlap_stats: bool = False):
        self.W_g, self.b_g, self.b_sel = W_g, b_g, b_sel
        self.W1, self.b1, self.W2, self.b2 = W1, b1, W2, b2
        self.shared = shared
        self.k, self.act = k, act
        self.cf = None if capacity_factor is None else Fraction(capacity_factor)
        self.alpha, self.beta, self.credit = alpha, beta, credit
        self.gather_rows = gather_rows
        self.noise, self.noise_std = noise, float(noise_std)
        self.temperature = float(temperature)
        self.overlap_shared = overlap_shared
        self.overlap_stats = overlap_stats
        self._side = None
        self._side_stats = None
        self.mlp_gate = mlp_gate
        self.fused = fused_route and gather_rows and mlp_gate is None
        self.E, self.F, self.d = W1.shape
        self.dtype = W1.dtype
        self.device = W1.device

    def capacity(self, T: int) -> int:
        if self.cf is None:
            return -1
        return api.moe_capacity(self.cf.numerator, self.cf.denominator, self.k, T, self.E)

    def allocate(self, T: int) -> MoEOutputs:
        E, k, d, F, dev, dt = self.E, self.k, self.d, self.F, self.device, self.dtype
        C = self.capacity(T)
        max_rows = T * k if C < 0 else min(T * k, E * C)
        rows = max(max_rows, 1)
        i32, f32 = torch.int32, torch.float32
        e = lambda *s, dtype=dt: torch.empty(*s, dtype=dtype, device=dev)
        S = 0 if self.shared is None else self.shared[0].shape[0]
        return MoEOutputs(
            T=T, capacity=C, max_rows=max_rows,
            logits=e(T, E, dtype=f32), lse=e(T, dtype=f32),
            topk_idx=e(T, k, dtype=i32), topk_gate=e(T, k, dtype=f32),
            expert_count=e(E, dtype=i32), expert_offset=e(E + 1, dtype=i32),
            slot=e(T, k, dtype=i32), row=e(T, k, dtype=i32), row_token=e(rows, dtype=i32),
            x_disp=None if self.gather_rows else e(rows, d), hidden=e(rows, F), y_disp=e(rows, d),
            sqnorm=e(rows, dtype=f32) if self.credit else None,
            shared_hidden=e(T, S * F) if S else None, shared_out=e(T, d) if S else None,
            y=e(T, d), f=e(E, dtype=f32), P=e(E, dtype=f32), losses=e(3, dtype=f32),
            credit=e(T, k, dtype=f32) if self.credit else None,
            mean_credit=e(E, dtype=f32) if self.credit else None,
            ws_router=_ws(api.moe_workspace_bytes(api.OP_MLP_ROUTER, T=T, F=self.mlp_gate[0].shape[0])
                          if self.mlp_gate is not None else api.moe_workspace_bytes(api.OP_ROUTER, T=T, d=d, E=E),
                          dev),
            ws_dispatch=_ws(api.moe_workspace_bytes(api.OP_DISPATCH, T=T, E=E), dev),
            ws_ffn=_ws(api.moe_workspace_bytes(api.OP_FFN, F=F, max_rows=rows), dev) if self.credit else None,
            ws_stats=_ws(api.moe_workspace_bytes(api.OP_STATS, T=T, E=E, k=k), dev),
            ws_route=_ws(api.moe_workspace_bytes(api.OP_ROUTE, T=T, d=d, E=E), dev) if self.fused else None,
        )

    def forward(self, x: torch.Tensor, out: Optional[MoEOutputs] = None, stream=None) -> MoEOutputs:
        T = x.shape[0]
        o = self.allocate(T) if out is None else out
        if o.T != T:
            raise ValueError("output buffers were allocated for another batch size")
        calls = self.calls(x, o, stream)
        names = [n for n, _ in calls]
        side_shared = self.shared is not None and self.overlap_shared
        side_stats = self.overlap_stats and "stats" in names and "expert_up" in names
        if not side_shared and not side_stats:
            for _, call in calls:
                call()
            return o
        main = torch.cuda.current_stream(self.device) if stream is None else stream
        joins = []
        shared_done = None
        for name, call in calls:
            if name == "shared" and side_shared:
                continue
            if name == "combine" and side_shared:
                main.wait_event(shared_done)
            if name == "stats" and side_stats:
                continue
            call()
            if name in ("route", "dispatch") and side_shared:
                # The shared experts need only x: they run on a side stream
                # beside the expert passes, and the combine waits for them.
                # Forked after the routing pass rather than before it, so the
                # router (fewer blocks than CUs on small batches) is not kept
                # waiting behind a GEMM that holds every CU (measured on the
                # 64-expert fine-grained layer: step 941 -> 926 us).
                side = self._side_stream()
                fork = torch.cuda.Event()
                fork.record(main)
                side.wait_event(fork)
                self.shared_experts(x, o, side)
                shared_done = torch.cuda.Event()
                shared_done.record(side)
            if name == "expert_up" and side_stats:
                # The statistics (with credit) need the routing outputs and the
                # up pass's ||a||^2 only, and nothing after them reads what they
                # write: they run on a second side stream beside the down pass
                # and the combine, and the pass ends when both are done.
                side2 = self._stats_stream()
                fork2 = torch.cuda.Event()
                fork2.record(main)
                side2.wait_event(fork2)
                self.stats(o, side2)
                stats_done = torch.cuda.Event()
                stats_done.record(side2)
                joins.append(stats_done)
        for ev in joins:
            main.wait_event(ev)
        return o

    def _side_stream(self):
        if self._side is None:
            self._side = torch.cuda.Stream(self.device)   # default priority
        return self._side

    def _stats_stream(self):
        if self._side_stats is None:
            self._side_stats = torch.cuda.Stream(self.device)   # default priority
        return self._side_stats

    def calls(self, x, o: MoEOutputs, stream=None):
        """The ABI calls of one forward pass, in order, as (name, thunk) pairs."""
        c = []
        if self.fused:
            c.append(("route", lambda: self.route(x, o, stream)))
        else:
            c.append(("router", lambda: self.router(x, o, stream)))
            c.append(("dispatch", lambda: self.dispatch(x, o, stream)))
        c.append(("expert_up", lambda: self.expert_up(o, stream)))
        c.append(("expert_down", lambda: self.expert_down(o, stream)))
        if self.shared is not None:
            c.append(("shared", lambda: self.shared_experts(x, o, stream)))
        c.append(("combine", lambda: self.combine(o, stream)))
        if not self.fused or self.credit:
            c.append(("stats", lambda: self.stats(o, stream)))
        return c

    # one method per C-ABI call, in forward order
    def route(self, x, o: MoEOutputs, stream=None) -> None:
        o.x = x
        api.moe_route(x, self.W_g, self.b_g, self.b_sel, self.k, o.capacity, self.alpha, self.beta,
                      o.logits, o.lse, o.topk_idx, o.topk_gate, o.expert_count, o.expert_offset, o.slot,
                      o.row, o.row_token, o.f, o.P, o.losses, o.ws_route, stream, noise=self.noise,
                      noise_std=self.noise_std, temperature=self.temperature)

    def router(self, x, o: MoEOutputs, stream=None) -> None:
        if self.mlp_gate is not None:
            gW1, gb1, gW2, gb2 = self.mlp_gate
            api.moe_mlp_router_topk(x, gW1, gb1, gW2, gb2, self.b_sel, self.k, o.logits, o.lse, o.topk_idx,
                                    o.topk_gate, o.ws_router, stream, noise=self.noise, noise_std=self.noise_std,
                                    temperature=self.temperature)
            return
        api.moe_router_topk(x, self.W_g, self.b_g, self.b_sel, self.k, o.logits, o.lse, o.topk_idx,
                            o.topk_gate, o.ws_router, stream, noise=self.noise, noise_std=self.noise_std,
                            temperature=self.temperature)

    def dispatch(self, x, o: MoEOutputs, stream=None) -> None:
        o.x = x
        api.moe_dispatch(o.topk_idx, self.E, o.capacity, None if self.gather_rows else x, o.expert_count,
                         o.expert_offset, o.slot, o.row, o.row_token, o.x_disp, o.ws_dispatch, stream)

    def expert_up(self, o: MoEOutputs, stream=None) -> None:
        if o.max_rows > 0:
            if self.gather_rows:
                api.moe_expert_up(o.x, o.expert_offset, o.max_rows, self.W1, self.b1, self.act, o.hidden,
                                  o.sqnorm, o.ws_ffn, a_rows=o.row_token, stream=stream)
            else:
                api.moe_expert_up(o.x_disp, o.expert_offset, o.max_rows, self.W1, self.b1, self.act,
                                  o.hidden, o.sqnorm, o.ws_ffn, stream=stream)

    def expert_down(self, o: MoEOutputs, stream=None) -> None:
        if o.max_rows > 0:
            api.moe_expert_down(o.hidden, o.expert_offset, o.max_rows, self.W2, self.b2, o.y_disp, stream)

    def shared_experts(self, x, o: MoEOutputs, stream=None) -> None:
        if self.shared is not None:
            sW1, sb1, sW2, sb2 = self.shared
            api.moe_shared_ffn(x, sW1, sb1, sW2, sb2, self.act, o.shared_hidden, o.shared_out, stream)

    def combine(self, o: MoEOutputs, stream=None) -> None:
        api.moe_combine(o.y_disp, o.row, o.topk_gate, o.shared_out, o.y, stream)

    def stats(self, o: MoEOutputs, stream=None) -> None:
        # after the fused routing call f, P and the losses are already there:
        # only the credit is asked for
        fpl = (None, None, None) if self.fused else (o.f, o.P, o.losses)
        api.moe_route_stats(o.logits, o.lse, o.topk_idx, o.topk_gate, o.expert_count, self.alpha,
                            self.beta, *fpl, o.sqnorm, o.row, o.expert_offset,
                            o.row_token, o.credit, o.mean_credit, o.ws_stats, stream)
