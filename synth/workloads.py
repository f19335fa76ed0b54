"""The five synthetic sparse-MoE layer workloads.

Each workload is a shape plus an initialisation recipe for the inputs of one
MoE sub-layer forward pass: tokens x, the linear router (W_g, optional router
bias b_g, optional selection-only bias b_sel) and E two-layer expert FFNs
(W1/b1 -> activation -> W2/b2), plus optional always-on shared experts.

Shapes and recipes follow the pages:
  * the tiny layer is the "Minimal example" of the SER walkthrough page
    (4 experts, 2 active, 8 -> 16 -> 8, seed 42);
  * the default layer is that page's "Configuration" block
    (8 experts, 2 active, 512 -> 1024 -> 512, load_balance_coef 0.01);
  * the other three widen the same layer along the axes the acronym appendix
    names: capacity factor and drops ("Capacity & communication"), fine-grained
    and shared experts ("Parameter accounting"), and the activation-weighted
    expert credit of the expert-credit diagram page, panel (b).

This module only describes inputs; it computes nothing of the layer.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from fractions import Fraction
from typing import Optional

SEED = 42

ACTS = ("relu", "gelu", "swish")


@dataclass(frozen=True)
class Workload:
    name: str
    tag: int                 # seeds the input streams together with SEED
    T: int                   # tokens in the batch
    d: int                   # model width (expert input and output width)
    E: int                   # routed experts
    k: int                   # experts per token
    F: int                   # expert hidden width
    act: str                 # "relu" | "gelu" | "swish"
    dtype: str               # "f32": everything fp32; "bf16": x and expert params bf16, router fp32
    capacity_factor: Optional[Fraction]   # None = dropless
    n_shared: int = 0        # always-on shared experts, each d -> F -> d
    alpha: float = 0.01      # Switch auxiliary-loss weight
    beta: float = 1e-3       # z-loss weight
    credit: bool = False     # also compute activation-weighted expert credit
    # router initialisation: "fan_in" = N(0, 1/d); "var:<v>" = N(0, v);
    # "unit_rows" = N(0, 1/d) rows rescaled to unit L2 norm (logit std 1)
    router_init: str = "fan_in"
    # router bias: None; "var:<v>" = N(0, v); "zipf:<s>" = calibrated Zipf popularity
    router_bias: Optional[str] = None
    # selection-only bias: None or "uniform:<a>" = U(-a, a)
    sel_bias: Optional[str] = None
    # noisy top-k: None (greedy) or the std sigma of the Gaussian noise added
    # to the router logits (the standard-normal draws are an input)
    router_noise: Optional[float] = None
    # router form: 0 = linear router W_g x + b_g; H > 0 = MLP gate of hidden
    # width H (its weights are inputs gW1 [H, d], gb1 [H], gW2 [E, H], gb2 [E])
    mlp_gate: int = 0
    # gate temperature tau > 0 (1 = none): the gate's logits are divided by it
    temperature: float = 1.0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def dropless(self) -> bool:
        return self.capacity_factor is None


TINY = Workload(
    name="tiny_fp32_T16_d8_E4_k2_F16_relu", tag=1,
    T=16, d=8, E=4, k=2, F=16, act="relu", dtype="f32",
    capacity_factor=Fraction(4), router_bias="var:0.01")

DEFAULT = Workload(
    name="default_bf16_T4096_d512_E8_k2_F1024_gelu", tag=2,
    T=4096, d=512, E=8, k=2, F=1024, act="gelu", dtype="bf16",
    capacity_factor=Fraction(5, 4), router_init="var:0.02")

SWITCH_ZIPF = Workload(
    name="switch_top1_zipf_bf16_T16384_d1024_E64_k1_F4096_relu", tag=3,
    T=16384, d=1024, E=64, k=1, F=4096, act="relu", dtype="bf16",
    capacity_factor=Fraction(1), router_bias="zipf:1.1")

FINE_SHARED = Workload(
    name="finegrained_shared2_bf16_T8192_d2048_E64_k6_F1408_swish", tag=4,
    T=8192, d=2048, E=64, k=6, F=1408, act="swish", dtype="bf16",
    capacity_factor=None, n_shared=2, sel_bias="uniform:0.1")

LARGE_CREDIT = Workload(
    name="large_credit_bf16_T32768_d4096_E128_k8_F1536_gelu", tag=5,
    T=32768, d=4096, E=128, k=8, F=1536, act="gelu", dtype="bf16",
    capacity_factor=None, credit=True, router_init="unit_rows")

ALL = (TINY, DEFAULT, SWITCH_ZIPF, FINE_SHARED, LARGE_CREDIT)
BY_NAME = {w.name: w for w in ALL}
