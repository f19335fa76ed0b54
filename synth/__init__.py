"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Holds the workload table and the input draws only; none of the MoE layer's
arithmetic lives here.
"""
from .workloads import (ALL, BY_NAME, DEFAULT, FINE_SHARED, LARGE_CREDIT, SEED,
                        SWITCH_ZIPF, TINY, Workload)
from .gen import Inputs, bf16_bits_to_f32, draw, f32_to_bf16_bits, token_losses, widen, zipf_router_bias

__all__ = [
    "ALL", "BY_NAME", "DEFAULT", "FINE_SHARED", "LARGE_CREDIT", "SEED", "SWITCH_ZIPF",
    "TINY", "Workload", "Inputs", "bf16_bits_to_f32", "draw", "f32_to_bf16_bits",
    "token_losses", "widen", "zipf_router_bias",
]
