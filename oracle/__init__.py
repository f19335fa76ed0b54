"""CPU oracle for the sparse-MoE sub-layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links anything under ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers or constant tables); the only
module both sides use is ``synth`` (seeded input draws, none of the layer's
arithmetic).

Everything is plain float64 NumPy on the stored input values (bf16 inputs are
widened exactly).  No intermediate rounding of the GPU path is mirrored here.

Sources, cited by page title and section:
  [Appendix C]  "Appendix C -- Acronyms & Symbols" (MoE lessons): sections
                "Core MoE symbols", "Parameter accounting", "Balancing",
                "Capacity & communication", "The two invariants, restated".
  [SER]         "Code Walkthrough -- SER (Sparse Expert Routing)": sections
                "Configuration", "The gating / routing path", "Load balancing",
                "Minimal example".
  [Credit]      "Sparse MoE Expert-Credit Loss Reweighting Diagram":
                "What the diagram shows", panels (b) and (c).

Parity status: every function here is pinned by a CPU test against a closed
form, an invariant, a textbook routine or brute force (tests/test_oracle_*.py).
"""
from .moe import (ACTIVATIONS, OracleResult, activation, capacity, combine, credit,
                  dispatch, expert_ffn, expert_rows, forward, gates, mlp_gate_logits, near_tie_gap, noisy_logits,
                  route_stats, router_logits, softmax_lse, tempered_logits, topk)
from .balance import (balance_losses, cv_squared, dro_update, expert_attributed_loss, importance,
                      selection_bias_update)
from .dense import dense_dispatch_combine, dense_softmax_mixture
from .brute import brute_topk

__all__ = [
    "ACTIVATIONS", "OracleResult", "activation", "capacity", "combine", "credit",
    "dispatch", "expert_ffn", "expert_rows", "forward", "gates", "near_tie_gap", "route_stats",
    "router_logits", "softmax_lse", "tempered_logits", "topk", "mlp_gate_logits", "noisy_logits", "dense_dispatch_combine",
    "dense_softmax_mixture", "brute_topk", "balance_losses", "cv_squared", "dro_update",
    "expert_attributed_loss", "importance", "selection_bias_update",
]
