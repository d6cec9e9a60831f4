"""CPU oracle for the routed SwiGLU MoE layer with ACE per-token expert-slot skipping.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything in this package.  The GPU library and its Python
binding never import it, and this package imports nothing of theirs.

What it follows: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based
LLMs" (picx.dev summary page): the SwiGLU expert equation and RMSNorm
factorisation (Theoretical Foundation), the GSP and RCR slot scores
(Methodology sections 1 and 2), conservative max-fusion and the top-1 rule
(Methodology section 3), and quantile-mapped thresholds (Efficiency Results,
Table 6), and the offline GSP and RCR tables (Methodology sections 1-2); and
the batch-level decode expert-pool cap of the ExFold listing page (abstract,
Tables 1, 5 and 6), without its folding.
It is written plainly: per-token loops, float64 arithmetic, each
function stating the passage it follows.

Pinning status of each function is listed in ``oracle/moe.py`` and
``oracle/thresholds.py`` headers.  Every function here is pinned by a
``-m "not gpu"`` test; none is "parity unpinned".
"""
from .moe import (rmsnorm, router_logits, topk_experts, topk_gates, skip_mask, silu, swiglu_expert,
                  dispatch_order, moe_layer, round_to_bf16, as_f64, store)
from .thresholds import slot_scores, quantile_thresholds
from .tables import gsp_raw, gsp_table, rcr_prototypes, rcr_raw, rcr_table, normalise
from .pool import pool_scores, expert_pool, cap_expert_pool

__all__ = ["rmsnorm", "router_logits", "topk_experts", "topk_gates", "skip_mask", "silu", "swiglu_expert",
           "dispatch_order", "moe_layer", "round_to_bf16", "as_f64", "store", "slot_scores", "quantile_thresholds",
           "gsp_raw", "gsp_table", "rcr_prototypes", "rcr_raw", "rcr_table", "normalise", "pool_scores",
           "expert_pool", "cap_expert_pool"]
