"""ORACLE: a plain, slow, CPU-only statement of what the routed-expert MoE layer computes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the ``expert_offload_cache_amd``
package and its HIP library) imports, links or calls anything here; only the
tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may.  It shares no code with the HIP path; both read inputs from
the ``synth`` generator module, which computes no step of the layer.

What is computed (the pages describe an offloaded-MoE runtime, not its
arithmetic; the layer form below is the plain reading, stated per function):

* route     -- router logits, top-k, renormalised softmax gates   (``route.py``)
* permute   -- tokens grouped by expert, stable within an expert  (``permute.py``)
* expert    -- SwiGLU expert FFN, float64, from exactly decoded weights (``ffn.py``)
* layer     -- gate-weighted combine (+ always-on shared expert)  (``layer.py``)
* lru       -- the slot cache shared by all layers: LRU simulator,
               brute-force LRU and a stack-distance recomputation (``lru.py``)

Precision: float64 everywhere except the router logits, which decide integer
results (the selected experts) and are therefore formed in binary32 in one
fixed summation order shared with the GPU router (``c/router_canon.c``).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library routines, special cases, invariants and brute
force on small inputs.
"""
from .numerics import bf16_to_f64, bf16_to_f32, dequant_int4, expert_to_f64
from .router import router_logits, topk_select, renorm_gates, route
from .permute import permute
from .ffn import swiglu_expert
from .layer import moe_layer, moe_layer_dense, moe_layer_tokens, layer_from_inputs
from .lru import LRUSim, BruteLRU, stack_distance_hits

__all__ = [
    "bf16_to_f64", "bf16_to_f32", "dequant_int4", "expert_to_f64", "router_logits", "topk_select",
    "renorm_gates", "route", "permute", "swiglu_expert", "moe_layer", "moe_layer_dense",
    "moe_layer_tokens", "layer_from_inputs", "LRUSim", "BruteLRU", "stack_distance_hits",
]
