"""Float64 CPU oracle of the routed-expert layer (test infrastructure only).

Importable by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py``; never by the library.
"""
from .moe_oracle import (  # noqa: F401
    bf16_to_f64, f16_to_f64, q3_fields, q3_pack, q3_dequant, expert_matrices,
    router_logits, route_topk, expert_histogram, permute, silu, expert_ffn, grouped_ffn,
    combine, moe_layer, dense_layer, rel_max_err,
)
