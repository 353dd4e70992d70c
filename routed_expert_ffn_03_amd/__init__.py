"""MI355X-native routed-expert (MoE) layer: a C-ABI HIP library
(``libmoe_mi355x.so``) with a thin ctypes binding.

    moe_route_topk   top-k gate, gate weights, load histogram
    moe_router_topk  the router GEMM fused with the same top-k gate
    moe_permute      per-expert route lists
    moe_route_permute_plan  gate + route lists + FFN plan (one launch for
                     decode-sized batches)
    moe_grouped_ffn  every expert's SwiGLU FFN (MFMA tiles for busy experts,
                     HBM-streaming tiles for the rest)
    moe_combine      gate-weighted sum per token
"""
from .binding import (  # noqa: F401
    MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
    MOE_WFMT_BF16, MOE_WFMT_Q3G128, MOE_WFMT_BF16_PAIRS, DEFAULT_FAT_THRESHOLD, EXPORTS, MoEError, lib,
    moe_workspace_size, moe_route_topk, moe_router_topk, moe_permute, moe_grouped_ffn, moe_ffn_plan, moe_ffn_gate_up,
    moe_ffn_down, moe_combine, moe_grouped_ffn_noalloc, moe_route_permute_plan, moe_pack_bf16_pairs,
)
from .layer import MoELayerBuffers  # noqa: F401
