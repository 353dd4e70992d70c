"""One routed-expert layer call on caller-owned buffers: the C entry points
in order on one stream.  Buffers are allocated once per shape with
torch (device memory only); the call itself allocates nothing.
"""
from __future__ import annotations

import torch

from . import binding as B


class MoELayerBuffers:
    """Outputs, intermediates and workspace of one layer shape."""

    def __init__(self, T: int, E: int, k: int, H: int, I: int, wfmt: int = B.MOE_WFMT_BF16,
                 device: str | torch.device = "cuda"):
        self.T, self.E, self.k, self.H, self.I, self.wfmt = T, E, k, H, I, wfmt
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_ids = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.expert_counts = torch.empty((E,), **i32)
        self.expert_offsets = torch.empty((E + 1,), **i32)
        self.sorted_pair = torch.empty((T * k,), **i32)
        self.pair_to_sorted = torch.empty((T * k,), **i32)
        self.y_sorted = torch.empty((T * k, H), dtype=torch.float16, device=device)
        self.out = torch.empty((T, H), dtype=torch.float32, device=device)
        ws = B.moe_workspace_size(T, E, k, H, I, wfmt)
        if ws == 0:
            raise ValueError("unsupported layer shape")
        self.workspace = torch.empty((ws,), dtype=torch.uint8, device=device)

    def forward(self, logits: torch.Tensor, x: torch.Tensor, w: dict, fat_threshold: int = B.DEFAULT_FAT_THRESHOLD,
                stream=None) -> torch.Tensor:
        """route -> permute -> grouped FFN -> combine; returns ``out`` (fp32 [T, H]).

        Decode-sized batches (T <= 64) run route, permute and the FFN plan as
        one launch (moe_route_permute_plan); the results are the same."""
        if self.T <= 64:
            B.moe_route_permute_plan(logits, self.k, self.H, self.I, self.topk_ids, self.topk_w, self.expert_counts,
                                     self.expert_offsets, self.sorted_pair, self.pair_to_sorted, self.workspace,
                                     fat_threshold=fat_threshold, wfmt=self.wfmt, stream=stream)
            B.moe_ffn_gate_up(x, w["gate"], w["up"], self.sorted_pair, self.E, self.k, self.workspace,
                              s_gate=w.get("gate_scale"), s_up=w.get("up_scale"), fat_threshold=fat_threshold,
                              wfmt=self.wfmt, stream=stream)
            B.moe_ffn_down(w["down"], self.T, self.E, self.k, self.I, self.y_sorted, self.workspace,
                           s_down=w.get("down_scale"), fat_threshold=fat_threshold, wfmt=self.wfmt, stream=stream)
        else:
            B.moe_route_topk(logits, self.k, self.topk_ids, self.topk_w, self.expert_counts, stream)
            B.moe_permute(self.topk_ids, self.E, self.expert_offsets, self.sorted_pair, self.pair_to_sorted,
                          self.workspace, stream)
            B.moe_grouped_ffn(x, w["gate"], w["up"], w["down"], self.expert_offsets, self.sorted_pair, self.k,
                              self.y_sorted, self.workspace, s_gate=w.get("gate_scale"), s_up=w.get("up_scale"),
                              s_down=w.get("down_scale"), fat_threshold=fat_threshold, wfmt=self.wfmt, stream=stream)
        B.moe_combine(self.y_sorted, self.topk_w, self.pair_to_sorted, self.out, stream)
        return self.out
