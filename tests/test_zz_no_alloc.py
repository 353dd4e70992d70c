"""The allocation-free grouped FFN (moe_grouped_ffn_noalloc) against the
grouped FFN with a caller workspace (moe_grouped_ffn): the same kernels on
the library's per-GPU scratch array, so y must match bit for bit.  Two calls
in a row, the second on a smaller batch, so that nothing the first call left
in the shared array leaks into the second; every weight format (bf16,
3-bit, and bf16 packed into the row-pair layout with W_down in fp16)."""
import numpy as np
import pytest
import torch

import routed_expert_ffn_03_amd as moe
from moe_inputs import LayerShape, layer_weights, routing_inputs
from tests.gpu_util import say, to_dev_weights, wfmt_id


def _routed(shape, seed, wfmt):
    logits, x = routing_inputs(shape, seed)
    b = moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, wfmt)
    moe.moe_route_topk(torch.from_numpy(logits).cuda(), shape.k, b.topk_ids, b.topk_w, b.expert_counts)
    moe.moe_permute(b.topk_ids, shape.E, b.expert_offsets, b.sorted_pair, b.pair_to_sorted, b.workspace)
    return b, torch.from_numpy(x.view(np.int16)).cuda()


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["bf16", "q3", "pairs"])
def test_noalloc_matches_workspace_entry_point(fmt):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    gen = "q3" if fmt == "q3" else "bf16"
    big = LayerShape(f"noalloc_{fmt}", 700, 512, 256, 16, 4, "zipf", gen)      # MFMA and streaming tiles
    small = LayerShape(f"noalloc_small_{fmt}", 5, 512, 256, 16, 4, "zipf", gen)  # streaming tiles only
    w = to_dev_weights(layer_weights(big, 0))
    wfmt = wfmt_id(big)
    if fmt == "pairs":
        wfmt = moe.MOE_WFMT_BF16_PAIRS
        for n in list(w):
            d = torch.empty_like(w[n])
            moe.moe_pack_bf16_pairs(w[n], d, to_fp16=(n == "down"))
            w[n] = d
    for shape, seed in ((big, 0), (small, 1)):
        say(f"[noalloc] {shape.name} T={shape.T} E={shape.E} k={shape.k} H={shape.H} I={shape.I}")
        b, x = _routed(shape, seed, wfmt)
        kw = dict(s_gate=w.get("gate_scale"), s_up=w.get("up_scale"), s_down=w.get("down_scale"),
                  fat_threshold=32, wfmt=wfmt)
        moe.moe_grouped_ffn(x, w["gate"], w["up"], w["down"], b.expert_offsets, b.sorted_pair, shape.k,
                            b.y_sorted, b.workspace, **kw)
        torch.cuda.synchronize()
        ref = b.y_sorted.clone()
        b.y_sorted.fill_(7.0)
        moe.moe_grouped_ffn_noalloc(x, w["gate"], w["up"], w["down"], b.expert_offsets, b.sorted_pair, shape.k,
                                    b.y_sorted, **kw)
        torch.cuda.synchronize()
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(b.y_sorted, ref), f"{shape.name}: y differs from moe_grouped_ffn"
        say("   identical to moe_grouped_ffn")


@pytest.mark.gpu
def test_noalloc_rejects_batches_beyond_the_array():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = moe.lib()
    F = 0x10000                     # never dereferenced: the size check comes first
    # 16,384 tokens x 8 x 2048 x 2 bytes of activation is far beyond 64 MiB
    st = L.moe_grouped_ffn_noalloc(F, 0, F, F, F, None, None, None, F, F, 16384, 384, 8, 4096, 2048, 32, F, None)
    assert st == moe.MOE_ERR_WORKSPACE
