"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare it with the float64 oracle."""
import sys

import numpy as np
import torch

import oracle
from moe_inputs import LayerShape, expert_weights, layer_weights, routing_inputs
from moe_inputs.device import upload_weights

# parity bars: integer outputs bit-exact; layer output max|err| / rms(ref)
TOL_BF16 = 1e-2
TOL_Q3 = 3e-2
# gate weights: fp32 exp/divide against float64 (a few ulp of 1.0)
TOL_W = 2e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def wfmt_id(shape: LayerShape) -> int:
    return 0 if shape.wfmt == "bf16" else 1


def to_dev_weights(W: dict, device="cuda") -> dict:
    out = {}
    for n, a in W.items():
        out[n] = torch.from_numpy(a.view(np.int16 if a.dtype == np.uint16 else np.int32)).to(device)
    return out


def host_raw(W: dict):
    return lambda e: {n: a[e] for n, a in W.items()}


def run_layer(bufs, logits_np, x_np, dw, fat_threshold=32):
    dl = torch.from_numpy(logits_np).cuda()
    dx = torch.from_numpy(x_np.view(np.int16)).cuda()
    bufs.forward(dl, dx, dw, fat_threshold=fat_threshold)
    torch.cuda.synchronize()
    return {
        "ids": bufs.topk_ids.cpu().numpy(), "w": bufs.topk_w.cpu().numpy(),
        "counts": bufs.expert_counts.cpu().numpy(), "offsets": bufs.expert_offsets.cpu().numpy(),
        "sorted_pair": bufs.sorted_pair.cpu().numpy(), "pair_to_sorted": bufs.pair_to_sorted.cpu().numpy(),
        "Y": bufs.y_sorted.float().cpu().numpy(), "out": bufs.out.cpu().numpy(),
    }


def check_indices(got, ref):
    assert np.array_equal(got["ids"], ref["ids"]), "topk ids differ"
    assert np.array_equal(got["counts"], ref["counts"]), "expert histogram differs"
    assert np.array_equal(got["offsets"], ref["offsets"]), "expert offsets differ"
    assert np.array_equal(got["sorted_pair"], ref["sorted_pair"]), "sorted_pair differs"
    assert np.array_equal(got["pair_to_sorted"], ref["pair_to_sorted"]), "pair_to_sorted differs"
    np.testing.assert_allclose(got["w"], ref["w"], rtol=0, atol=TOL_W)
