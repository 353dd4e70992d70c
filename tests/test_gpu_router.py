"""Fused router (GEMM + top-k gate) through the C ABI against the oracle.

* logits (written when asked for) within the fp32 summation bound of the
  float64 logits: the bf16 products are exact in fp32, so whatever the order
  of the K - 1 additions, |err| <= gamma_{K-1} * sum_k |x_k w_k|;
* ids, gate weights and histogram equal the oracle's gate applied to the
  kernel's own fp32 logits -- the selection is decided in the kernel's
  precision on both sides, so indices must match bit for bit;
* the fused call (no logits output) gives bit-identical ids, weights and
  histogram -- for a few tokens the call with logits runs the GEMM split over
  the experts, so this also checks that both kernels compute the same logits;
* every selected expert is a valid top-k choice for the float64 logits up to
  twice that bound (the sets can differ only between near-equal logits).
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_03_amd as moe
from moe_inputs import float32_to_bf16_bits, router_weights
from tests.gpu_util import TOL_W, say

pytestmark = pytest.mark.gpu

# (T, E, H, k): ragged token blocks, every supported expert count, decode and the 16k chunk.  With the logits
# asked for, T <= 32 splits the GEMM over the experts (512-k batches; a deeper ring of 16 token rows at T <= 16):
# T = 16 / 17 and 32 / 33 sit on either side of those switches, H = 1056 and 4128 end in a partial batch;
# k = 16 and 32 take the per-wave selection, k <= 8 the per-lane one.
CASES = [(64, 128, 256, 2), (333, 256, 512, 4), (700, 384, 1024, 8), (1, 384, 4096, 8), (4, 512, 4096, 8),
         (16, 384, 1056, 8), (32, 256, 1056, 4), (17, 128, 4128, 8), (33, 128, 512, 2), (16384, 384, 4096, 8),
         (100, 256, 512, 16), (70, 512, 256, 32)]


def _x(T, H, seed):
    rng = np.random.default_rng([seed, 0x5EED, T, H])
    return float32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T,E,H,k", CASES, ids=[f"T{c[0]}_E{c[1]}_H{c[2]}_k{c[3]}" for c in CASES])
def test_router_topk(T, E, H, k):
    say(f"[router] T={T} E={E} H={H} k={k}")
    x = _x(T, H, 0)
    w = router_weights(E, H, 0)
    dx = torch.from_numpy(x.view(np.int16)).cuda()
    dw = torch.from_numpy(w.view(np.int16)).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    cnt = torch.empty((E,), dtype=torch.int32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(dx, dw, k, ids, tw, cnt, logits=lg)
    torch.cuda.synchronize()
    got_l = lg.cpu().numpy()
    got_ids, got_w, got_c = ids.cpu().numpy(), tw.cpu().numpy(), cnt.cpu().numpy()

    ref_l = oracle.router_logits(x, w)
    xa, wa = np.abs(oracle.bf16_to_f64(x)), np.abs(oracle.bf16_to_f64(w))
    u = 2.0 ** -24
    gamma = (H - 1) * u / (1 - (H - 1) * u)
    bound = gamma * (xa @ wa.T)
    excess = np.abs(got_l - ref_l) - bound
    assert excess.max() <= 0, f"logit error above the fp32 bound by {excess.max():.3e}"
    say(f"   max |logit err| {np.abs(got_l - ref_l).max():.3e} (bound at that entry "
        f"{bound.flat[np.argmax(np.abs(got_l - ref_l))]:.3e})")

    ref_ids, ref_w = oracle.route_topk(got_l, k)
    assert np.array_equal(got_ids, ref_ids), "ids differ from the gate on the kernel's logits"
    np.testing.assert_allclose(got_w, ref_w, rtol=0, atol=TOL_W)
    assert np.array_equal(got_c, oracle.expert_histogram(ref_ids, E))

    # fused: no logits output, same choice; then with only a workspace (at
    # most 32 tokens: the split GEMM writes its logits there), same choice
    ids2, tw2, cnt2 = torch.empty_like(ids), torch.empty_like(tw), torch.empty_like(cnt)
    moe.moe_router_topk(dx, dw, k, ids2, tw2, cnt2)
    torch.cuda.synchronize()
    assert torch.equal(ids2, ids) and torch.equal(tw2, tw) and torch.equal(cnt2, cnt)
    ws = torch.empty(T * E * 4, dtype=torch.uint8, device="cuda")
    ids3, tw3, cnt3 = torch.empty_like(ids), torch.empty_like(tw), torch.full_like(cnt, 77)
    moe.moe_router_topk(dx, dw, k, ids3, tw3, cnt3, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(ids3, ids) and torch.equal(tw3, tw) and torch.equal(cnt3, cnt)

    # validity against float64: a selected logit is not below an unselected one by more than the bounds
    sel = np.take_along_axis(ref_l, got_ids.astype(np.int64), axis=1)
    mask = np.ones_like(ref_l, dtype=bool)
    np.put_along_axis(mask, got_ids.astype(np.int64), False, axis=1)
    best_unsel = np.where(mask, ref_l, -np.inf).max(axis=1)
    slack = 2 * bound.max(axis=1)
    assert np.all(sel.min(axis=1) >= best_unsel - slack)
