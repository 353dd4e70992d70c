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


def oracle_rows(shape, seed, x_bits, sorted_pair, offsets, rows, chunk=16):
    """Float64 oracle Y for the sorted rows ``rows`` only (dict row -> [H]).

    The experts those rows belong to are generated a few at a time (never the
    whole layer on the host) and each runs oracle.expert_ffn on just its
    requested rows."""
    from moe_inputs import for_each_expert
    rows = np.unique(np.asarray(rows, dtype=np.int64))
    owner = np.searchsorted(offsets, rows, side="right") - 1
    x = oracle.bf16_to_f64(x_bits)
    out = {}
    experts = np.unique(owner).tolist()
    for c0 in range(0, len(experts), chunk):
        part = experts[c0:c0 + chunk]
        raw = {}
        for_each_expert(shape, seed, lambda e, a: raw.__setitem__(e, a), experts=part)
        for e in part:
            r = rows[owner == e]
            tok = np.asarray(sorted_pair)[r] // shape.k
            y = oracle.expert_ffn(x[tok], *oracle.expert_matrices(raw.pop(e)))
            for i, row in enumerate(r.tolist()):
                out[row] = y[i]
    return out


def oracle_out_tokens(yrows: dict, w, pair_to_sorted, k, tokens):
    """oracle.combine for ``tokens`` on the compact rows of ``oracle_rows``."""
    keys = sorted(yrows)
    index = {r: i for i, r in enumerate(keys)}
    Yc = np.stack([yrows[r] for r in keys])
    p2s = np.full(len(pair_to_sorted), -1, dtype=np.int64)
    for t in tokens:
        for j in range(k):
            p2s[t * k + j] = index[int(pair_to_sorted[t * k + j])]
    return oracle.combine(Yc, np.asarray(w, dtype=np.float64), p2s, k, tokens=list(tokens))


def tile_edge_rows(offsets, tile=32):
    """First and last sorted row of every 32-row tile of every route list.
    Every MFMA M-tile and every streaming tile is made of whole 32-row tiles,
    so these rows touch each of them."""
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for r0 in range(lo, hi, tile):
            rows.append(r0)
            rows.append(min(r0 + tile, hi) - 1)
    return rows


def parity_line(config, what, err, bar, n):
    """One machine-readable parity record in the test log."""
    say(f"PARITY {config} {what} err={err:.4e} bar={bar:.0e} n={n}")
