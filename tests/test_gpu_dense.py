"""Dense GPU parity at the headline sizes and at the edges of the work split.

The layer runs at full size through the C ABI (fat threshold 32) and is
compared with the float64 oracle on:

* every 32-row tile of every route list (its first and last row), so every
  MFMA M-tile and every streaming tile of the batch is checked, including the
  items the gate/up MFMA kernel hands out from its counter at the end;
* every row of the hottest expert, of the coldest expert that runs as MFMA
  tiles, of the last two such experts by index (the counter-handed items are
  theirs) and of 8 seeded random experts;
* the layer output of a seeded sample of tokens (256 at 16k);

and, at small hidden sizes, the whole output of layers whose route lists sit
on both sides of the fat threshold (31 / 32 / 33 rows) or whose MFMA items
outnumber the blocks four times over.  Parity bars: integer outputs
bit-exact; max|err| / rms(ref) <= 1e-2 (bf16 experts) or 3e-2 (3-bit).
Each compared quantity is logged as one ``PARITY`` line.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_03_amd as moe
from moe_inputs import SHAPES, LayerShape, layer_weights, routing_inputs
from moe_inputs.device import upload_weights
from tests.gpu_util import (TOL_BF16, TOL_Q3, check_indices, host_raw, oracle_out_tokens, oracle_rows,
                            parity_line, run_layer, say, tile_edge_rows, to_dev_weights, wfmt_id)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    yield


def tol(shape):
    return TOL_BF16 if shape.wfmt == "bf16" else TOL_Q3


_DEV_W = {}


def device_weights(shape, seed):
    key = (shape.H, shape.I, shape.E, shape.wfmt, seed)
    if key not in _DEV_W:
        _DEV_W.clear()
        torch.cuda.empty_cache()
        say(f"[weights] {shape.wfmt} H={shape.H} I={shape.I} E={shape.E} seed={seed}")
        _DEV_W[key] = upload_weights(shape, seed)
    return _DEV_W[key]


def _host_outputs(bufs, rows, tokens):
    ridx = torch.tensor(rows, dtype=torch.int64, device="cuda")
    tidx = torch.tensor(tokens, dtype=torch.int64, device="cuda")
    return bufs.y_sorted[ridx].float().cpu().numpy(), bufs.out[tidx].cpu().numpy()


def big_layer_case(shape, seed, n_tokens, dense_rows=True):
    """Run the full-size layer and compare the checked rows and tokens."""
    thr = 32
    logits, x = routing_inputs(shape, seed)
    dw = device_weights(shape, seed)
    bufs = moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, wfmt_id(shape))
    say(f"[dense] {shape.name} T={shape.T} seed={seed} wfmt={shape.wfmt}: layer on the GPU")
    bufs.forward(torch.from_numpy(logits).cuda(), torch.from_numpy(x.view(np.int16)).cuda(), dw,
                 fat_threshold=thr)
    torch.cuda.synchronize()
    ids, w = oracle.route_topk(logits, shape.k)
    counts, offsets, sp, p2s = oracle.permute(ids, shape.E)
    got = {"ids": bufs.topk_ids.cpu().numpy(), "w": bufs.topk_w.cpu().numpy(),
           "counts": bufs.expert_counts.cpu().numpy(), "offsets": bufs.expert_offsets.cpu().numpy(),
           "sorted_pair": bufs.sorted_pair.cpu().numpy(), "pair_to_sorted": bufs.pair_to_sorted.cpu().numpy()}
    check_indices(got, dict(ids=ids, w=w, counts=counts, offsets=offsets, sorted_pair=sp, pair_to_sorted=p2s))
    say(f"   indices bit-exact ({shape.T * shape.k} pairs)")

    rng = np.random.default_rng([77, seed, shape.T])
    fat = np.flatnonzero(counts >= thr)
    groups = {}
    if fat.size:
        groups["hottest"] = [int(np.argmax(counts))]
        groups["coldest_fat"] = [int(fat[np.argmin(counts[fat])])]
        groups["last_fat"] = [int(e) for e in fat[-2:]]
    touched = np.flatnonzero(counts > 0)
    groups["random8"] = sorted(int(e) for e in rng.choice(touched, size=min(8, touched.size), replace=False))
    rows = set()
    if dense_rows:
        rows.update(tile_edge_rows(offsets))
    for es in groups.values():
        for e in es:
            rows.update(range(int(offsets[e]), int(offsets[e + 1])))
    tokens = sorted({0, shape.T - 1, *rng.choice(shape.T, size=min(n_tokens, shape.T) - 2, replace=False).tolist()})
    rows.update(int(p2s[t * shape.k + j]) for t in tokens for j in range(shape.k))
    rows = sorted(rows)
    say(f"   oracle on {len(rows)} sorted rows of {int(np.unique(np.searchsorted(offsets, rows, 'right') - 1).size)} "
        f"experts, {len(tokens)} tokens; groups {groups}")
    ref = oracle_rows(shape, seed, x, sp, offsets, rows)
    y_got, out_got = _host_outputs(bufs, rows, tokens)
    y_ref = np.stack([ref[r] for r in rows])
    cfg = f"{shape.name}/seed{seed}"
    bar = tol(shape)
    errs = {}
    errs["Y(all checked rows)"] = (oracle.rel_max_err(y_got, y_ref), len(rows))
    pos = {r: i for i, r in enumerate(rows)}
    for name, es in groups.items():
        sel = [pos[r] for e in es for r in range(int(offsets[e]), int(offsets[e + 1]))]
        errs[f"Y({name} {es})"] = (oracle.rel_max_err(y_got[sel], y_ref[sel]), len(sel))
    out_ref = oracle_out_tokens(ref, w, p2s, shape.k, tokens)
    errs["out(sampled tokens)"] = (oracle.rel_max_err(out_got, out_ref), len(tokens))
    for what, (e, n) in errs.items():
        parity_line(cfg, what, e, bar, n)
    for what, (e, n) in errs.items():
        assert e <= bar, f"{cfg} {what}: {e:.3e} > {bar}"
    n = np.diff(offsets)
    say(f"   experts touched {int((n > 0).sum())}, fat {int((n >= thr).sum())}, "
        f"max rows {int(n.max())}, min fat rows {int(n[n >= thr].min()) if (n >= thr).any() else 0}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,seed", [("prefill16k", 0), ("prefill16k", 1), ("prefill16k", 2),
                                       ("prefill16k_q3", 0)])
def test_headline_dense(name, seed):
    big_layer_case(SHAPES[name], seed, 256)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [32768, 65536])
def test_chunk_sizes_beyond_16k(T):
    """The chunk sweep's larger chunks: 32k (every tile edge checked) and 64k
    (the activation buffer reaches 2 GiB and y 4 GiB; the hottest and the
    tail experts and 64 tokens checked)."""
    shape = SHAPES["prefill16k"].with_tokens(T)
    shape = LayerShape(f"chunk{T}", T, shape.H, shape.I, shape.E, shape.k, shape.router, shape.wfmt)
    big_layer_case(shape, 0, 64, dense_rows=(T <= 32768))


def _owner_logits(counts, seed):
    """Logits that route token t (k = 1) to one expert by a wide margin so
    that expert e gets exactly counts[e] tokens, in shuffled order."""
    E, T = len(counts), int(sum(counts))
    rng = np.random.default_rng([seed, T, E])
    owner = np.repeat(np.arange(E), counts)
    rng.shuffle(owner)
    lg = (0.1 * rng.standard_normal((T, E))).astype(np.float32)
    lg[np.arange(T), owner] += np.float32(5.0)
    return lg


# Route lists on both sides of the fat threshold: 31 rows (streaming) next to
# 32 and 33 (MFMA tiles), plus lists that fill whole 256-row M-tiles and pass
# them by one row.
EDGE_COUNTS = [31, 32, 33, 1, 64, 65, 256, 257, 300, 16, 17]


@pytest.mark.parametrize("wfmt", ["bf16", "q3"])
def test_fat_threshold_edges(wfmt):
    E, k = len(EDGE_COUNTS), 1
    T = sum(EDGE_COUNTS)
    shape = LayerShape(f"fat_edges_{wfmt}", T, 256, 256, E, k, "normal", wfmt)
    _, x = routing_inputs(shape, 0)
    logits = _owner_logits(EDGE_COUNTS, 5)
    W = layer_weights(shape, 0)
    ref = oracle.moe_layer(logits, x, host_raw(W), k)
    assert np.array_equal(ref["counts"], EDGE_COUNTS)
    bufs = moe.MoELayerBuffers(T, E, k, shape.H, shape.I, wfmt_id(shape))
    for thr in (32, 33):
        say(f"[fat edges] {wfmt} T={T} counts={EDGE_COUNTS} fat_threshold={thr}")
        got = run_layer(bufs, logits, x, to_dev_weights(W), fat_threshold=thr)
        check_indices(got, ref)
        ey = oracle.rel_max_err(got["Y"], ref["Y"])
        eo = oracle.rel_max_err(got["out"], ref["out"])
        parity_line(f"{shape.name}/thr{thr}", "Y(all rows)", ey, tol(shape), T)
        parity_line(f"{shape.name}/thr{thr}", "out(all tokens)", eo, tol(shape), T)
        assert ey <= tol(shape) and eo <= tol(shape)
        # each route list on its own, so a bad list cannot hide in the global max
        for e, (lo, hi) in enumerate(zip(ref["offsets"][:-1], ref["offsets"][1:])):
            assert oracle.rel_max_err(got["Y"][lo:hi], ref["Y"][lo:hi]) <= tol(shape), f"expert {e} ({hi - lo} rows)"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wfmt", ["bf16", "q3"])
def test_whole_output_many_items(wfmt):
    """Two experts of about 8k rows each (32 M-tiles apiece) and I = 2048: the
    gate/up MFMA kernel has four items per block, so it runs static rounds and
    the counter-driven tail; every output element is compared."""
    shape = LayerShape(f"many_items_{wfmt}", 16384, 256, 2048, 2, 1, "normal", wfmt)
    logits, x = routing_inputs(shape, 0)
    W = layer_weights(shape, 0)
    say(f"[many items] {wfmt}: oracle over the whole layer")
    ref = oracle.moe_layer(logits, x, host_raw(W), 1)
    bufs = moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, wfmt_id(shape))
    got = run_layer(bufs, logits, x, to_dev_weights(W), fat_threshold=32)
    check_indices(got, ref)
    ey = oracle.rel_max_err(got["Y"], ref["Y"])
    eo = oracle.rel_max_err(got["out"], ref["out"])
    parity_line(shape.name, "Y(all rows)", ey, tol(shape), shape.T)
    parity_line(shape.name, "out(all tokens)", eo, tol(shape), shape.T)
    say(f"   counts {ref['counts'].tolist()}")
    assert ey <= tol(shape) and eo <= tol(shape)
