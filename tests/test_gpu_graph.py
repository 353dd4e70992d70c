"""A whole layer call (route, permute, grouped FFN, combine) captured into a
HIP graph through torch.cuda.CUDAGraph and replayed.

The library enqueues only kernels on the caller's stream -- no memset, no
allocation, no host synchronisation, and the work lists stay on the device --
so a layer call can be captured, and every replay must reproduce eager
execution bit for bit, also when the inputs in the captured buffers change
between replays (the routing, the per-expert lists and the tile plan all
change with them).  Between replays the outputs are cleared by eager kernels
and the host synchronises, so a replay that did not recompute them would
fail the comparison.
"""
import numpy as np
import pytest
import torch

import routed_expert_ffn_03_amd as moe
from moe_inputs import LayerShape, layer_weights, routing_inputs
from tests.gpu_util import say, to_dev_weights, wfmt_id

CASES = [
    # fat experts (about 230 rows each) on the MFMA tile path
    LayerShape("mid", 700, 512, 384, 6, 2, "normal", "bf16"),
    LayerShape("mid_q3", 700, 512, 384, 6, 2, "normal", "q3"),
    # a decode-sized step: every expert thin
    LayerShape("step", 4, 512, 384, 64, 8, "zipf", "bf16"),
    LayerShape("step_q3", 4, 512, 384, 64, 8, "zipf", "q3"),
]


def _outputs(b):
    return [t.clone() for t in (b.topk_ids, b.topk_w, b.expert_counts, b.expert_offsets, b.sorted_pair,
                                b.pair_to_sorted, b.y_sorted, b.out)]


@pytest.mark.gpu
@pytest.mark.parametrize("shape", CASES, ids=[s.name for s in CASES])
def test_layer_graph_replay_matches_eager(shape):
    say(f"[graph] {shape.name} T={shape.T} E={shape.E} k={shape.k} H={shape.H} I={shape.I} wfmt={shape.wfmt}")
    inputs = [routing_inputs(shape, seed) for seed in (0, 1)]
    w = to_dev_weights(layer_weights(shape, 0))
    b = moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, wfmt_id(shape))
    logits = torch.empty((shape.T, shape.E), dtype=torch.float32, device="cuda")
    x = torch.empty((shape.T, shape.H), dtype=torch.int16, device="cuda")

    def load(i):
        lg, xx = inputs[i]
        logits.copy_(torch.from_numpy(lg))
        x.copy_(torch.from_numpy(xx.view(np.int16)))

    refs = []
    for i in range(2):
        load(i)
        b.forward(logits, x, w)
        torch.cuda.synchronize()
        refs.append(_outputs(b))

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.forward(logits, x, w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        b.forward(logits, x, w)
    torch.cuda.synchronize()

    for rep in range(5):
        i = (rep + 1) % 2
        load(i)
        for t in (b.topk_ids, b.sorted_pair, b.y_sorted, b.out):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(b)
        for name, g, r in zip(("ids", "w", "counts", "offsets", "sorted_pair", "pair_to_sorted", "y", "out"),
                              got, refs[i]):
            assert torch.equal(g, r), f"replay {rep} (inputs {i}): {name} differs from eager"
        say(f"   replay {rep} on inputs {i}: identical to eager")


# More fat items than one round of blocks, so the gate/up phase runs both its
# static rounds and its counter-driven tail; and a layer with fewer items than
# blocks (all of them from the counter).
REPEAT_CASES = [
    LayerShape("mid", 700, 512, 384, 6, 2, "normal", "bf16"),
    LayerShape("many", 8192, 256, 1024, 64, 8, "normal", "bf16"),
    LayerShape("many_q3", 8192, 256, 1024, 64, 8, "normal", "q3"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("shape", REPEAT_CASES, ids=[s.name for s in REPEAT_CASES])
def test_ffn_phases_repeat_on_one_plan(shape):
    """The fat gate/up kernel hands out its last rounds of items from a
    counter in the workspace; the last block of each launch re-zeroes it.
    Gate/up and down run again and again on one plan (no re-plan in between),
    alternating two activation inputs with the same routing, must reproduce
    each input's y bit for bit: an item skipped because the counter was left
    high would keep the other input's activations."""
    say(f"[repeat] {shape.name} T={shape.T} E={shape.E} k={shape.k} H={shape.H} I={shape.I} wfmt={shape.wfmt}")
    lg, x0 = routing_inputs(shape, 0)
    _, x1 = routing_inputs(shape, 1)
    w = to_dev_weights(layer_weights(shape, 0))
    b = moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, wfmt_id(shape))
    logits = torch.from_numpy(lg).cuda()
    xs = [torch.from_numpy(xx.view(np.int16)).cuda() for xx in (x0, x1)]
    refs = []
    for x in xs:
        b.forward(logits, x, w)
        torch.cuda.synchronize()
        refs.append(b.y_sorted.clone())
    assert not torch.equal(refs[0], refs[1])
    for rep in range(4):
        i = rep % 2
        b.y_sorted.zero_()
        moe.moe_ffn_gate_up(xs[i], w["gate"], w["up"], b.sorted_pair, shape.E, shape.k, b.workspace,
                            s_gate=w.get("gate_scale"), s_up=w.get("up_scale"), wfmt=wfmt_id(shape))
        moe.moe_ffn_down(w["down"], shape.T, shape.E, shape.k, shape.I, b.y_sorted, b.workspace,
                         s_down=w.get("down_scale"), wfmt=wfmt_id(shape))
        torch.cuda.synchronize()
        assert torch.equal(b.y_sorted, refs[i]), f"repeat {rep} (input {i}): y differs"
        say(f"   repeat {rep} on input {i}: identical")


# Several decode layers captured into one graph and replayed, every layer's
# output checked against the float64 oracle on every replay (not only against
# eager execution): the pages run decode as captured graphs and re-enabled
# them only after a parity run over many decode steps showed no mismatch.
MULTI_CASES = [
    (LayerShape("dec_small", 4, 512, 256, 64, 8, "zipf", "bf16"), 3),
    (LayerShape("dec_small_q3", 4, 512, 256, 64, 8, "zipf", "q3"), 3),
    (LayerShape("dec_full_q3", 4, 4096, 2048, 384, 8, "zipf", "q3"), 3),
    (LayerShape("dec_full_b1_q3", 1, 4096, 2048, 384, 8, "zipf", "q3"), 2),
]


@pytest.mark.gpu
@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape,n_layers", MULTI_CASES, ids=[s.name for s, _ in MULTI_CASES])
def test_multilayer_decode_graph_against_oracle(shape, n_layers):
    import oracle
    from moe_inputs import for_each_expert
    from moe_inputs.device import upload_weights
    from tests.gpu_util import TOL_BF16, TOL_Q3, oracle_out_tokens, oracle_rows, parity_line

    bar = TOL_BF16 if shape.wfmt == "bf16" else TOL_Q3
    say(f"[multilayer graph] {shape.name}: {n_layers} layers, T={shape.T} H={shape.H} I={shape.I} E={shape.E}")
    layers, bufs, ins, refs = [], [], [], []
    for li in range(n_layers):
        wseed = 50 + li
        layers.append(upload_weights(shape, wseed))
        bufs.append(moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, wfmt_id(shape)))
        ins.append((torch.empty((shape.T, shape.E), dtype=torch.float32, device="cuda"),
                    torch.empty((shape.T, shape.H), dtype=torch.int16, device="cuda")))
        # two input sets per layer: the replays alternate between them
        per = []
        for iset in range(2):
            lg, x = routing_inputs(shape, 1000 * iset + li)
            ids, w = oracle.route_topk(lg, shape.k)
            _, offsets, sp, p2s = oracle.permute(ids, shape.E)
            yrows = oracle_rows(shape, wseed, x, sp, offsets, range(shape.T * shape.k))
            out = oracle_out_tokens(yrows, w, p2s, shape.k, range(shape.T))
            per.append((lg, x, ids, out))
        refs.append(per)

    def load(iset):
        for li in range(n_layers):
            lg, x = refs[li][iset][0], refs[li][iset][1]
            ins[li][0].copy_(torch.from_numpy(lg))
            ins[li][1].copy_(torch.from_numpy(x.view(np.int16)))

    def step():
        for li in range(n_layers):
            bufs[li].forward(ins[li][0], ins[li][1], layers[li])

    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(6):
        iset = rep % 2
        load(iset)
        for b in bufs:
            b.out.zero_()
            b.topk_ids.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for li in range(n_layers):
            _, _, ids, out_ref = refs[li][iset]
            assert np.array_equal(bufs[li].topk_ids.cpu().numpy(), ids), f"replay {rep} layer {li}: ids"
            err = oracle.rel_max_err(bufs[li].out.cpu().numpy(), out_ref)
            if rep < 2:
                parity_line(f"{shape.name}/graph/layer{li}/inputs{iset}", "out(all tokens)", err, bar, shape.T)
            assert err <= bar, f"replay {rep} layer {li}: {err:.3e}"
    say(f"   6 replays x {n_layers} layers match the oracle")
    del graph
