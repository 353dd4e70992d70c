#!/usr/bin/env python3
"""Throughput of the routed-expert layer on one MI355X.

One step = one full layer call (route -> permute -> plan -> gate/up -> down
-> combine; the first three in one launch for decode-sized batches) over one
batch of synthetic inputs already resident in HBM.
The headline workload is the 16,384-token prefill chunk (bf16 experts,
Zipf-skewed router); the 4-token decode step is measured in the same run on
the same weights and reported under "decode" (with --workload prefill16k_q3:
the decode step on the same 3-bit weights).  Every timed step sits between
its own pair of HIP events on the library's stream, and a 512 MiB scratch
buffer is read between steps (outside the events) so that no step starts
with the previous one's weights in the MALL; the line reports the
mean (value, ms_per_step) and the median, p10 and p90.  The dominant
kernel's time (the gate/up phase) is taken the same way in a second timed
run of the same steps (an event between two kernels idles the GPU for a few
microseconds, so it is kept out of the layer timing).

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 16k-token prefill and 4-token decode; % MFMA/HBM peak"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}      # dense, MI355X published
PEAK_HBM_GBS = 8000.0
FLUSH_BYTES = 512 << 20                                   # > the 256 MB MALL
# gate/up phase kernels (template argument: the phase)
GATE_UP_KERNELS = {"bf16": ("ffn_fat8_kernel<1>", "ffn_stream_kernel<1>"),
                   "q3": ("ffn_fat_kernel<1, 1, 6>", "ffn_thin_q3_kernel<1> or, at decode, ffn_q3_decode_kernel")}
# the sources of the expert-FFN kernels; their hash keys the counter figures in profiles/hbm_traffic.md
FFN_SOURCES = ("ffn.hip", "fat8.hip", "stream.hip", "q3dec.hip", "ffn_shared.h", "lds_dma.h", "common.h")


def ffn_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in FFN_SOURCES:
        with open(os.path.join(ROOT, "routed_expert_ffn_03_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:12]


def measured_traffic(workload: str):
    """HBM bytes per launch of the gate/up phase from the committed counter
    summary (profiles/hbm_traffic.md), or None when it was measured on a
    different version of the kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    want = ffn_source_hash()
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 6 and cells[0] == workload and cells[1] == "gate/up" and cells[2] == want:
            try:
                return float(cells[3]) + float(cells[4])
            except ValueError:
                return None
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="prefill16k",
                   choices=["prefill16k", "decode", "prefill1k", "prefill16k_q3", "decode_q3"])
    p.add_argument("--decode-steps", type=int, default=200, help="steps of the secondary decode measurement")
    p.add_argument("--no-decode", action="store_true", help="skip the secondary decode measurement")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=1024, help="tokens of the batch the oracle is timed on")
    p.add_argument("--no-flush", action="store_true",
                   help="do not read the 512 MiB scratch buffer between timed steps")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--layout", choices=("pairs", "plain"), default="pairs",
                   help="storage of bf16 expert weights: the row-pair layout (MOE_WFMT_BF16_PAIRS, packed once "
                        "after upload, outside any timed region) or plain row-major (MOE_WFMT_BF16)")
    p.add_argument("--fat-threshold", type=int, default=32)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (HBM counter calibration)")
    p.add_argument("--sweep", default=None,
                   help="comma-separated token counts: time the bf16 Zipf layer at each chunk size "
                        "(one JSON line per size) instead of the headline measurement")
    p.add_argument("--multilayer-decode", type=int, default=0, metavar="LAYERS",
                   help="decode through LAYERS layers of 3-bit experts, eager and as one captured graph, "
                        "at the batch sizes of --batches (one JSON line) instead of the headline measurement")
    p.add_argument("--batches", default="1,4,8,16,24", help="decode batch sizes of --multilayer-decode")
    p.add_argument("--router", action="store_true",
                   help="time the fused router GEMM + top-k (moe_router_topk) on the 16k and decode batches "
                        "(one JSON line) instead of the headline measurement")
    return p.parse_args()


def workload_desc(shape, thr, pairs=False):
    router = "Zipf(s=1.1) bias, beta=0.4" if shape.router == "zipf" else "N(0,1), no skew"
    layout = ("row pairs interleaved every 32 k, W_down stored fp16 (MOE_WFMT_BF16_PAIRS)" if pairs
              else "plain row-major") \
        if shape.wfmt == "bf16" else "3-bit groups of 128 (MOE_WFMT_Q3G128)"
    return {
        "workload": f"{shape.name}: routed-expert layer, {shape.T} tokens, hidden {shape.H}, "
                    f"expert inter {shape.I}, {shape.E} experts, top-{shape.k}, {shape.wfmt} experts",
        "tokens": shape.T, "hidden": shape.H, "inter": shape.I, "experts": shape.E, "top_k": shape.k,
        "router": router, "expert_weights": shape.wfmt, "weight_layout": layout, "fat_threshold": thr,
    }


def pack_pairs(dev_w):
    """bf16 expert weights -> the row-pair layout (moe_pack_bf16_pairs; W_down
    converted to fp16), one matrix family at a time, the plain copy freed as
    soon as it is packed."""
    import torch

    import routed_expert_ffn_03_amd as moe
    t0 = time.perf_counter()
    for name in list(dev_w):
        src = dev_w[name]
        dst = torch.empty_like(src)
        moe.moe_pack_bf16_pairs(src, dst, to_fp16=(name == "down"))
        torch.cuda.synchronize()
        dev_w[name] = dst
        del src
    torch.cuda.empty_cache()
    log(f"[bench] bf16 weights packed into the row-pair layout in {time.perf_counter() - t0:.2f} s")
    return dev_w


class StepTimes:
    """Per-step layer and gate/up-phase times (ms) of one timed run."""

    def __init__(self, layer_ms, gate_up_ms, wall_ms):
        import numpy as np
        self.layer = np.asarray(layer_ms)
        self.gate_up = np.asarray(gate_up_ms)
        self.wall_ms = wall_ms                        # host clock per step, flush included

    @property
    def mean(self):
        return float(self.layer.mean())

    @property
    def gate_up_mean(self):
        return float(self.gate_up.mean())

    def stats(self):
        import numpy as np
        q = lambda a, p: float(np.percentile(a, p))
        return {"mean_ms": self.mean, "median_ms": q(self.layer, 50), "p10_ms": q(self.layer, 10),
                "p90_ms": q(self.layer, 90), "gate_up_median_ms": q(self.gate_up, 50),
                "wall_ms_per_step_incl_flush": self.wall_ms, "reps": int(self.layer.size)}


class Runner:
    """Buffers of one workload and a step that times the gate/up phase with events."""

    def __init__(self, shape, seed, dev_w, thr, pairs=False):
        import numpy as np
        import torch

        import routed_expert_ffn_03_amd as moe
        from moe_inputs import routing_inputs

        self.moe, self.torch, self.shape, self.w, self.thr = moe, torch, shape, dev_w, thr
        self.logits_np, self.x_np = routing_inputs(shape, seed)
        self.logits = torch.from_numpy(self.logits_np).cuda()
        self.x = torch.from_numpy(self.x_np.view(np.int16)).cuda()
        self.pairs = pairs and shape.wfmt == "bf16"
        self.wfmt = moe.MOE_WFMT_Q3G128 if shape.wfmt != "bf16" else (
            moe.MOE_WFMT_BF16_PAIRS if self.pairs else moe.MOE_WFMT_BF16)
        self.b = moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, self.wfmt)

    def step(self, ev=None):
        m, b, s, w = self.moe, self.b, self.shape, self.w
        # route + permute + plan (one launch for decode-sized batches)
        m.moe_route_permute_plan(self.logits, s.k, s.H, s.I, b.topk_ids, b.topk_w, b.expert_counts,
                                 b.expert_offsets, b.sorted_pair, b.pair_to_sorted, b.workspace,
                                 fat_threshold=self.thr, wfmt=self.wfmt)
        if ev is not None:
            ev[0].record()
        m.moe_ffn_gate_up(self.x, w["gate"], w["up"], b.sorted_pair, s.E, s.k, b.workspace,
                          s_gate=w.get("gate_scale"), s_up=w.get("up_scale"), fat_threshold=self.thr, wfmt=self.wfmt)
        if ev is not None:
            ev[1].record()
        m.moe_ffn_down(w["down"], s.T, s.E, s.k, s.I, b.y_sorted, b.workspace, s_down=w.get("down_scale"),
                       fat_threshold=self.thr, wfmt=self.wfmt)
        m.moe_combine(b.y_sorted, b.topk_w, b.pair_to_sorted, b.out)

    def measure(self, steps, warmup, flush=None):
        """Two timed runs of `steps` layer calls each.  Run 1: each call between
        its own pair of HIP events on the library's stream (the layer time).
        Run 2: events around the gate/up phase only (the dominant kernel's
        time).  An event between two kernels leaves the GPU idle for several
        microseconds, so the layer is not timed with the phase events inside
        it.  With `flush` (a 512 MiB device buffer) the buffer is read in full
        before every call, outside the events, so no call finds the previous
        one's weights in the 256 MB MALL or the L2s; a read leaves only clean
        lines behind (a write would leave dirty ones that the timed call would
        then have to write back)."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        ev = lambda: torch.cuda.Event(enable_timing=True)
        layer = [(ev(), ev()) for _ in range(steps)]
        gu = [(ev(), ev()) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if flush is not None:
                flush.sum()
            layer[i][0].record()
            self.step()
            layer[i][1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(steps):
            if flush is not None:
                flush.sum()
            self.step(gu[i])
        torch.cuda.synchronize()
        return StepTimes([a.elapsed_time(b) for a, b in layer], [a.elapsed_time(b) for a, b in gu],
                         (t1 - t0) * 1e3 / steps)

    def roofline(self, gate_up_ms):
        import numpy as np
        s = self.shape
        counts = self.b.expert_counts.cpu().numpy()
        touched = int((counts > 0).sum())
        P = s.T * s.k
        # gate+up weight bytes of one expert: bf16, or 13 words + one fp16 scale per 128 weights
        per_expert = 2 * s.I * s.H * 2 if s.wfmt == "bf16" else 2 * s.I * (s.H // 128) * (13 * 4 + 2)
        wbytes_gate_up = touched * per_expert
        flops_gate_up = 4.0 * s.H * s.I * P
        t = gate_up_ms * 1e-3
        fat = int((counts >= self.thr).sum())
        # MFMA-bound when the pairs per touched expert pass the ridge: flops per
        # pair / MFMA peak = expert bytes / HBM peak (about 313 rows for bf16
        # experts, 66 for 3-bit ones)
        ridge = (per_expert / (PEAK_HBM_GBS * 1e9)) / (4.0 * s.H * s.I / (PEAK_MFMA_TFLOPS["bf16"] * 1e12))
        if P / max(touched, 1) >= ridge:
            r = {"bound": "mfma", "achieved": flops_gate_up / t / 1e12, "peak": PEAK_MFMA_TFLOPS["bf16"],
                 "unit": "TFLOP/s"}
            per = f"{4 * s.H * s.I} flop per (token, expert) pair x {P} pairs"
        else:
            r = {"bound": "hbm", "achieved": wbytes_gate_up / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
            per = f"{per_expert} gate+up weight bytes per touched expert x {touched} experts"
        r["frac"] = r["achieved"] / r["peak"]
        r["traffic"] = measured_traffic(s.name)
        r["traffic_source"] = ("rocprofv3 FETCH_SIZE + WRITE_SIZE of these kernel sources "
                               f"(sha256[:12] {ffn_source_hash()}), profiles/hbm_traffic.md"
                               if r["traffic"] is not None else "not measured for these kernel sources")
        fat_name, thin_name = GATE_UP_KERNELS[s.wfmt]
        r["kernel"] = f"gate/up phase ({fat_name} + {thin_name})"
        r["kernel_ms"] = gate_up_ms
        r["algorithmic"] = per
        r["experts_touched"] = touched
        r["experts_fat"] = fat
        return r

    def layer_hbm(self, layer_ms):
        """Whole-layer weight streaming rate: every touched expert's gate, up and
        down bytes over the layer step time (the decode bound)."""
        s = self.shape
        counts = self.b.expert_counts.cpu().numpy()
        touched = int((counts > 0).sum())
        per_expert = (3 * s.I * s.H * 2 if s.wfmt == "bf16"
                      else 2 * s.I * (s.H // 128) * (13 * 4 + 2) + s.H * (s.I // 128) * (13 * 4 + 2))
        gbs = touched * per_expert / (layer_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "algorithmic": f"{per_expert} gate+up+down weight bytes per touched expert x {touched} experts "
                               f"over the whole layer step"}


def _time_oracle(shape, seed, n_tokens, threads):
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from moe_inputs import for_each_expert, routing_inputs

    logits, x = routing_inputs(shape, seed)
    logits, x = logits[:n_tokens], x[:n_tokens]
    ids, _ = oracle.route_topk(logits, shape.k)
    need = sorted({int(e) for e in ids.ravel()})
    raw = {}
    for_each_expert(shape, seed, lambda e, a: raw.__setitem__(e, a), experts=need)
    with threadpool_limits(limits=threads):
        blas = sorted({(i["internal_api"], i["num_threads"]) for i in threadpool_info()})
        t0 = time.perf_counter()
        oracle.moe_layer(logits, x, lambda e: raw[e], shape.k)
        dt = time.perf_counter() - t0
    return n_tokens / dt, dt, len(need), blas


def cpu_baseline(shape, seed, n_tokens):
    """The float64 oracle as it is (numpy, BLAS per expert), timed on the host
    cores available to this process: the first n_tokens tokens of the headline
    batch with every core, plus 1-thread figures for the tiny layer and the
    4-token decode step.  Expert generation is excluded."""
    from moe_inputs import SHAPES

    cores = len(os.sched_getaffinity(0))
    v, dt, ne, blas = _time_oracle(shape, seed, n_tokens, cores)
    res = {"value": v, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"first {n_tokens} tokens of the {shape.name} batch (seed {seed}): route, permute, {ne} experts' "
                     f"SwiGLU FFN and combine in float64 numpy, {cores} host threads (BLAS {blas}); {dt:.1f} s"}
    single = {}
    for name in ("tiny", "decode" if shape.wfmt == "bf16" else "decode_q3"):
        s1 = SHAPES[name]
        v1, dt1, ne1, _ = _time_oracle(s1, seed, s1.T, 1)
        single[name] = {"value": v1, "unit": "tokens/s", "cores": 1, "seconds": dt1, "experts": ne1}
    res["single_thread"] = single
    return res


def chunk_sweep(sizes, seed, thr, pairs):
    """The bf16 layer (Zipf router) at several chunk sizes: where the step turns
    from weight streaming (HBM) to MFMA bound.  One JSON line per size."""
    import torch

    from moe_inputs import SHAPES, LayerShape
    from moe_inputs.device import upload_weights

    base = SHAPES["prefill16k"]
    dev_w = upload_weights(base, seed)
    if pairs:
        dev_w = pack_pairs(dev_w)
    for T in sizes:
        shape = LayerShape(f"chunk{T}", T, base.H, base.I, base.E, base.k, base.router, base.wfmt)
        run = Runner(shape, seed, dev_w, thr, pairs)
        steps = max(3, min(50, int(2e5 / T)))
        st = run.measure(steps, 2)
        ms, gu = st.mean, st.gate_up_mean
        roof = run.roofline(gu)
        line = {"mode": "chunk_sweep", "tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
                "gate_up_ms": gu, "gate_up_roofline": roof, "steps": steps,
                "config": workload_desc(shape, thr, pairs)}
        log(f"[sweep] T={T}: {ms:.3f} ms/step, {T / ms * 1e3:.0f} tok/s, gate/up {gu:.3f} ms "
            f"({roof['bound']}, {100 * roof['frac']:.1f}% of peak)")
        print(json.dumps(line), flush=True)
        del run
        torch.cuda.empty_cache()


def multilayer_decode(n_layers, batches, steps, seed, thr):
    """Decode through n_layers independent layers of 3-bit experts (weights
    generated on the device: random codes with the unused bits cleared, fp16
    scales in [0.001, 0.01]), eager and as one captured graph per batch size.
    Each layer has its own router logits (Zipf-biased) and input rows; the
    layers are not chained (the MoE part is timed, not the rest of a block)."""
    import numpy as np
    import torch

    import routed_expert_ffn_03_amd as moe
    from moe_inputs import LayerShape, routing_inputs

    H, I, E, k = 4096, 2048, 384, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    # unused bits: 30-31 of words 0..11, 24-31 of word 12
    mask = torch.tensor([0x3FFFFFFF] * 12 + [0x00FFFFFF], dtype=torch.int32, device="cuda")

    def q3_matrix(n_out, n_in):
        w = torch.randint(-2 ** 31, 2 ** 31 - 1, (E, n_out, n_in // 128, 13), dtype=torch.int32, device="cuda",
                          generator=gen)
        w &= mask
        s = (torch.rand((E, n_out, n_in // 128), device="cuda", generator=gen) * 0.009 + 0.001).half()
        return w, s.view(torch.int16)

    t0 = time.perf_counter()
    layers = []
    for _ in range(n_layers):
        (gw, gs), (uw, us), (dw, ds) = q3_matrix(I, H), q3_matrix(I, H), q3_matrix(H, I)
        layers.append({"gate": gw, "up": uw, "down": dw, "gate_scale": gs, "up_scale": us, "down_scale": ds})
    torch.cuda.synchronize()
    wbytes = sum(t.numel() * t.element_size() for L in layers for t in L.values())
    log(f"[multilayer] {n_layers} layers of 3-bit experts ({wbytes / 1e9:.1f} GB) generated in "
        f"{time.perf_counter() - t0:.1f} s")
    per_expert = 2 * I * (H // 128) * (13 * 4 + 2) + H * (I // 128) * (13 * 4 + 2)
    results = []
    for T in batches:
        shape = LayerShape(f"decode{T}_q3", T, H, I, E, k, "zipf", "q3")
        bufs, ins, touched = [], [], 0
        for li in range(n_layers):
            lg, x = routing_inputs(shape, seed * 1000 + li)
            ins.append((torch.from_numpy(lg).cuda(), torch.from_numpy(x.view(np.int16)).cuda()))
            bufs.append(moe.MoELayerBuffers(T, E, k, H, I, moe.MOE_WFMT_Q3G128))

        def step():
            for li in range(n_layers):
                bufs[li].forward(ins[li][0], ins[li][1], layers[li], fat_threshold=thr)

        for _ in range(3):
            step()
        torch.cuda.synchronize()
        touched = sum(int((b.expert_counts > 0).sum().item()) for b in bufs)
        a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            step()
        b2.record()
        torch.cuda.synchronize()
        eager_ms = a.elapsed_time(b2) / steps
        eager_out = [b.out.clone() for b in bufs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(b.out, o) for b, o in zip(bufs, eager_out))
        a.record()
        for _ in range(steps):
            graph.replay()
        b2.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b2) / steps
        gbs = touched * per_expert / (graph_ms * 1e-3) / 1e9
        r = {"batch": T, "eager_ms": eager_ms, "graph_ms": graph_ms, "graph_us_per_layer": graph_ms * 1e3 / n_layers,
             "launch_overhead_us_per_layer": (eager_ms - graph_ms) * 1e3 / n_layers,
             "tokens_per_s_graph": T / (graph_ms * 1e-3), "touched_experts_per_layer": touched / n_layers,
             "touched_weight_GBps": gbs, "hbm_frac": gbs / PEAK_HBM_GBS, "graph_equals_eager": same}
        log(f"[multilayer] T={T}: eager {eager_ms:.3f} ms, graph {graph_ms:.3f} ms for {n_layers} layers "
            f"({r['graph_us_per_layer']:.1f} us/layer, {touched / n_layers:.1f} experts/layer, "
            f"{gbs:.0f} GB/s of touched weights), replay == eager: {same}")
        results.append(r)
        del graph, bufs
        torch.cuda.empty_cache()
    print(json.dumps({"mode": "multilayer_decode", "layers": n_layers, "expert_weights": "q3",
                      "weights_GB": wbytes / 1e9, "steps": steps, "data": "synthetic (device-generated codes)",
                      "results": results}), flush=True)


def router_bench(seed, steps):
    """The fused router (x . W_router^T on MFMA, then the top-k gate) on the
    hidden states of the 16k and decode workloads, 384 experts, top-8; the
    time of the gate alone on given logits (moe_route_topk) beside it."""
    import numpy as np
    import torch

    import routed_expert_ffn_03_amd as moe
    from moe_inputs import SHAPES, router_weights, routing_inputs

    res = []
    for name in ("prefill16k", "decode"):
        s = SHAPES[name]
        _, x = routing_inputs(s, seed)
        dx = torch.from_numpy(x.view(np.int16)).cuda()
        dw = torch.from_numpy(router_weights(s.E, s.H, seed).view(np.int16)).cuda()
        ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
        tw = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
        cnt = torch.empty((s.E,), dtype=torch.int32, device="cuda")
        lg = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
        n = steps if s.T > 64 else 10 * steps

        def timed(fn):
            for _ in range(3):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n

        ws = torch.empty(s.T * s.E * 4, dtype=torch.uint8, device="cuda")
        fused = timed(lambda: moe.moe_router_topk(dx, dw, s.k, ids, tw, cnt))
        fused_ws = timed(lambda: moe.moe_router_topk(dx, dw, s.k, ids, tw, cnt, workspace=ws))
        with_logits = timed(lambda: moe.moe_router_topk(dx, dw, s.k, ids, tw, cnt, logits=lg))
        gate_only = timed(lambda: moe.moe_route_topk(lg, s.k, ids, tw, cnt))
        flops = 2.0 * s.T * s.E * s.H
        r = {"workload": name, "tokens": s.T, "experts": s.E, "hidden": s.H, "top_k": s.k,
             "fused_ms": fused, "fused_with_workspace_ms": fused_ws, "with_logits_ms": with_logits,
             "gate_on_given_logits_ms": gate_only,
             "fused_tflops": flops / (fused * 1e-3) / 1e12,
             "fused_mfma_frac": flops / (fused * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS["bf16"]}
        log(f"[router] {name}: fused {fused * 1e3:.1f} us ({r['fused_tflops']:.0f} TFLOP/s), with a workspace "
            f"{fused_ws * 1e3:.1f} us, with logits out "
            f"{with_logits * 1e3:.1f} us, gate alone on given logits {gate_only * 1e3:.1f} us")
        res.append(r)
    print(json.dumps({"mode": "router", "data": "synthetic", "results": res}), flush=True)


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def moe_lib_check():
    import routed_expert_ffn_03_amd as moe
    moe.lib()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only: the layer runs on a single MI355X "
                                   "with no collectives; run with --gpus 1"}), flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.sweep:
        moe_lib_check()
        chunk_sweep([int(v) for v in args.sweep.split(",")], args.seed, args.fat_threshold, args.layout == "pairs")
        return
    if args.router:
        moe_lib_check()
        router_bench(args.seed, args.steps)
        return
    if args.multilayer_decode:
        moe_lib_check()
        multilayer_decode(args.multilayer_decode, [int(v) for v in args.batches.split(",")], args.steps,
                          args.seed, args.fat_threshold)
        return

    import routed_expert_ffn_03_amd as moe
    from moe_inputs import SHAPES
    from moe_inputs.device import upload_weights

    moe.lib()
    shape = SHAPES[args.workload]
    t0 = time.perf_counter()
    dev_w = upload_weights(shape, args.seed)
    log(f"[bench] weights for {shape.name} generated and uploaded in {time.perf_counter() - t0:.1f} s")
    pairs = shape.wfmt == "bf16" and args.layout == "pairs"
    if pairs:
        dev_w = pack_pairs(dev_w)

    flush = None if args.no_flush else torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda")
    run = Runner(shape, args.seed, dev_w, args.fat_threshold, pairs)
    st = run.measure(args.steps, args.warmup, flush)
    ms, gu_ms = st.mean, st.gate_up_mean
    roof = run.roofline(gu_ms)
    log(f"[bench] {shape.name}: {ms:.3f} ms/step (median {st.stats()['median_ms']:.3f}, p10 "
        f"{st.stats()['p10_ms']:.3f}, p90 {st.stats()['p90_ms']:.3f}), gate/up {gu_ms:.3f} ms, "
        f"{roof['achieved']:.1f} {roof['unit']} ({100 * roof['frac']:.1f}% of peak)")
    res = {
        "metric": METRIC, "value": shape.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": shape.wfmt, "data": "synthetic",
        "config": workload_desc(shape, args.fat_threshold, pairs), "roofline": roof,
        "timing": {**st.stats(), "mall_flush_bytes": 0 if flush is None else FLUSH_BYTES,
                   "method": "HIP events around each layer call on the library's stream (the gate/up phase timed "
                             "in a second run of the same steps); a 512 MiB scratch buffer is read between "
                             "steps outside the events"},
    }
    if shape.T <= 64:
        res["layer_roofline"] = run.layer_hbm(ms)
    if not args.no_decode and not args.workload.startswith("decode"):
        # the 4-token decode step on the same weights (same format, same layer)
        dshape = SHAPES["decode" if shape.wfmt == "bf16" else "decode_q3"]
        drun = Runner(dshape, args.seed, dev_w, args.fat_threshold, pairs)
        dst = drun.measure(args.decode_steps, 20, flush)
        dms, dgu = dst.mean, dst.gate_up_mean
        droof = drun.roofline(dgu)
        dlayer = drun.layer_hbm(dms)
        log(f"[bench] decode: {dms * 1e3:.1f} us/step (median {dst.stats()['median_ms'] * 1e3:.1f}), gate/up "
            f"{dgu * 1e3:.1f} us, {droof['achieved']:.1f} {droof['unit']} ({100 * droof['frac']:.1f}% of peak); "
            f"whole layer {dlayer['achieved']:.0f} GB/s ({100 * dlayer['frac']:.1f}%)")
        res["decode"] = {"value": dshape.T / (dms * 1e-3), "unit": "tokens/s", "ms_per_step": dms,
                         "steps": args.decode_steps, "config": workload_desc(dshape, args.fat_threshold, pairs),
                         "roofline": droof, "layer_roofline": dlayer, "timing": dst.stats()}
    if not args.no_cpu_baseline:
        n = min(args.cpu_sample, shape.T)
        res["cpu_baseline"] = cpu_baseline(shape, args.seed, n)
        log(f"[bench] cpu baseline: {res['cpu_baseline']['value']:.3f} tokens/s")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
