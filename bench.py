#!/usr/bin/env python3
"""Throughput of the routed-expert layer on one MI355X.

One step = one full layer call (route -> permute -> plan -> gate/up -> down
-> combine) over one batch of synthetic inputs already resident in HBM.
The headline workload is the 16,384-token prefill chunk (bf16 experts,
Zipf-skewed router); the 4-token decode step is measured in the same run on
the same weights and reported under "decode" (with --workload prefill16k_q3:
the decode step on the same 3-bit weights).  The dominant kernel's time
(the gate/up phase) is taken live with HIP events on the library's stream.

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


def ffn_source_hash() -> str:
    import hashlib
    src = os.path.join(ROOT, "routed_expert_ffn_03_amd", "csrc", "ffn.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:12]


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
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="prefill16k",
                   choices=["prefill16k", "decode", "prefill1k", "prefill16k_q3", "decode_q3"])
    p.add_argument("--decode-steps", type=int, default=200, help="steps of the secondary decode measurement")
    p.add_argument("--no-decode", action="store_true", help="skip the secondary decode measurement")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=128, help="tokens of the batch the oracle is timed on")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--fat-threshold", type=int, default=32)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (HBM counter calibration)")
    return p.parse_args()


def workload_desc(shape, thr):
    router = "Zipf(s=1.1) bias, beta=0.4" if shape.router == "zipf" else "N(0,1), no skew"
    return {
        "workload": f"{shape.name}: routed-expert layer, {shape.T} tokens, hidden {shape.H}, "
                    f"expert inter {shape.I}, {shape.E} experts, top-{shape.k}, {shape.wfmt} experts",
        "tokens": shape.T, "hidden": shape.H, "inter": shape.I, "experts": shape.E, "top_k": shape.k,
        "router": router, "expert_weights": shape.wfmt, "fat_threshold": thr,
    }


class Runner:
    """Buffers of one workload and a step that times the gate/up phase with events."""

    def __init__(self, shape, seed, dev_w, thr):
        import numpy as np
        import torch

        import routed_expert_ffn_03_amd as moe
        from moe_inputs import routing_inputs

        self.moe, self.torch, self.shape, self.w, self.thr = moe, torch, shape, dev_w, thr
        self.logits_np, self.x_np = routing_inputs(shape, seed)
        self.logits = torch.from_numpy(self.logits_np).cuda()
        self.x = torch.from_numpy(self.x_np.view(np.int16)).cuda()
        self.wfmt = 0 if shape.wfmt == "bf16" else 1
        self.b = moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, self.wfmt)

    def step(self, ev=None):
        m, b, s, w = self.moe, self.b, self.shape, self.w
        m.moe_route_topk(self.logits, s.k, b.topk_ids, b.topk_w, b.expert_counts)
        m.moe_permute(b.topk_ids, s.E, b.expert_offsets, b.sorted_pair, b.pair_to_sorted, b.workspace)
        m.moe_ffn_plan(b.expert_offsets, s.T, s.k, s.H, s.I, b.workspace, fat_threshold=self.thr, wfmt=self.wfmt)
        if ev is not None:
            ev[0].record()
        m.moe_ffn_gate_up(self.x, w["gate"], w["up"], b.sorted_pair, s.E, s.k, b.workspace,
                          s_gate=w.get("gate_scale"), s_up=w.get("up_scale"), fat_threshold=self.thr, wfmt=self.wfmt)
        if ev is not None:
            ev[1].record()
        m.moe_ffn_down(w["down"], s.T, s.E, s.k, s.I, b.y_sorted, b.workspace, s_down=w.get("down_scale"),
                       fat_threshold=self.thr, wfmt=self.wfmt)
        m.moe_combine(b.y_sorted, b.topk_w, b.pair_to_sorted, b.out)

    def measure(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gate_up_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
        return (t1 - t0) * 1e3 / steps, gate_up_ms

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
        # fat kernel template arguments: <phase, weight format, LDS ring stages>
        fat_name = "ffn_fat_kernel<1, 0, 5>" if s.wfmt == "bf16" else "ffn_fat_kernel<1, 1, 6>"
        r["kernel"] = f"gate/up phase ({fat_name} + ffn_thin_kernel<1, {0 if s.wfmt == 'bf16' else 1}, w>)"
        r["kernel_ms"] = gate_up_ms
        r["algorithmic"] = per
        r["experts_touched"] = touched
        r["experts_fat"] = fat
        return r


def cpu_baseline(shape, seed, n_tokens):
    """The float64 oracle as it is, on the first n_tokens tokens of the same batch, 1 BLAS thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from moe_inputs import for_each_expert, routing_inputs

    logits, x = routing_inputs(shape, seed)
    logits, x = logits[:n_tokens], x[:n_tokens]
    ids, _ = oracle.route_topk(logits, shape.k)
    need = sorted({int(e) for e in ids.ravel()})
    raw = {}
    for_each_expert(shape, seed, lambda e, a: raw.__setitem__(e, a), experts=need)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.moe_layer(logits, x, lambda e: raw[e], shape.k)
        dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_tokens} tokens of the {shape.name} batch (seed {seed}): route, permute, "
                      f"{len(need)} experts' SwiGLU FFN and combine in float64 numpy, 1 thread; "
                      f"{dt:.1f} s"}


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

    import routed_expert_ffn_03_amd as moe
    from moe_inputs import SHAPES
    from moe_inputs.device import upload_weights

    moe.lib()
    shape = SHAPES[args.workload]
    t0 = time.perf_counter()
    dev_w = upload_weights(shape, args.seed)
    log(f"[bench] weights for {shape.name} generated and uploaded in {time.perf_counter() - t0:.1f} s")

    run = Runner(shape, args.seed, dev_w, args.fat_threshold)
    ms, gu_ms = run.measure(args.steps, args.warmup)
    roof = run.roofline(gu_ms)
    log(f"[bench] {shape.name}: {ms:.3f} ms/step, gate/up {gu_ms:.3f} ms, "
        f"{roof['achieved']:.1f} {roof['unit']} ({100 * roof['frac']:.1f}% of peak)")
    res = {
        "metric": METRIC, "value": shape.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": shape.wfmt, "data": "synthetic",
        "config": workload_desc(shape, args.fat_threshold), "roofline": roof,
    }
    if not args.no_decode and not args.workload.startswith("decode"):
        # the 4-token decode step on the same weights (same format, same layer)
        dshape = SHAPES["decode" if shape.wfmt == "bf16" else "decode_q3"]
        drun = Runner(dshape, args.seed, dev_w, args.fat_threshold)
        dms, dgu = drun.measure(args.decode_steps, 20)
        droof = drun.roofline(dgu)
        log(f"[bench] decode: {dms * 1e3:.1f} us/step, gate/up {dgu * 1e3:.1f} us, "
            f"{droof['achieved']:.1f} {droof['unit']} ({100 * droof['frac']:.1f}% of peak)")
        res["decode"] = {"value": dshape.T / (dms * 1e-3), "unit": "tokens/s", "ms_per_step": dms,
                         "steps": args.decode_steps, "config": workload_desc(dshape, args.fat_threshold),
                         "roofline": droof}
    if not args.no_cpu_baseline:
        n = min(args.cpu_sample, shape.T)
        res["cpu_baseline"] = cpu_baseline(shape, args.seed, n)
        log(f"[bench] cpu baseline: {res['cpu_baseline']['value']:.3f} tokens/s")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
