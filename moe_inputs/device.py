"""Upload the seeded synthetic inputs to GPU memory (torch tensors).

Plumbing only: the arrays are the ones :mod:`moe_inputs` draws; experts are
generated on host threads and copied one by one, so the whole layer never
sits in host memory at once.
"""
from __future__ import annotations

import queue
import threading

import numpy as np
import torch

from . import LayerShape, default_threads, expert_weights, routing_inputs, weight_array_shapes

_TORCH_DTYPE = {np.uint16: torch.int16, np.uint32: torch.int32}


def upload_routing(shape: LayerShape, seed: int, device="cuda"):
    """(logits fp32 [T,E], x as int16 bf16-bits [T,H]) on the device, plus host copies."""
    logits, x = routing_inputs(shape, seed)
    dl = torch.from_numpy(logits).to(device)
    dx = torch.from_numpy(x.view(np.int16)).to(device)
    return dl, dx, logits, x


def upload_weights(shape: LayerShape, seed: int, device="cuda", threads: int | None = None) -> dict:
    """Every expert's weights on the device; 16-bit patterns as int16, 3-bit words as int32."""
    out = {}
    for name, (shp, dt) in weight_array_shapes(shape).items():
        out[name] = torch.empty(shp, dtype=_TORCH_DTYPE[dt], device=device)
    q: queue.Queue = queue.Queue(maxsize=2 * (threads or default_threads()))
    n_threads = threads or default_threads()
    next_e = iter(range(shape.E))
    lock = threading.Lock()

    def worker():
        while True:
            with lock:
                e = next(next_e, None)
            if e is None:
                q.put(None)
                return
            q.put((e, expert_weights(shape, seed, e)))

    ts = [threading.Thread(target=worker, daemon=True) for _ in range(n_threads)]
    for t in ts:
        t.start()
    done = 0
    while done < n_threads:
        item = q.get()
        if item is None:
            done += 1
            continue
        e, arrs = item
        for name, a in arrs.items():
            out[name][e].copy_(torch.from_numpy(a.view(np.int16 if a.dtype == np.uint16 else np.int32)))
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    return out
