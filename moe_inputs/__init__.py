"""Seeded synthetic inputs for the routed-expert layer.

This module is shared by the oracle-side tests and the GPU-side tests and
benchmark. It only *draws* inputs; it holds none of the layer's arithmetic
(no routing, sorting, matrix products, activation or quantised decoding).

Workload shapes follow the layer served on the pages: 384 routed experts per
MoE layer (dsv41-flash-offload wiki, opening paragraph), prefill chunks of
16,384 tokens (recipe page "DeepSeek-V4.1-Flash / RTX 3090", step 5 launch
flags) and the 1,024-token chunks it replaced (wiki, paragraph on PCIe being
the bottleneck).  Everything else about the synthetic data (hidden and
intermediate sizes, top-8, value distributions, the Zipf skew of the router,
the 3-bit grouped format) is this library's own reading because the pages
publish no weights or layer sizes.

Value recipes (all exact and reproducible from ``seed``):

* router logits  : float32( N(0,1) + bias_e ), drawn and summed in float64 and
                   rounded once to float32.  ``bias_e = beta * ln p(rank_e)``,
                   ``p(r) = r^-s / sum_{r'<=E} r'^-s`` (Zipf, s = 1.1,
                   beta = 0.4), ``rank_e = perm[e] + 1`` for a seeded
                   permutation ``perm``; bias = 0 for the unskewed router.
* activations x  : bf16_rne( float32 N(0,1) ), shape [T, H].
* bf16 weights   : bf16_rne( float32(0.02) * float32 N(0,1) ), stored
                   [E, out, in] (the reduction index contiguous):
                   gate, up: [E, I, H]; down: [E, H, I].
* 3-bit weights  : per (expert, output row, 128-wide group of the reduction
                   index) 13 uint32 words of uniformly random bits, bits 30-31
                   of every word and bits 24-31 of the 13th word cleared, so
                   each of the 128 three-bit fields is uniform over its 8
                   values; one fp16 scale per group,
                   fp16( 0.02/sqrt(5.5) * U[0.5, 1.5) ).

Draw order: the top-level generator ``default_rng(seed)`` draws the Zipf
permutation (skewed router only), then the logits, then x.  Each expert's
weight tensors come from their own generator seeded with
``[seed, tensor_tag, expert]`` so any subset of experts can be regenerated
on its own, in parallel, without materialising the whole layer.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

ZIPF_S = 1.1
ZIPF_BETA = 0.4
WEIGHT_STD = 0.02
Q3_GROUP = 128
Q3_WORDS = 13            # 12 words of 10 fields + 1 word of 8 fields = 128
TAG_BF16 = {"gate": 1000, "up": 1001, "down": 1002}
TAG_Q3 = {"gate": 2000, "up": 2001, "down": 2002}


@dataclass(frozen=True)
class LayerShape:
    """One synthetic workload: tokens, hidden, intermediate, experts, top-k."""
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    router: str = "normal"     # "normal" | "zipf"
    wfmt: str = "bf16"         # "bf16" | "q3"

    @property
    def P(self) -> int:
        return self.T * self.k

    def with_tokens(self, T: int) -> "LayerShape":
        return LayerShape(self.name, T, self.H, self.I, self.E, self.k, self.router, self.wfmt)


# The workloads: a tiny layer for exhaustive parity, a 4-token decode step,
# 1k and 16k prefill chunks (Zipf-skewed router), the 16k chunk with 3-bit
# grouped weights under an unskewed router, and the 4-token decode step on the
# same 3-bit weights (Zipf router as the bf16 decode step).
SHAPES = {
    "tiny": LayerShape("tiny", 64, 256, 128, 16, 2, "normal", "bf16"),
    "decode": LayerShape("decode", 4, 4096, 2048, 384, 8, "zipf", "bf16"),
    "prefill1k": LayerShape("prefill1k", 1024, 4096, 2048, 384, 8, "zipf", "bf16"),
    "prefill16k": LayerShape("prefill16k", 16384, 4096, 2048, 384, 8, "zipf", "bf16"),
    "prefill16k_q3": LayerShape("prefill16k_q3", 16384, 4096, 2048, 384, 8, "normal", "q3"),
    "decode_q3": LayerShape("decode_q3", 4, 4096, 2048, 384, 8, "zipf", "q3"),
}


def float32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite, so the carry into the exponent cannot overflow.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).copy()
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def zipf_bias(E: int, perm: np.ndarray, s: float = ZIPF_S, beta: float = ZIPF_BETA) -> np.ndarray:
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    return beta * np.log(p[perm])          # expert e gets rank perm[e] + 1


def routing_inputs(shape: LayerShape, seed: int):
    """Return (logits float32 [T,E], x bf16 bits uint16 [T,H])."""
    rng = np.random.default_rng(seed)
    if shape.router == "zipf":
        perm = rng.permutation(shape.E)
        bias = zipf_bias(shape.E, perm)
    elif shape.router == "normal":
        bias = np.zeros(shape.E)
    else:
        raise ValueError(shape.router)
    logits = (rng.standard_normal((shape.T, shape.E)) + bias[None, :]).astype(np.float32)
    x = float32_to_bf16_bits(rng.standard_normal((shape.T, shape.H), dtype=np.float32))
    return logits, x


def _out_in(shape: LayerShape, which: str):
    return (shape.I, shape.H) if which in ("gate", "up") else (shape.H, shape.I)


def expert_weight_bf16(shape: LayerShape, seed: int, which: str, e: int) -> np.ndarray:
    """bf16 bits, shape [out, in], of one expert's gate/up/down matrix."""
    n_out, n_in = _out_in(shape, which)
    rng = np.random.default_rng([seed, TAG_BF16[which], e])
    w = rng.standard_normal(n_out * n_in, dtype=np.float32)
    w *= np.float32(WEIGHT_STD)
    return float32_to_bf16_bits(w).reshape(n_out, n_in)


def expert_weight_q3(shape: LayerShape, seed: int, which: str, e: int):
    """(words uint32 [out, in/128, 13], scales fp16 bits uint16 [out, in/128])."""
    n_out, n_in = _out_in(shape, which)
    if n_in % Q3_GROUP:
        raise ValueError("reduction size must be a multiple of 128 for 3-bit groups")
    g = n_in // Q3_GROUP
    rng = np.random.default_rng([seed, TAG_Q3[which], e])
    words = rng.integers(0, 1 << 30, size=(n_out, g, Q3_WORDS), dtype=np.uint32)
    words[..., Q3_WORDS - 1] &= np.uint32((1 << 24) - 1)
    sc = (WEIGHT_STD / math.sqrt(5.5)) * rng.uniform(0.5, 1.5, size=(n_out, g))
    scales = sc.astype(np.float16).view(np.uint16)
    return words, scales


def router_weights(E: int, H: int, seed: int) -> np.ndarray:
    """Router matrix [E, H] as bf16 bits: bf16_rne(0.02 * N(0,1)) from its own
    generator, so that with x ~ N(0,1) the logits have a spread near 0.02 * sqrt(H)."""
    rng = np.random.default_rng([seed, 0x7207, E, H])
    return float32_to_bf16_bits((0.02 * rng.standard_normal((E, H))).astype(np.float32))


def expert_weights(shape: LayerShape, seed: int, e: int) -> dict:
    """All weight arrays of expert ``e`` keyed like :func:`layer_weights`."""
    out = {}
    for which in ("gate", "up", "down"):
        if shape.wfmt == "bf16":
            out[which] = expert_weight_bf16(shape, seed, which, e)
        else:
            q, s = expert_weight_q3(shape, seed, which, e)
            out[which] = q
            out[which + "_scale"] = s
    return out


def weight_array_shapes(shape: LayerShape) -> dict:
    """Name -> (full-layer array shape, numpy dtype)."""
    res = {}
    for which in ("gate", "up", "down"):
        n_out, n_in = _out_in(shape, which)
        if shape.wfmt == "bf16":
            res[which] = ((shape.E, n_out, n_in), np.uint16)
        else:
            res[which] = ((shape.E, n_out, n_in // Q3_GROUP, Q3_WORDS), np.uint32)
            res[which + "_scale"] = ((shape.E, n_out, n_in // Q3_GROUP), np.uint16)
    return res


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def for_each_expert(shape: LayerShape, seed: int, fn, experts=None, threads: int | None = None):
    """Generate experts in parallel threads and hand each to ``fn(e, arrays)``.

    ``fn`` is called from worker threads; numpy's generators release the GIL,
    so generation scales with cores while only a few experts are alive.
    """
    experts = range(shape.E) if experts is None else list(experts)
    threads = threads or default_threads()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda e: fn(e, expert_weights(shape, seed, e)), experts))


def layer_weights(shape: LayerShape, seed: int, threads: int | None = None) -> dict:
    """Every expert's weights stacked on the host (small shapes or ample RAM)."""
    out = {name: np.empty(shp, dt) for name, (shp, dt) in weight_array_shapes(shape).items()}

    def put(e, arrs):
        for name, a in arrs.items():
            out[name][e] = a

    for_each_expert(shape, seed, put, threads=threads)
    return out
