"""Synthetic-input recipes: determinism, rounding, and the workload mix.

The workload checks confirm the reading of the Zipf router skew: with the
bias temperature used here the 4-token decode step touches a few dozen
experts, the 1k chunk mixes fat (>= 32 tokens) and thin experts, and in the
16k chunk every expert is fat, matching the described workloads.
"""
import numpy as np
import pytest

import oracle
from moe_inputs import (SHAPES, float32_to_bf16_bits, routing_inputs, expert_weights,
                        expert_weight_q3, layer_weights, LayerShape)


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 1.0 + 2**-8 + 2**-20,
                     -0.0, 3.0e38], dtype=np.float32)
    got = oracle.bf16_to_f64(float32_to_bf16_bits(vals))
    assert got.tolist()[:5] == [1.0, 1.0, 1.0 + 2**-6, -1.0, 1.0 + 2**-7]
    assert np.signbit(got[5]) and got[5] == 0.0


def test_generation_is_deterministic_and_expert_local():
    shape = SHAPES["tiny"]
    a = routing_inputs(shape, 1)
    b = routing_inputs(shape, 1)
    c = routing_inputs(shape, 2)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    assert not np.array_equal(a[0], c[0])
    W = layer_weights(shape, 1)
    e5 = expert_weights(shape, 1, 5)
    for n in ("gate", "up", "down"):
        assert np.array_equal(W[n][5], e5[n])
    assert W["gate"].shape == (16, 128, 256) and W["down"].shape == (16, 256, 128)
    std = oracle.bf16_to_f64(W["gate"]).std()
    assert 0.018 < std < 0.022


def test_q3_words_and_scales():
    shape = LayerShape("q", 4, 256, 128, 3, 2, "normal", "q3")
    words, scales = expert_weight_q3(shape, 0, "gate", 1)
    assert words.shape == (128, 2, 13) and scales.shape == (128, 2)
    assert np.all(words >> 30 == 0) and np.all(words[..., 12] >> 24 == 0)
    fields = oracle.q3_fields(words)
    hist = np.bincount(fields.ravel(), minlength=8) / fields.size
    assert np.all(np.abs(hist - 1 / 8) < 0.01)
    s = oracle.f16_to_f64(scales)
    lo, hi = 0.02 / np.sqrt(5.5) * 0.5, 0.02 / np.sqrt(5.5) * 1.5
    assert s.min() >= lo * 0.999 and s.max() <= hi * 1.001


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_workload_mix(seed):
    thr = 32
    # decode: a few dozen distinct experts out of 32 slots
    lg, _ = routing_inputs(SHAPES["decode"], seed)
    ids, _ = oracle.route_topk(lg, 8)
    assert 20 <= len(np.unique(ids)) <= 32
    # 1k chunk: both fat and thin experts present
    lg, _ = routing_inputs(SHAPES["prefill1k"], seed)
    c = oracle.expert_histogram(oracle.route_topk(lg, 8)[0], 384)
    assert 30 <= (c >= thr).sum() <= 90 and (c[c > 0] < thr).sum() >= 250
    # 16k chunk (Zipf) and the unskewed 3-bit chunk: every expert is fat
    for name in ("prefill16k", "prefill16k_q3"):
        lg, _ = routing_inputs(SHAPES[name], seed)
        c = oracle.expert_histogram(oracle.route_topk(lg, 8)[0], 384)
        assert c.sum() == 16384 * 8 and c.min() >= thr
