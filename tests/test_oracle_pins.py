"""Pins of the float64 oracle against things other than itself.

Each test checks the oracle against a hand-worked fixture (tests/golden), a
brute-force evaluation written independently here, a closed form, an
invariant, or a special case that reduces to a library routine (torch's
float64 SiLU / linear on CPU).  No GPU is used.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import LayerShape, SHAPES, float32_to_bf16_bits, routing_inputs, layer_weights
from tests.golden_io import lines, ints

TINY = SHAPES["tiny"]


def _raw_from_layer(W):
    return lambda e: {name: arr[e] for name, arr in W.items()}


# ------------------------------------------------------------------ route

def test_route_worked_cases():
    n = 0
    for key, val in lines("route_worked.txt"):
        assert key == "case"
        lg, k, ids, w = [s.strip() for s in val.split("|")]
        logits = np.array([[float(v) for v in lg.split()]], dtype=np.float32)
        got_ids, got_w = oracle.route_topk(logits, int(k))
        assert got_ids[0].tolist() == [int(v) for v in ids.split()]
        np.testing.assert_allclose(got_w[0], [float(v) for v in w.split()], rtol=0, atol=1e-15)
        n += 1
    assert n >= 6


def _brute_topk(row, k):
    # independent rule: Python's sort on (-value, index); -0.0 == 0.0 in float compare
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("k", [1, 2, 5, 16])
def test_route_brute_force_with_ties(seed, k):
    rng = np.random.default_rng(100 + seed)
    T, E = 40, 16
    # quarter-integer logits create many exact ties; sprinkle signed zeros
    logits = (np.round(rng.standard_normal((T, E)) * 4) / 4).astype(np.float32)
    logits[rng.random((T, E)) < 0.1] = np.float32(-0.0)
    logits[rng.random((T, E)) < 0.1] = np.float32(0.0)
    ids, w = oracle.route_topk(logits, k)
    for t in range(T):
        assert ids[t].tolist() == _brute_topk(logits[t], k)
        sel = logits[t, ids[t]].astype(np.float64)
        assert len(set(ids[t].tolist())) == k
        assert np.all(np.diff(sel) <= 0)
        kth = sel[-1]
        for e in range(E):
            if e in ids[t]:
                continue
            assert logits[t, e] <= kth
            if logits[t, e] == kth:
                assert e > ids[t][-1]
        # weights: closed form against math.exp, sum, monotone
        z = [math.exp(float(v) - float(sel[0])) for v in sel]
        np.testing.assert_allclose(w[t], [v / sum(z) for v in z], rtol=1e-15, atol=0)
        assert abs(w[t].sum() - 1.0) < 1e-15
        assert np.all(np.diff(w[t]) <= 0)


def test_route_special_weights():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((10, 12)).astype(np.float32)
    _, w1 = oracle.route_topk(logits, 1)
    assert np.all(w1 == 1.0)
    eq = np.full((3, 12), 0.75, dtype=np.float32)
    ids, w = oracle.route_topk(eq, 5)
    assert np.all(w == 0.2) and ids.tolist() == [[0, 1, 2, 3, 4]] * 3


def test_route_rejects_non_finite():
    bad = np.zeros((2, 4), np.float32)
    bad[1, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.route_topk(bad, 2)
    bad[1, 2] = np.inf
    with pytest.raises(ValueError):
        oracle.route_topk(bad, 2)


# ---------------------------------------------------------------- permute

def test_permute_worked():
    d = dict(lines("permute_worked.txt"))
    ids = np.array(ints(d["ids"]), dtype=np.int32).reshape(3, 2)
    counts, offsets, sp, p2s = oracle.permute(ids, 4)
    assert counts.tolist() == ints(d["counts"])
    assert offsets.tolist() == ints(d["offsets"])
    assert sp.tolist() == ints(d["sorted_pair"])
    assert p2s.tolist() == ints(d["pair_to_sorted"])


@pytest.mark.parametrize("seed", [0, 1])
def test_permute_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, E, k = 57, 11, 3
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, sp, p2s = oracle.permute(ids, E)
    # independent bucket lists in pair order
    buckets = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            buckets[ids[t, j]].append(t * k + j)
    assert sp.tolist() == [p for b in buckets for p in b]
    assert counts.tolist() == [len(b) for b in buckets]
    assert offsets[0] == 0 and offsets[-1] == T * k and counts.sum() == T * k
    assert np.all(p2s[sp] == np.arange(T * k)) and np.all(sp[p2s] == np.arange(T * k))
    # every sorted row of expert e holds a pair routed to e, token ascending
    for e in range(E):
        rows = sp[offsets[e]:offsets[e + 1]]
        assert np.all(ids.ravel()[rows] == e) and np.all(np.diff(rows // k) > 0)
    # gather rows by sorted_pair, scatter back by pair_to_sorted: identity
    x = rng.integers(0, 1 << 16, size=(T, 5), dtype=np.uint16)
    gathered = x[sp // k]
    assert np.array_equal(gathered[p2s].reshape(T, k, 5), np.repeat(x[:, None, :], k, axis=1))


# ------------------------------------------------------------- expert FFN

def _bf16_exact(vals):
    a = np.asarray(vals, dtype=np.float32)
    bits = float32_to_bf16_bits(a)
    assert np.array_equal(oracle.bf16_to_f64(bits), a.astype(np.float64)), "fixture value not bf16-exact"
    return bits


def test_swiglu_worked_and_layer():
    experts = []
    layer = {}
    for key, val in lines("swiglu_worked.txt"):
        if key == "expert":
            x, wg, wu, wd, y = [np.array([float(v) for v in s.split()]) for s in val.split("|")]
            H, I = len(x), len(wg) // len(x)
            got = oracle.expert_ffn(x[None, :], wg.reshape(I, H), wu.reshape(I, H), wd.reshape(H, I))
            np.testing.assert_allclose(got[0], y, rtol=1e-15, atol=0)
            experts.append((x, wg.reshape(I, H), wu.reshape(I, H), wd.reshape(H, I)))
        else:
            layer[key] = np.array([float(v) for v in val.split()])
    x = _bf16_exact(experts[0][0])[None, :]
    mats = [experts[0][1:], experts[2][1:]]
    raw = lambda e: {n: _bf16_exact(m) for n, m in zip(("gate", "up", "down"), mats[e])}
    logits = layer["layer_logits"].astype(np.float32)[None, :]
    res = oracle.moe_layer(logits, x, raw, 2)
    np.testing.assert_allclose(res["out"][0], layer["layer_out"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(oracle.dense_layer(logits, x, raw, 2)[0], layer["layer_out"], rtol=1e-15)


def test_single_expert_reduces_to_torch_swiglu():
    shape = LayerShape("one", 9, 64, 32, 1, 1)
    logits, x = routing_inputs(shape, 3)
    W = layer_weights(shape, 3)
    res = oracle.moe_layer(logits, x, _raw_from_layer(W), 1)
    assert np.all(res["w"] == 1.0)
    xt = torch.from_numpy(oracle.bf16_to_f64(x))
    wg, wu, wd = (torch.from_numpy(oracle.bf16_to_f64(W[n][0])) for n in ("gate", "up", "down"))
    F = torch.nn.functional
    ref = F.linear(F.silu(F.linear(xt, wg)) * F.linear(xt, wu), wd).numpy()
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-15)


def test_identical_experts_give_plain_ffn():
    shape = LayerShape("same", 20, 64, 32, 6, 3)
    logits, x = routing_inputs(shape, 5)
    W = layer_weights(shape, 5)
    for n in W:
        W[n][:] = W[n][0]
    out = oracle.moe_layer(logits, x, _raw_from_layer(W), 3)["out"]
    mats = oracle.expert_matrices({n: W[n][0] for n in W})
    ref = oracle.expert_ffn(oracle.bf16_to_f64(x), *mats)
    assert oracle.rel_max_err(out, ref) < 1e-13


def test_zero_input_and_down_scaling():
    shape = LayerShape("lin", 12, 64, 32, 5, 2)
    logits, x = routing_inputs(shape, 9)
    W = layer_weights(shape, 9)
    raw = _raw_from_layer(W)
    zero = np.zeros_like(x)
    assert np.all(oracle.moe_layer(logits, zero, raw, 2)["out"] == 0.0)
    base = oracle.moe_layer(logits, x, raw, 2)["out"]
    W2 = dict(W)
    W2["down"] = float32_to_bf16_bits(oracle.bf16_to_f64(W["down"]).astype(np.float32) * 2)
    doubled = oracle.moe_layer(logits, x, _raw_from_layer(W2), 2)["out"]
    assert np.array_equal(doubled, 2 * base)


@pytest.mark.parametrize("wfmt", ["bf16", "q3"])
def test_dense_brute_force_matches_grouped(wfmt):
    shape = LayerShape("tiny", TINY.T, TINY.H, TINY.I, TINY.E, TINY.k, "normal", wfmt)
    logits, x = routing_inputs(shape, 0)
    W = layer_weights(shape, 0)
    raw = _raw_from_layer(W)
    res = oracle.moe_layer(logits, x, raw, shape.k)
    dense = oracle.dense_layer(logits, x, raw, shape.k)
    assert oracle.rel_max_err(res["out"], dense) < 1e-12
    assert np.abs(res["out"]).max() > 0


def test_sampled_tokens_equal_full_layer():
    shape = LayerShape("s", 30, 64, 32, 7, 2, "zipf")
    logits, x = routing_inputs(shape, 4)
    raw = _raw_from_layer(layer_weights(shape, 4))
    full = oracle.moe_layer(logits, x, raw, 2)
    toks = [0, 7, 29]
    part = oracle.moe_layer(logits, x, raw, 2, tokens=toks)
    # BLAS may round differently for a different row count: equal to 1e-14
    assert oracle.rel_max_err(part["out"], full["out"][toks]) < 1e-14
    assert np.all(np.isnan(part["Y"]).sum(axis=1) % shape.H == 0)


# -------------------------------------------------------------------- Q3

def test_q3_worked_words():
    n = 0
    for key, val in lines("q3_words.txt"):
        if key != "word":
            continue
        w, fields = val.split("|")
        words = np.zeros(13, np.uint32)
        words[0] = int(w, 16)
        got = oracle.q3_fields(words)
        assert got[:10].tolist() == [int(v) for v in fields.split()]
        assert np.all(got[10:] == 0)
        n += 1
    assert n >= 5
    d = dict(lines("q3_words.txt"))
    words = np.array(ints(d["group_words"]), np.uint32)[None, None, :]
    sc = np.array([[int(d["group_scale"], 16)]], np.uint16)
    assert np.all(oracle.q3_dequant(words, sc) == float(d["group_value"]))
    words = np.array(ints(d["onehot_words"]), np.uint32)[None, None, :]
    vals = oracle.q3_dequant(words, sc)[0]
    i = int(d["onehot_index"])
    assert vals[i] == float(d["onehot_value"])
    assert np.all(np.delete(vals, i) == float(d["onehot_rest"]))


def test_q3_pack_round_trip_and_bitwise_decode():
    rng = np.random.default_rng(11)
    fields = rng.integers(0, 8, size=(3, 4, 128), dtype=np.uint8)
    words = oracle.q3_pack(fields)
    assert np.array_equal(oracle.q3_fields(words), fields)
    assert np.all(words[..., :12] >> 30 == 0) and np.all(words[..., 12] >> 24 == 0)
    # independent decode: walk the bit stream one bit at a time
    for n in range(3):
        for g in range(4):
            for f in range(128):
                wi, pos = divmod(f, 10)
                v = sum(((int(words[n, g, wi]) >> (3 * pos + b)) & 1) << b for b in range(3))
                assert v == fields[n, g, f]
    scales = np.float16(rng.uniform(0.001, 0.01, size=(3, 4))).view(np.uint16)
    deq = oracle.q3_dequant(words, scales)
    ref = (fields.astype(np.float64) - 4) * scales.view(np.float16).astype(np.float64)[..., None]
    assert np.array_equal(deq, ref.reshape(3, 512))


def test_router_logits_closed_forms():
    """Router logits: a one-hot hidden state picks one column of W_router; the
    map is linear in x; a hand-worked 2 x 3 case."""
    rng = np.random.default_rng(5)
    E, H = 8, 16
    w = float32_to_bf16_bits((rng.standard_normal((E, H)) * 0.25).astype(np.float32))
    wv = oracle.bf16_to_f64(w)
    for h in (0, 7, 15):
        x = np.zeros((1, H), dtype=np.float32)
        x[0, h] = 1.0
        got = oracle.router_logits(float32_to_bf16_bits(x), w)
        assert np.array_equal(got[0], wv[:, h])
    a = float32_to_bf16_bits(rng.standard_normal((3, H)).astype(np.float32))
    b = float32_to_bf16_bits(rng.standard_normal((3, H)).astype(np.float32))
    la, lb = oracle.router_logits(a, w), oracle.router_logits(b, w)
    # x values are bf16-exact; 2 * a is exact too
    a2 = float32_to_bf16_bits((2 * oracle.bf16_to_f64(a)).astype(np.float32))
    assert np.allclose(oracle.router_logits(a2, w), 2 * la, rtol=0, atol=1e-12)
    assert la.shape == (3, E) and lb.shape == (3, E)
    # hand-worked: x = [1, 2], W = [[1, 0], [0.5, -1], [-2, 0.25]] -> [1, -1.5, -1.5]
    x = float32_to_bf16_bits(np.array([[1.0, 2.0]], dtype=np.float32))
    W = float32_to_bf16_bits(np.array([[1.0, 0.0], [0.5, -1.0], [-2.0, 0.25]], dtype=np.float32))
    assert np.array_equal(oracle.router_logits(x, W), np.array([[1.0, -1.5, -1.5]]))
    # and the gate on top of it breaks the tie between experts 1 and 2 by index
    ids, _ = oracle.route_topk(oracle.router_logits(x, W).astype(np.float32), 2)
    assert ids.tolist() == [[0, 1]]


# ------------------------------------------------- parity metric, histogram

def test_rel_max_err_worked_values():
    n = 0
    for key, val in lines("metric_worked.txt"):
        if key != "metric":
            continue
        got, ref, shp, want = [s.strip() for s in val.split("|")]
        shape = tuple(int(v) for v in shp.split())
        g = np.array([float(v) for v in got.split()]).reshape(shape)
        r = np.array([float(v) for v in ref.split()]).reshape(shape)
        assert oracle.rel_max_err(g, r) == pytest.approx(float(want), rel=1e-15, abs=0)
        # symmetric in the sign of the error, and scale-free
        assert oracle.rel_max_err(2 * r - g, r) == pytest.approx(float(want), rel=1e-15, abs=0)
        if np.any(r):
            assert oracle.rel_max_err(8 * g, 8 * r) == pytest.approx(float(want), rel=1e-15, abs=0)
        n += 1
    assert n >= 4


def test_expert_histogram_worked_values():
    n = 0
    for key, val in lines("metric_worked.txt"):
        if key != "hist":
            continue
        E, ids, k, counts = [s.strip() for s in val.split("|")]
        a = np.array(ints(ids), dtype=np.int32).reshape(-1, int(k))
        got = oracle.expert_histogram(a, int(E))
        assert got.dtype == np.int32 and got.shape == (int(E),)
        assert got.tolist() == ints(counts)
        n += 1
    assert n >= 3
    # against the permutation's own counts (an independent bucket walk is in
    # test_permute_brute_force): same totals on a random routing
    rng = np.random.default_rng(12)
    ids = np.stack([rng.choice(9, size=3, replace=False) for _ in range(40)]).astype(np.int32)
    buckets = [0] * 12
    for e in ids.ravel():
        buckets[int(e)] += 1
    assert oracle.expert_histogram(ids, 12).tolist() == buckets
