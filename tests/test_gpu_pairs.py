"""The row-pair weight format (MOE_WFMT_BF16_PAIRS) on the GPU.

``moe_pack_bf16_pairs`` is a permutation of 16-bit values, optionally with a
bf16 -> fp16 conversion toward zero: it is checked bit for bit against the
layout written out with numpy reshapes and the conversion written out with
numpy's float16 (a round-to-nearest step taken back toward zero where it went
away).  The layer with packed weights (W_down converted to fp16, as the
format stores it) does the same arithmetic in the same order as with plain
bf16 weights -- the plain path converts W_down with the same instruction
after loading it -- so every output must equal the plain layer's bit for bit;
the small layers are also compared with the float64 oracle at the bf16 bar
(max|err| / rms(ref) <= 1e-2).
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_03_amd as moe
from moe_inputs import SHAPES, LayerShape, layer_weights, routing_inputs
from tests.gpu_util import TOL_BF16, check_indices, host_raw, parity_line, run_layer, say, to_dev_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    yield


def pairs_layout(a: np.ndarray) -> np.ndarray:
    """[mats, rows, cols] -> the row-pair layout, as a flat array: rows 2p
    and 2p+1 alternate every 32 columns."""
    m, r, c = a.shape
    return a.reshape(m, r // 2, 2, c // 32, 32).transpose(0, 1, 3, 2, 4).reshape(-1)


def bf16_to_f16_toward_zero(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp16 bit patterns, rounded toward zero (finite fp16
    results saturate at 65504; infinities and zeros keep their sign)."""
    f = (bits.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        h = f.astype(np.float16)
    away = np.abs(h.astype(np.float64)) > np.abs(f)
    h = np.where(away, np.nextafter(h, np.float16(0)), h)
    return h.astype(np.float16).view(np.uint16)


def packed(w: dict) -> dict:
    out = {}
    for n, t in w.items():
        d = torch.empty_like(t)
        moe.moe_pack_bf16_pairs(t, d, to_fp16=(n == "down"))
        out[n] = d
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("shape", [(1, 2, 32), (3, 6, 64), (2, 256, 4096), (5, 130, 96), (4, 2048, 256)])
def test_pack_matches_layout(shape):
    rng = np.random.default_rng(list(shape))
    a = rng.integers(-(1 << 15), 1 << 15, size=shape, dtype=np.int64).astype(np.int16)
    src = torch.from_numpy(a).cuda()
    dst = torch.full_like(src, 0x7BCD)
    moe.moe_pack_bf16_pairs(src, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().reshape(-1), pairs_layout(a))
    assert np.array_equal(src.cpu().numpy(), a)                      # the source is left as it was


def test_pack_to_fp16():
    """Finite bf16 values over fp16's whole range and beyond: normal, subnormal
    and underflowing magnitudes, values past 65504, signed zeros, infinities."""
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.uniform(-30.0, 20.0, size=(3, 64, 256)))
    v = (mag * rng.choice([-1.0, 1.0], size=mag.shape)).astype(np.float32)
    v.reshape(-1)[:6] = [0.0, -0.0, np.inf, -np.inf, 65504.0, 65520.0]
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)             # bf16 by truncation
    src = torch.from_numpy(bits.view(np.int16)).cuda()
    dst = torch.empty_like(src)
    moe.moe_pack_bf16_pairs(src, dst, to_fp16=True)
    torch.cuda.synchronize()
    want = pairs_layout(bf16_to_f16_toward_zero(bits).view(np.int16))
    got = dst.cpu().numpy().reshape(-1)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} values differ, e.g. index {bad[:4]}: got {got[bad[:4]]} want {want[bad[:4]]}"


SMALL = [
    (LayerShape("p_tiny", 64, 256, 256, 16, 2, "normal", "bf16"), [1, 8, 32, 10**6]),
    (LayerShape("p_mid", 700, 512, 512, 6, 2, "normal", "bf16"), [1, 32, 10**6]),
    (LayerShape("p_skew", 333, 256, 256, 40, 4, "zipf", "bf16"), [32]),
    (LayerShape("p_t1", 1, 256, 256, 16, 2, "normal", "bf16"), [1, 32]),
    (LayerShape("p_kE", 8, 256, 768, 16, 16, "normal", "bf16"), [1, 32]),
]


@pytest.mark.parametrize("shape,thresholds", SMALL, ids=[s.name for s, _ in SMALL])
def test_pairs_small_layers(shape, thresholds):
    logits, x = routing_inputs(shape, 0)
    W = layer_weights(shape, 0)
    ref = oracle.moe_layer(logits, x, host_raw(W), shape.k)
    dw = to_dev_weights(W)
    pw = packed(dw)
    plain = moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, moe.MOE_WFMT_BF16)
    pairs = moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, moe.MOE_WFMT_BF16_PAIRS)
    for thr in thresholds:
        say(f"[pairs {shape.name}] T={shape.T} E={shape.E} k={shape.k} H={shape.H} I={shape.I} fat_threshold={thr}")
        a = run_layer(plain, logits, x, dw, fat_threshold=thr)
        b = run_layer(pairs, logits, x, pw, fat_threshold=thr)
        check_indices(b, ref)
        ey = oracle.rel_max_err(b["Y"], ref["Y"])
        eo = oracle.rel_max_err(b["out"], ref["out"])
        parity_line(f"{shape.name}/pairs/thr{thr}", "Y(all rows)", ey, TOL_BF16, shape.T * shape.k)
        parity_line(f"{shape.name}/pairs/thr{thr}", "out(all tokens)", eo, TOL_BF16, shape.T)
        assert ey <= TOL_BF16 and eo <= TOL_BF16
        assert np.array_equal(a["Y"], b["Y"]) and np.array_equal(a["out"], b["out"]), "pairs != plain"


# Route lists on both sides of the fat threshold and of the 256-row M-tile,
# and thin tiles of 1, 15, 16, 17 rows next to full ones.
EDGE_COUNTS = [31, 32, 33, 1, 64, 65, 256, 257, 300, 16, 17, 15, 48, 49]


def _owner_logits(counts, seed):
    E, T = len(counts), int(sum(counts))
    rng = np.random.default_rng([seed, T, E])
    owner = np.repeat(np.arange(E), counts)
    rng.shuffle(owner)
    lg = (0.1 * rng.standard_normal((T, E))).astype(np.float32)
    lg[np.arange(T), owner] += np.float32(5.0)
    return lg


def test_pairs_tile_edges():
    E, k = len(EDGE_COUNTS), 1
    T = sum(EDGE_COUNTS)
    shape = LayerShape("p_edges", T, 256, 256, E, k, "normal", "bf16")
    _, x = routing_inputs(shape, 0)
    logits = _owner_logits(EDGE_COUNTS, 3)
    W = layer_weights(shape, 0)
    ref = oracle.moe_layer(logits, x, host_raw(W), k)
    assert np.array_equal(ref["counts"], EDGE_COUNTS)
    dw = to_dev_weights(W)
    pw = packed(dw)
    plain = moe.MoELayerBuffers(T, E, k, shape.H, shape.I, moe.MOE_WFMT_BF16)
    pairs = moe.MoELayerBuffers(T, E, k, shape.H, shape.I, moe.MOE_WFMT_BF16_PAIRS)
    for thr in (1, 32, 33, 10**6):
        say(f"[pairs edges] T={T} counts={EDGE_COUNTS} fat_threshold={thr}")
        a = run_layer(plain, logits, x, dw, fat_threshold=thr)
        b = run_layer(pairs, logits, x, pw, fat_threshold=thr)
        check_indices(b, ref)
        for e, (lo, hi) in enumerate(zip(ref["offsets"][:-1], ref["offsets"][1:])):
            assert oracle.rel_max_err(b["Y"][lo:hi], ref["Y"][lo:hi]) <= TOL_BF16, f"expert {e} ({hi - lo} rows)"
        assert np.array_equal(a["Y"], b["Y"]) and np.array_equal(a["out"], b["out"]), "pairs != plain"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill16k", "prefill1k", "decode"])
def test_pairs_full_size_equal_plain(name):
    """The benchmarked workloads: the packed layer's y (every sorted row) and
    out (every token) equal the plain layer's bit for bit."""
    from tests.test_gpu_dense import device_weights
    shape = SHAPES[name]
    logits, x = routing_inputs(shape, 0)
    dw = device_weights(shape, 0)
    say(f"[pairs full] {name} T={shape.T}: packing {sum(t.numel() for t in dw.values()) * 2 / 1e9:.1f} GB")
    pw = packed(dw)
    dl = torch.from_numpy(logits).cuda()
    dx = torch.from_numpy(x.view(np.int16)).cuda()
    res = []
    for wfmt, w in ((moe.MOE_WFMT_BF16, dw), (moe.MOE_WFMT_BF16_PAIRS, pw)):
        b = moe.MoELayerBuffers(shape.T, shape.E, shape.k, shape.H, shape.I, wfmt)
        b.forward(dl, dx, w, fat_threshold=32)
        torch.cuda.synchronize()
        res.append(b)
    a, b = res
    assert torch.equal(a.sorted_pair, b.sorted_pair)
    assert torch.equal(a.y_sorted, b.y_sorted), "y differs"
    assert torch.equal(a.out, b.out), "out differs"
    say(f"   y ({a.y_sorted.numel()} values) and out ({a.out.numel()}) identical")
    del pw, res, a, b
    torch.cuda.empty_cache()
