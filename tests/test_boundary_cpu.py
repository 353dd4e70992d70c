"""C-ABI boundary checks that need no GPU: the library loads, exports every
entry point its header declares, and rejects every invalid argument with the
documented status before touching the device.
"""
import ctypes
import os
import re

import pytest

import routed_expert_ffn_03_amd as moe
from routed_expert_ffn_03_amd.build import LIB

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_mi355x.h")
FAKE = 0x10000        # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+char\s*\*|size_t|moe_status)\s*(\w+)\s*\(", src, flags=re.M)


def test_library_exports_every_declared_symbol():
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS)
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), n


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    return moe.lib()


def test_status_strings(L):
    for s in range(5):
        assert L.moe_status_string(s).startswith(b"MOE_")
    assert L.moe_status_string(99) == b"MOE_ERR_UNKNOWN"
    assert L.moe_version() == b"0.1.0"


def test_workspace_size(L):
    ws = L.moe_workspace_size(16384, 384, 8, 4096, 2048, 0)
    assert ws >= 16384 * 8 * 2048 * 2             # the fp16 activation dominates
    r256 = lambda v: (v + 255) // 256 * 256
    # 3-bit: plus the reordered thin activation rows and their 128-group sums
    assert L.moe_workspace_size(16384, 384, 8, 4096, 2048, 1) == ws + r256(16384 * 4096 * 2) + r256(16384 * 32 * 4)
    assert L.moe_workspace_size(4, 384, 8, 4096, 2048, 0) > 0
    # the row-pair bf16 layout: the same workspace, but I a multiple of 256
    assert L.moe_workspace_size(16384, 384, 8, 4096, 2048, 2) == ws
    assert L.moe_workspace_size(64, 16, 2, 256, 384, 0) > 0
    assert L.moe_workspace_size(64, 16, 2, 256, 384, 2) == 0
    for bad in [(0, 384, 8, 4096, 2048, 0), (4, 2000, 8, 4096, 2048, 0), (4, 384, 0, 4096, 2048, 0),
                (4, 384, 33, 4096, 2048, 0), (4, 4, 5, 4096, 2048, 0), (4, 384, 8, 4000, 2048, 0),
                (4, 384, 8, 4096, 2000, 0), (4, 384, 8, 4096, 2048, 5), (1 << 28, 384, 8, 4096, 2048, 0),
                (1 << 19, 384, 8, 4096, 2048, 0)]:
        assert L.moe_workspace_size(*bad) == 0, bad


def test_route_rejects(L):
    ok = (FAKE, 64, 16, 2, FAKE, FAKE, FAKE, None)
    for i in (0, 4, 5, 6):
        args = list(ok)
        args[i] = None
        assert L.moe_route_topk(*args) == moe.MOE_ERR_INVALID_ARG
    for T, E, k in [(0, 16, 2), (64, 0, 1), (64, 1025, 2), (64, 16, 0), (64, 16, 17), (64, 64, 33),
                    (1 << 30, 16, 2)]:
        assert L.moe_route_topk(FAKE, T, E, k, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG


def test_router_rejects(L):
    ok = dict(x=FAKE, w=FAKE, T=64, E=384, H=4096, k=8, ids=FAKE, tw=FAKE, cnt=FAKE, lg=None, ws=None, wsb=0)
    call = lambda **kw: L.moe_router_topk(*[{**ok, **kw}[n] for n in ("x", "w", "T", "E", "H", "k", "ids", "tw",
                                                                         "cnt", "lg", "ws", "wsb")], None)
    for key in ("x", "w", "ids", "tw", "cnt"):
        assert call(**{key: None}) == moe.MOE_ERR_INVALID_ARG, key
    assert call(T=0) == moe.MOE_ERR_INVALID_ARG
    assert call(k=0) == moe.MOE_ERR_INVALID_ARG
    assert call(k=33) == moe.MOE_ERR_INVALID_ARG
    assert call(E=2048) == moe.MOE_ERR_INVALID_ARG
    for E in (16, 200, 640, 1024):
        assert call(E=E, k=2) == moe.MOE_ERR_UNSUPPORTED, E
    assert call(H=4080) == moe.MOE_ERR_UNSUPPORTED                      # not a multiple of 32
    assert call(T=1 << 19, H=4096, k=1) == moe.MOE_ERR_UNSUPPORTED      # x = 4 GiB
    # a workspace, when given, holds the batch's logits
    assert call(T=4, ws=FAKE, wsb=4 * 384 * 4 - 1) == moe.MOE_ERR_WORKSPACE


def test_permute_rejects(L):
    assert L.moe_permute(None, 64, 16, 2, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_permute(FAKE, 64, 16, 0, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_permute(FAKE, 64, 16, 2, FAKE, FAKE, FAKE, None, 1 << 20, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_permute(FAKE, 4096, 384, 8, FAKE, FAKE, FAKE, FAKE, 100, None) == moe.MOE_ERR_WORKSPACE


def _ffn(L, **kw):
    a = dict(x=FAKE, wfmt=0, wg=FAKE, wu=FAKE, wd=FAKE, sg=None, su=None, sd=None, off=FAKE, sp=FAKE,
             T=64, E=16, k=2, H=256, I=128, thr=32, y=FAKE, ws=FAKE, wsb=1 << 40, s=None)
    a.update(kw)
    return L.moe_grouped_ffn(a["x"], a["wfmt"], a["wg"], a["wu"], a["wd"], a["sg"], a["su"], a["sd"], a["off"],
                             a["sp"], a["T"], a["E"], a["k"], a["H"], a["I"], a["thr"], a["y"], a["ws"], a["wsb"],
                             a["s"])


def test_grouped_ffn_rejects(L):
    for key in ("x", "wg", "wu", "wd", "off", "sp", "y"):
        assert _ffn(L, **{key: None}) == moe.MOE_ERR_INVALID_ARG, key
    assert _ffn(L, thr=0) == moe.MOE_ERR_INVALID_ARG
    assert _ffn(L, sg=FAKE) == moe.MOE_ERR_INVALID_ARG                 # bf16 takes no scales
    assert _ffn(L, wfmt=1) == moe.MOE_ERR_INVALID_ARG                  # 3-bit needs scales
    assert _ffn(L, wfmt=2) == moe.MOE_ERR_UNSUPPORTED                  # row pairs: I % 256 != 0
    assert _ffn(L, wfmt=2, I=256, sg=FAKE) == moe.MOE_ERR_INVALID_ARG  # bf16 pairs take no scales
    assert _ffn(L, wfmt=3) == moe.MOE_ERR_UNSUPPORTED
    assert _ffn(L, H=384) == moe.MOE_ERR_UNSUPPORTED
    assert _ffn(L, I=192) == moe.MOE_ERR_UNSUPPORTED
    # 32-bit buffer offsets: x, the activation and one expert matrix stay below 4 GiB
    assert _ffn(L, T=1 << 19, H=4096, I=128, k=1) == moe.MOE_ERR_UNSUPPORTED    # x = 4 GiB
    assert _ffn(L, T=1 << 18, H=256, I=4096, k=2) == moe.MOE_ERR_UNSUPPORTED    # a = 4 GiB
    assert _ffn(L, T=64, H=65536, I=32768, k=2) == moe.MOE_ERR_UNSUPPORTED      # W = 4 GiB
    assert _ffn(L, k=17) == moe.MOE_ERR_INVALID_ARG
    assert _ffn(L, ws=None) == moe.MOE_ERR_WORKSPACE
    assert _ffn(L, wsb=1024) == moe.MOE_ERR_WORKSPACE


def test_split_ffn_rejects(L):
    assert L.moe_ffn_plan(None, 64, 16, 2, 256, 128, 0, 32, FAKE, 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_ffn_plan(FAKE, 64, 16, 2, 256, 128, 0, 0, FAKE, 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_ffn_plan(FAKE, 64, 16, 2, 256, 128, 0, 32, FAKE, 16, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_ffn_plan(FAKE, 64, 16, 2, 250, 128, 0, 32, FAKE, 1 << 40, None) == moe.MOE_ERR_UNSUPPORTED
    gu = lambda **kw: L.moe_ffn_gate_up(kw.get("x", FAKE), kw.get("wfmt", 0), FAKE, FAKE, kw.get("sg"),
                                        kw.get("su"), FAKE, 64, 16, 2, 256, 128, kw.get("thr", 32), FAKE,
                                        kw.get("wsb", 1 << 40), None)
    assert gu(x=None) == moe.MOE_ERR_INVALID_ARG
    assert gu(sg=FAKE) == moe.MOE_ERR_INVALID_ARG
    assert gu(wfmt=1, sg=FAKE) == moe.MOE_ERR_INVALID_ARG
    assert gu(wfmt=3) == moe.MOE_ERR_UNSUPPORTED
    assert gu(wsb=8) == moe.MOE_ERR_WORKSPACE
    assert gu(thr=0) == moe.MOE_ERR_INVALID_ARG
    dn = lambda *a: L.moe_ffn_down(*a, FAKE, 1 << 40, None)
    assert dn(0, FAKE, None, 64, 16, 2, 256, 128, 32, None) == moe.MOE_ERR_INVALID_ARG
    assert dn(1, FAKE, None, 64, 16, 2, 256, 128, 32, FAKE) == moe.MOE_ERR_INVALID_ARG
    assert dn(0, FAKE, FAKE, 64, 16, 2, 256, 128, 32, FAKE) == moe.MOE_ERR_INVALID_ARG
    assert dn(0, FAKE, None, 64, 16, 2, 256, 128, 0, FAKE) == moe.MOE_ERR_INVALID_ARG


def test_combine_rejects(L):
    assert L.moe_combine(None, FAKE, FAKE, 4, 2, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_combine(FAKE, FAKE, FAKE, 0, 2, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 33, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 2, 60, FAKE, None) == moe.MOE_ERR_UNSUPPORTED


def test_noalloc_rejects(L):
    F = FAKE
    args = [F, 0, F, F, F, None, None, None, F, F, 64, 16, 2, 256, 128, 32, F, None]
    for i in (0, 2, 3, 4, 8, 9, 16):
        bad = list(args)
        bad[i] = None
        assert L.moe_grouped_ffn_noalloc(*bad) == moe.MOE_ERR_INVALID_ARG, i
    bad = list(args)
    bad[15] = 0                                     # fat_threshold
    assert L.moe_grouped_ffn_noalloc(*bad) == moe.MOE_ERR_INVALID_ARG
    bad = list(args)
    bad[5] = F                                      # bf16 weights take no scales
    assert L.moe_grouped_ffn_noalloc(*bad) == moe.MOE_ERR_INVALID_ARG
    bad = list(args)
    bad[1] = 1                                      # 3-bit without scales
    assert L.moe_grouped_ffn_noalloc(*bad) == moe.MOE_ERR_INVALID_ARG
    bad = list(args)
    bad[13] = 200                                   # H not a multiple of 256
    assert L.moe_grouped_ffn_noalloc(*bad) == moe.MOE_ERR_UNSUPPORTED
    bad = list(args)
    bad[1] = 2                                      # row pairs need I % 256 == 0
    assert L.moe_grouped_ffn_noalloc(*bad) == moe.MOE_ERR_UNSUPPORTED
    # beyond the 64 MiB array: 4096 x 8 pairs x 2048 x 2 bytes of activation
    big = list(args)
    big[10:15] = [4096, 384, 8, 4096, 2048]
    assert L.moe_grouped_ffn_noalloc(*big) == moe.MOE_ERR_WORKSPACE


def test_route_permute_plan_rejects(L):
    F = FAKE
    args = [F, 4, 384, 8, 4096, 2048, 0, 32, F, F, F, F, F, F, F, 1 << 40, None]
    for i in (0, 8, 9, 10, 11, 12, 13):
        bad = list(args)
        bad[i] = None
        assert L.moe_route_permute_plan(*bad) == moe.MOE_ERR_INVALID_ARG, i
    bad = list(args)
    bad[7] = 0
    assert L.moe_route_permute_plan(*bad) == moe.MOE_ERR_INVALID_ARG
    bad = list(args)
    bad[15] = 1024                                    # workspace too small
    assert L.moe_route_permute_plan(*bad) == moe.MOE_ERR_WORKSPACE
    bad = list(args)
    bad[6] = 7                                        # unknown weight format
    assert L.moe_route_permute_plan(*bad) == moe.MOE_ERR_UNSUPPORTED


def test_pack_rejects(L):
    i64 = ctypes.c_int64
    call = lambda src, dst, mats, rows, cols, f16=0: L.moe_pack_bf16_pairs(src, dst, i64(mats), rows, cols, f16, None)
    D = FAKE + (1 << 30)                               # a destination far from FAKE
    assert call(None, D, 1, 2, 32) == moe.MOE_ERR_INVALID_ARG
    assert call(FAKE, None, 1, 2, 32) == moe.MOE_ERR_INVALID_ARG
    for mats, rows, cols in [(0, 2, 32), (1, 0, 32), (1, 3, 32), (1, 2, 16), (1, 2, 48), (-1, 2, 32),
                             (1 << 60, 2048, 4096)]:
        assert call(FAKE, D, mats, rows, cols) == moe.MOE_ERR_INVALID_ARG, (mats, rows, cols)
    assert call(FAKE + 8, D, 1, 2, 32) == moe.MOE_ERR_INVALID_ARG     # not 16-byte aligned
    assert call(FAKE, D + 2, 1, 2, 32) == moe.MOE_ERR_INVALID_ARG
    assert call(FAKE, FAKE, 1, 2, 32) == moe.MOE_ERR_INVALID_ARG       # in place
    assert call(FAKE, FAKE + 64, 1, 2, 32) == moe.MOE_ERR_INVALID_ARG  # overlapping (128 bytes each)
    assert call(FAKE, D, 1, 2, 32, 2) == moe.MOE_ERR_INVALID_ARG       # to_fp16 is 0 or 1
