"""ctypes binding of ``libmoe_mi355x.so``: the C entry points under the same
names, taking torch tensors.  Argument marshalling only -- every step of the
layer runs in the library's HIP kernels; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4
MOE_WFMT_BF16 = 0
MOE_WFMT_Q3G128 = 1
MOE_WFMT_BF16_PAIRS = 2

DEFAULT_FAT_THRESHOLD = 32

EXPORTS = ("moe_status_string", "moe_version", "moe_workspace_size", "moe_route_topk", "moe_router_topk",
           "moe_permute", "moe_grouped_ffn", "moe_ffn_plan", "moe_ffn_gate_up", "moe_ffn_down",
           "moe_combine", "moe_grouped_ffn_noalloc", "moe_route_permute_plan", "moe_pack_bf16_pairs")

NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {lib().moe_status_string(status).decode()} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the built library (fails loudly if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: build it with `python -m routed_expert_ffn_03_amd.build`")
        L = ctypes.CDLL(LIB)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [i32]
        L.moe_version.restype = ctypes.c_char_p
        L.moe_version.argtypes = []
        L.moe_workspace_size.restype = sz
        L.moe_workspace_size.argtypes = [i32] * 6
        L.moe_route_topk.restype = i32
        L.moe_route_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.moe_router_topk.restype = i32
        L.moe_router_topk.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_permute.restype = i32
        L.moe_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.moe_grouped_ffn.restype = i32
        L.moe_grouped_ffn.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                      i32, i32, i32, i32, i32, i32, vp, vp, sz, vp]
        L.moe_ffn_plan.restype = i32
        L.moe_ffn_plan.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.moe_ffn_gate_up.restype = i32
        L.moe_ffn_gate_up.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.moe_ffn_down.restype = i32
        L.moe_ffn_down.argtypes = [i32, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, sz, vp]
        L.moe_grouped_ffn_noalloc.restype = i32
        L.moe_grouped_ffn_noalloc.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                              i32, i32, i32, i32, i32, i32, vp, vp]
        L.moe_route_permute_plan.restype = i32
        L.moe_route_permute_plan.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_combine.restype = i32
        L.moe_combine.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
        L.moe_pack_bf16_pairs.restype = i32
        L.moe_pack_bf16_pairs.argtypes = [vp, vp, ctypes.c_int64, i32, i32, i32, vp]
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoEError(status, what)


def _dev(t: torch.Tensor, dtype, name: str):
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor on the GPU")


def moe_workspace_size(T: int, E: int, k: int, H: int, I: int, wfmt: int = MOE_WFMT_BF16) -> int:
    return int(lib().moe_workspace_size(T, E, k, H, I, wfmt))


def moe_route_topk(logits, k, topk_ids, topk_w, expert_counts, stream=None):
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    for t, dt, n, shp in ((topk_ids, torch.int32, "topk_ids", (T, k)), (topk_w, torch.float32, "topk_w", (T, k)),
                          (expert_counts, torch.int32, "expert_counts", (E,))):
        _dev(t, dt, n)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n}: shape {tuple(t.shape)} != {shp}")
    _check(lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w), _ptr(expert_counts),
                                _stream(stream)), "moe_route_topk")


def moe_router_topk(x, w_router, k, topk_ids, topk_w, expert_counts, logits=None, workspace=None, stream=None):
    """Router GEMM (x [T, H] bf16 bits . w_router [E, H] bf16 bits) fused with the top-k gate;
    ``logits`` (fp32 [T, E]) is written only when given; ``workspace`` (uint8, >= T * E * 4
    bytes) lets a batch of at most 32 tokens spread the GEMM over E / 32 blocks without it."""
    T, H = x.shape
    E = w_router.shape[0]
    if x.dtype not in (torch.int16, torch.bfloat16) or w_router.dtype not in (torch.int16, torch.bfloat16):
        raise ValueError("x and w_router: bf16 bit patterns (int16 or bfloat16 tensors)")
    for t, name in ((x, "x"), (w_router, "w_router")):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name}: expected a contiguous tensor on the GPU")
    if w_router.shape[1] != H:
        raise ValueError("w_router must be [E, H]")
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(topk_w, torch.float32, "topk_w")
    _dev(expert_counts, torch.int32, "expert_counts")
    if logits is not None:
        _dev(logits, torch.float32, "logits")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    _check(lib().moe_router_topk(_ptr(x), _ptr(w_router), T, E, H, k, _ptr(topk_ids), _ptr(topk_w),
                                 _ptr(expert_counts), _ptr(logits), _ptr(workspace), ws_bytes, _stream(stream)),
           "moe_router_topk")


def moe_permute(topk_ids, E, expert_offsets, sorted_pair, pair_to_sorted, workspace, stream=None):
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    for t, n, shp in ((expert_offsets, "expert_offsets", (E + 1,)), (sorted_pair, "sorted_pair", (T * k,)),
                      (pair_to_sorted, "pair_to_sorted", (T * k,))):
        _dev(t, torch.int32, n)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n}: shape {tuple(t.shape)} != {shp}")
    _dev(workspace, torch.uint8, "workspace")
    _check(lib().moe_permute(_ptr(topk_ids), T, E, k, _ptr(expert_offsets), _ptr(sorted_pair),
                             _ptr(pair_to_sorted), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_permute")


def moe_grouped_ffn(x, w_gate, w_up, w_down, expert_offsets, sorted_pair, k, y_sorted, workspace,
                    s_gate=None, s_up=None, s_down=None, fat_threshold=DEFAULT_FAT_THRESHOLD,
                    wfmt=MOE_WFMT_BF16, stream=None):
    """x, weights and y_sorted hold bf16/fp16 bit patterns (torch.bfloat16 /
    torch.float16 / int16 tensors are all accepted; 3-bit words are int32)."""
    T, H = x.shape
    E = expert_offsets.numel() - 1
    I = w_gate.shape[1]          # [E, I, H] bf16 or [E, I, H/128, 13] 3-bit words
    for t, n in ((x, "x"), (y_sorted, "y_sorted"), (w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down"),
                 (expert_offsets, "expert_offsets"), (sorted_pair, "sorted_pair"), (workspace, "workspace")):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{n}: expected a contiguous GPU tensor")
    if x.element_size() != 2 or y_sorted.element_size() != 2:
        raise ValueError("x and y_sorted must have 16-bit elements")
    if tuple(y_sorted.shape) != (T * k, H):
        raise ValueError(f"y_sorted: shape {tuple(y_sorted.shape)} != {(T * k, H)}")
    _check(lib().moe_grouped_ffn(_ptr(x), wfmt, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate),
                                 _ptr(s_up), _ptr(s_down), _ptr(expert_offsets), _ptr(sorted_pair), T, E, k, H, I,
                                 fat_threshold, _ptr(y_sorted), _ptr(workspace), workspace.numel(),
                                 _stream(stream)), "moe_grouped_ffn")


def moe_route_permute_plan(logits, k, H, I, topk_ids, topk_w, expert_counts, expert_offsets, sorted_pair,
                           pair_to_sorted, workspace, fat_threshold=DEFAULT_FAT_THRESHOLD, wfmt=MOE_WFMT_BF16,
                           stream=None):
    """moe_route_topk + moe_permute + moe_ffn_plan (one launch for T <= 64)."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    for t, dt, n, shp in ((topk_ids, torch.int32, "topk_ids", (T, k)), (topk_w, torch.float32, "topk_w", (T, k)),
                          (expert_counts, torch.int32, "expert_counts", (E,)),
                          (expert_offsets, torch.int32, "expert_offsets", (E + 1,)),
                          (sorted_pair, torch.int32, "sorted_pair", (T * k,)),
                          (pair_to_sorted, torch.int32, "pair_to_sorted", (T * k,))):
        _dev(t, dt, n)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n}: shape {tuple(t.shape)} != {shp}")
    _dev(workspace, torch.uint8, "workspace")
    _check(lib().moe_route_permute_plan(_ptr(logits), T, E, k, H, I, wfmt, fat_threshold, _ptr(topk_ids),
                                        _ptr(topk_w), _ptr(expert_counts), _ptr(expert_offsets), _ptr(sorted_pair),
                                        _ptr(pair_to_sorted), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_route_permute_plan")


def moe_grouped_ffn_noalloc(x, w_gate, w_up, w_down, expert_offsets, sorted_pair, k, y_sorted, s_gate=None,
                            s_up=None, s_down=None, fat_threshold=DEFAULT_FAT_THRESHOLD, wfmt=MOE_WFMT_BF16,
                            stream=None):
    """moe_grouped_ffn with the library's own per-GPU scratch array as its
    workspace (no allocation; calls that overlap on one GPU race)."""
    T, H = x.shape
    E = expert_offsets.numel() - 1
    I = w_gate.shape[1]
    for t, n in ((x, "x"), (y_sorted, "y_sorted"), (w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down"),
                 (expert_offsets, "expert_offsets"), (sorted_pair, "sorted_pair")):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{n}: expected a contiguous GPU tensor")
    if x.element_size() != 2 or y_sorted.element_size() != 2:
        raise ValueError("x and y_sorted must have 16-bit elements")
    if tuple(y_sorted.shape) != (T * k, H):
        raise ValueError(f"y_sorted: shape {tuple(y_sorted.shape)} != {(T * k, H)}")
    _check(lib().moe_grouped_ffn_noalloc(_ptr(x), wfmt, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate),
                                         _ptr(s_up), _ptr(s_down), _ptr(expert_offsets), _ptr(sorted_pair), T, E,
                                         k, H, I, fat_threshold, _ptr(y_sorted), _stream(stream)),
           "moe_grouped_ffn_noalloc")


def moe_ffn_plan(expert_offsets, T, k, H, I, workspace, fat_threshold=DEFAULT_FAT_THRESHOLD,
                 wfmt=MOE_WFMT_BF16, stream=None):
    E = expert_offsets.numel() - 1
    _dev(expert_offsets, torch.int32, "expert_offsets")
    _dev(workspace, torch.uint8, "workspace")
    _check(lib().moe_ffn_plan(_ptr(expert_offsets), T, E, k, H, I, wfmt, fat_threshold, _ptr(workspace),
                              workspace.numel(), _stream(stream)), "moe_ffn_plan")


def moe_ffn_gate_up(x, w_gate, w_up, sorted_pair, E, k, workspace, s_gate=None, s_up=None,
                    fat_threshold=DEFAULT_FAT_THRESHOLD, wfmt=MOE_WFMT_BF16, stream=None):
    T, H = x.shape
    I = w_gate.shape[1]
    _check(lib().moe_ffn_gate_up(_ptr(x), wfmt, _ptr(w_gate), _ptr(w_up), _ptr(s_gate), _ptr(s_up),
                                 _ptr(sorted_pair), T, E, k, H, I, fat_threshold, _ptr(workspace),
                                 workspace.numel(), _stream(stream)), "moe_ffn_gate_up")


def moe_ffn_down(w_down, T, E, k, I, y_sorted, workspace, s_down=None, fat_threshold=DEFAULT_FAT_THRESHOLD,
                 wfmt=MOE_WFMT_BF16, stream=None):
    H = y_sorted.shape[1]
    _check(lib().moe_ffn_down(wfmt, _ptr(w_down), _ptr(s_down), T, E, k, H, I, fat_threshold, _ptr(y_sorted),
                              _ptr(workspace), workspace.numel(), _stream(stream)), "moe_ffn_down")


def moe_combine(y_sorted, topk_w, pair_to_sorted, out, stream=None):
    T, k = topk_w.shape
    H = out.shape[1]
    _dev(topk_w, torch.float32, "topk_w")
    _dev(pair_to_sorted, torch.int32, "pair_to_sorted")
    _dev(out, torch.float32, "out")
    if not (y_sorted.is_cuda and y_sorted.is_contiguous() and y_sorted.element_size() == 2):
        raise ValueError("y_sorted: expected a contiguous 16-bit GPU tensor")
    _check(lib().moe_combine(_ptr(y_sorted), _ptr(topk_w), _ptr(pair_to_sorted), T, k, H, _ptr(out),
                             _stream(stream)), "moe_combine")


def moe_pack_bf16_pairs(src, dst, to_fp16=False, stream=None):
    """Copy bf16 matrices ``src`` [..., rows, cols] into ``dst`` (same shape) in the row-pair layout
    that ``MOE_WFMT_BF16_PAIRS`` reads: rows 2p and 2p+1 alternate every 32 columns; with
    ``to_fp16`` the values are converted to fp16 toward zero (that format's W_down)."""
    for t, name in ((src, "src"), (dst, "dst")):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous() and t.element_size() == 2):
            raise ValueError(f"{name}: expected a contiguous 16-bit GPU tensor")
    if src.dim() < 2 or tuple(src.shape) != tuple(dst.shape):
        raise ValueError(f"src {tuple(src.shape)} and dst {tuple(dst.shape)}: same shape [..., rows, cols] expected")
    rows, cols = int(src.shape[-2]), int(src.shape[-1])
    mats = src.numel() // (rows * cols) if rows * cols else 0
    _check(lib().moe_pack_bf16_pairs(_ptr(src), _ptr(dst), mats, rows, cols, int(bool(to_fp16)), _stream(stream)),
           "moe_pack_bf16_pairs")
