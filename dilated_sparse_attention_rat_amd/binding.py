"""Thin ctypes binding of ``librat.so`` (argument marshalling only).

Every entry point of ``include/rat.h`` has a Python function of the same
name.  The functions take torch tensors (device memory and streams are the
only things torch is used for), check that each tensor has the shape, dtype,
device and contiguity the C ABI expects (the library itself can only check
pointers), pass ``data_ptr()`` and the current HIP stream, and raise
:class:`RatError` on a non-zero status.  All computation happens in the HIP
kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librat.so")

RAT_OK = 0
RAT_ERR_INVALID_ARG = -1
RAT_ERR_UNSUPPORTED = -2
RAT_ERR_CAPACITY = -3
RAT_ERR_WORKSPACE = -4
RAT_ERR_HIP = -5
RAT_DTYPE_BF16 = 0
RAT_DTYPE_F32 = 1
RAT_MAX_HEADS = 128

EXPORTED = [
    "rat_version", "rat_status_string", "rat_anchor_rows", "rat_ring_rows",
    "rat_scan_workspace_bytes", "rat_scan_prefill", "rat_dilated_attn_prefill",
    "rat_scan_prefill_continue", "rat_dilated_attn_prefill_continue",
    "rat_decode_workspace_bytes", "rat_decode_step", "rat_decode_step_noalloc",
    "rat_prefill_backward_workspace_bytes", "rat_prefill_backward",
    "rat_layer_workspace_bytes", "rat_layer_prefill",
    "rat_stack_workspace_bytes", "rat_stack_prefill",
    "rat_topk_cache_build", "rat_decode_step_topk",
]

TOPK_BLOCK = 64   # RAT_TOPK_BLOCK
NOALLOC_SCRATCH_BYTES = 16 << 20  # RAT_NOALLOC_SCRATCH_BYTES
TOPK_MAX_K = 64   # RAT_TOPK_MAX_K


class RatError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({_status_string(status)})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; fails loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m dilated_sparse_attention_rat_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                ctypes.c_float, ctypes.c_size_t)
        L.rat_version.restype = ctypes.c_char_p
        L.rat_status_string.argtypes = [i32]
        L.rat_status_string.restype = ctypes.c_char_p
        L.rat_anchor_rows.argtypes = [i32, i64, P, P]
        L.rat_anchor_rows.restype = i64
        L.rat_ring_rows.argtypes = [i32, P, P]
        L.rat_ring_rows.restype = i64
        L.rat_scan_workspace_bytes.argtypes = [i32, i32, i64, i32]
        L.rat_scan_workspace_bytes.restype = i64
        L.rat_scan_prefill.argtypes = [i32, i32, i32, i64, i32, P, P, i64,
                                       P, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.rat_scan_prefill.restype = i32
        L.rat_dilated_attn_prefill.argtypes = [i32, i32, i32, i64, i32, P, P,
                                               f32, i64, P, P, P, P, P, P, P, P]
        L.rat_dilated_attn_prefill.restype = i32
        L.rat_scan_prefill_continue.argtypes = [i32, i32, i32, i64, i32, P, P, i64, i64,
                                                P, P, P, P, P, P, P, P, P, P, P, P, P,
                                                P, P, P, sz, P]
        L.rat_scan_prefill_continue.restype = i32
        L.rat_dilated_attn_prefill_continue.argtypes = [i32, i32, i32, i64, i32, P, P, f32,
                                                        i64, i64, P, P, P, P, P, P, P, P, P, P]
        L.rat_dilated_attn_prefill_continue.restype = i32
        L.rat_prefill_backward_workspace_bytes.argtypes = [i32, i32, i64, i32, P, P]
        L.rat_prefill_backward_workspace_bytes.restype = i64
        L.rat_prefill_backward.argtypes = [i32, i32, i32, i64, i32, P, P, f32] + [P] * 14 + [sz, P]
        L.rat_prefill_backward.restype = i32
        L.rat_layer_workspace_bytes.argtypes = [i32, i32, i32, i64, i32]
        L.rat_layer_workspace_bytes.restype = i64
        L.rat_layer_prefill.argtypes = [i32, i32, i32, i64, i32, i32, P, P, f32, i64] + [P] * 16 + [sz, P]
        L.rat_layer_prefill.restype = i32
        L.rat_stack_workspace_bytes.argtypes = [i32, i32, i32, i64, i32, i32]
        L.rat_stack_workspace_bytes.restype = i64
        L.rat_stack_prefill.argtypes = [i32, i32, i32, i32, i64, i32, i32, P, P, f32, i64] + [P] * 15 + [sz, P]
        L.rat_stack_prefill.restype = i32
        L.rat_decode_workspace_bytes.argtypes = [i32, i32, i32, i64, P, P, i32]
        L.rat_decode_workspace_bytes.restype = i64
        L.rat_decode_step.argtypes = [i32, i32, i32, i32, P, P, f32, i64, i64,
                                      P, P, P, P, P, P, P, P, P, P, P, i32, P,
                                      sz, P]
        L.rat_decode_step.restype = i32
        L.rat_decode_step_noalloc.argtypes = [i32, i32, i32, i32, P, P, f32, i64, i64] + [P] * 11 + [i32, P]
        L.rat_decode_step_noalloc.restype = i32
        L.rat_topk_cache_build.argtypes = [i32, i32, i32, i64, i32, i64, i64, P, P, P, P, P, P]
        L.rat_topk_cache_build.restype = i32
        L.rat_decode_step_topk.argtypes = [i32, i32, i32, i32, P, P, f32, i64, i64, i32] + [P] * 16
        L.rat_decode_step_topk.restype = i32
        _lib = L
    return _lib


def _status_string(status: int) -> str:
    try:
        return lib().rat_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - only while the library is missing
        return "?"


def _check(fn: str, status: int):
    if status != RAT_OK:
        raise RatError(fn, status)


def _heads(x, H: int) -> np.ndarray:
    a = np.ascontiguousarray(np.broadcast_to(np.asarray(x, dtype=np.int32), (H,)))
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# tensor marshalling helpers
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return RAT_DTYPE_BF16
    if t.dtype == torch.float32:
        return RAT_DTYPE_F32
    raise TypeError(f"unsupported storage dtype {t.dtype} (bf16 or fp32)")


def _dev(t, name, shape, dtype, device):
    """Pointer of a required device tensor after checking it."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: device {t.device} != {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _opt(t, name, shape, dtype, device):
    return None if t is None else _dev(t, name, shape, dtype, device)


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def rat_version() -> str:
    return lib().rat_version().decode()


def rat_status_string(status: int) -> str:
    return _status_string(status)


def rat_anchor_rows(H: int, T_cap: int, D):
    """Returns (R, offsets[H+1]) of the anchor-only cache."""
    Dh = _heads(D, H)
    off = np.zeros(H + 1, dtype=np.int64)
    r = lib().rat_anchor_rows(H, T_cap, _ptr(Dh), _ptr(off))
    if r < 0:
        raise RatError("rat_anchor_rows", int(r))
    return int(r), off


def rat_ring_rows(H: int, W):
    Wh = _heads(W, H)
    off = np.zeros(H + 1, dtype=np.int64)
    r = lib().rat_ring_rows(H, _ptr(Wh), _ptr(off))
    if r < 0:
        raise RatError("rat_ring_rows", int(r))
    return int(r), off


def rat_scan_workspace_bytes(B: int, H: int, T: int, hd: int) -> int:
    r = lib().rat_scan_workspace_bytes(B, H, T, hd)
    if r < 0:
        raise RatError("rat_scan_workspace_bytes", int(r))
    return int(r)


def rat_decode_workspace_bytes(B: int, H: int, hd: int, T_cap: int, D, W,
                               num_splits: int = 0) -> int:
    r = lib().rat_decode_workspace_bytes(B, H, hd, T_cap, _ptr(_heads(D, H)),
                                         _ptr(_heads(W, H)), num_splits)
    if r < 0:
        raise RatError("rat_decode_workspace_bytes", int(r))
    return int(r)


def rat_scan_prefill(k, v, g, D, W, T_cap: int, Kc, Vc, state_k, state_v,
                     workspace, hk=None, hv=None, k_ring=None, v_ring=None,
                     stream=None):
    """Recurrence + fused anchor compaction.  k, v, g: [B,H,T,hd]."""
    torch = _torch()
    B, H, T, hd = k.shape
    st = k.dtype
    dev = k.device
    Dh, Wh = _heads(D, H), _heads(W, H)
    R, _ = rat_anchor_rows(H, T_cap, Dh)
    WS, _ = rat_ring_rows(H, Wh)
    args = [
        _dtype_code(k), B, H, T, hd, _ptr(Dh), _ptr(Wh), T_cap,
        _dev(k, "k", (B, H, T, hd), st, dev), _dev(v, "v", (B, H, T, hd), st, dev),
        _dev(g, "g", (B, H, T, hd), st, dev),
        _opt(hk, "hk", (B, H, T, hd), st, dev), _opt(hv, "hv", (B, H, T, hd), st, dev),
        _opt(Kc, "Kc", (B, R, hd), st, dev), _opt(Vc, "Vc", (B, R, hd), st, dev),
        _opt(k_ring, "k_ring", (B, WS, hd), st, dev), _opt(v_ring, "v_ring", (B, WS, hd), st, dev),
        _dev(state_k, "state_k", (B, H, hd), torch.float32, dev),
        _dev(state_v, "state_v", (B, H, hd), torch.float32, dev),
    ]
    need = rat_scan_workspace_bytes(B, H, T, hd)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    args += [ctypes.c_void_p(workspace.data_ptr()),
             workspace.numel() * workspace.element_size(), _stream(stream, dev)]
    _check("rat_scan_prefill", lib().rat_scan_prefill(*args))


def rat_dilated_attn_prefill(q, hk, hv, Kc, Vc, D, W, T_cap: int, o, lse=None,
                             scale: float = 0.0, stream=None):
    """Dilated causal attention.  q, hk, hv, o: [B,H,T,hd]; Kc, Vc: [B,R,hd]."""
    torch = _torch()
    B, H, T, hd = q.shape
    st = q.dtype
    dev = q.device
    Dh, Wh = _heads(D, H), _heads(W, H)
    R, _ = rat_anchor_rows(H, T_cap, Dh)
    args = [
        _dtype_code(q), B, H, T, hd, _ptr(Dh), _ptr(Wh), float(scale), T_cap,
        _dev(q, "q", (B, H, T, hd), st, dev), _dev(hk, "hk", (B, H, T, hd), st, dev),
        _dev(hv, "hv", (B, H, T, hd), st, dev),
        _opt(Kc, "Kc", (B, R, hd), st, dev), _opt(Vc, "Vc", (B, R, hd), st, dev),
        _dev(o, "o", (B, H, T, hd), st, dev),
        _opt(lse, "lse", (B, H, T), torch.float32, dev), _stream(stream, dev),
    ]
    _check("rat_dilated_attn_prefill", lib().rat_dilated_attn_prefill(*args))


def rat_scan_prefill_continue(k, v, g, D, W, T_cap: int, t0: int, state_k_in,
                              state_v_in, Kc, Vc, state_k, state_v, workspace,
                              hk=None, hv=None, k_ring_in=None, v_ring_in=None,
                              k_ring=None, v_ring=None, stream=None):
    """Recurrence of a chunk at positions t0 .. t0+T-1.  k, v, g: [B,H,T,hd]."""
    torch = _torch()
    B, H, T, hd = k.shape
    st = k.dtype
    dev = k.device
    Dh, Wh = _heads(D, H), _heads(W, H)
    R, _ = rat_anchor_rows(H, T_cap, Dh)
    WS, _ = rat_ring_rows(H, Wh)
    args = [
        _dtype_code(k), B, H, T, hd, _ptr(Dh), _ptr(Wh), T_cap, int(t0),
        _dev(k, "k", (B, H, T, hd), st, dev), _dev(v, "v", (B, H, T, hd), st, dev),
        _dev(g, "g", (B, H, T, hd), st, dev),
        _dev(state_k_in, "state_k_in", (B, H, hd), torch.float32, dev),
        _dev(state_v_in, "state_v_in", (B, H, hd), torch.float32, dev),
        _opt(hk, "hk", (B, H, T, hd), st, dev), _opt(hv, "hv", (B, H, T, hd), st, dev),
        _opt(Kc, "Kc", (B, R, hd), st, dev), _opt(Vc, "Vc", (B, R, hd), st, dev),
        _opt(k_ring_in, "k_ring_in", (B, WS, hd), st, dev),
        _opt(v_ring_in, "v_ring_in", (B, WS, hd), st, dev),
        _opt(k_ring, "k_ring", (B, WS, hd), st, dev), _opt(v_ring, "v_ring", (B, WS, hd), st, dev),
        _dev(state_k, "state_k", (B, H, hd), torch.float32, dev),
        _dev(state_v, "state_v", (B, H, hd), torch.float32, dev),
    ]
    need = rat_scan_workspace_bytes(B, H, T, hd)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    args += [ctypes.c_void_p(workspace.data_ptr()),
             workspace.numel() * workspace.element_size(), _stream(stream, dev)]
    _check("rat_scan_prefill_continue", lib().rat_scan_prefill_continue(*args))


def rat_dilated_attn_prefill_continue(q, hk, hv, Kc, Vc, D, W, T_cap: int, t0: int, o,
                                      k_ring_prev=None, v_ring_prev=None, lse=None,
                                      scale: float = 0.0, stream=None):
    """Attention of a chunk's queries at positions t0 .. t0+T-1."""
    torch = _torch()
    B, H, T, hd = q.shape
    st = q.dtype
    dev = q.device
    Dh, Wh = _heads(D, H), _heads(W, H)
    R, _ = rat_anchor_rows(H, T_cap, Dh)
    WS, _ = rat_ring_rows(H, Wh)
    args = [
        _dtype_code(q), B, H, T, hd, _ptr(Dh), _ptr(Wh), float(scale), T_cap, int(t0),
        _dev(q, "q", (B, H, T, hd), st, dev), _dev(hk, "hk", (B, H, T, hd), st, dev),
        _dev(hv, "hv", (B, H, T, hd), st, dev),
        _opt(Kc, "Kc", (B, R, hd), st, dev), _opt(Vc, "Vc", (B, R, hd), st, dev),
        _opt(k_ring_prev, "k_ring_prev", (B, WS, hd), st, dev),
        _opt(v_ring_prev, "v_ring_prev", (B, WS, hd), st, dev),
        _dev(o, "o", (B, H, T, hd), st, dev),
        _opt(lse, "lse", (B, H, T), torch.float32, dev), _stream(stream, dev),
    ]
    _check("rat_dilated_attn_prefill_continue",
           lib().rat_dilated_attn_prefill_continue(*args))


def rat_decode_step(q, k, v, g, state_k, state_v, Kc, Vc, k_ring, v_ring, o,
                    D, W, pos: int, T_cap: int, scale: float = 0.0,
                    num_splits: int = 0, workspace=None, stream=None):
    """One decode step at position pos.  q, k, v, g, o: [B,H,hd]."""
    torch = _torch()
    B, H, hd = q.shape
    st = q.dtype
    dev = q.device
    Dh, Wh = _heads(D, H), _heads(W, H)
    R, _ = rat_anchor_rows(H, T_cap, Dh)
    WS, _ = rat_ring_rows(H, Wh)
    need = rat_decode_workspace_bytes(B, H, hd, T_cap, Dh, Wh, num_splits)
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace must hold {need} bytes")
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the same device")
        ws_ptr = ctypes.c_void_p(workspace.data_ptr())
        ws_bytes = workspace.numel() * workspace.element_size()
    args = [
        _dtype_code(q), B, H, hd, _ptr(Dh), _ptr(Wh), float(scale), pos, T_cap,
        _dev(q, "q", (B, H, hd), st, dev), _dev(k, "k", (B, H, hd), st, dev),
        _dev(v, "v", (B, H, hd), st, dev), _dev(g, "g", (B, H, hd), st, dev),
        _dev(state_k, "state_k", (B, H, hd), torch.float32, dev),
        _dev(state_v, "state_v", (B, H, hd), torch.float32, dev),
        _opt(Kc, "Kc", (B, R, hd), st, dev), _opt(Vc, "Vc", (B, R, hd), st, dev),
        _opt(k_ring, "k_ring", (B, WS, hd), st, dev), _opt(v_ring, "v_ring", (B, WS, hd), st, dev),
        _dev(o, "o", (B, H, hd), st, dev), int(num_splits), ws_ptr, ws_bytes,
        _stream(stream, dev),
    ]
    _check("rat_decode_step", lib().rat_decode_step(*args))


def rat_decode_step_noalloc(q, k, v, g, state_k, state_v, Kc, Vc, k_ring, v_ring, o,
                            D, W, pos: int, T_cap: int, scale: float = 0.0,
                            num_splits: int = 0, stream=None):
    """rat_decode_step with the split-K partials in the library's own device
    array (no workspace argument; calls on one device must not overlap)."""
    torch = _torch()
    B, H, hd = q.shape
    st = q.dtype
    dev = q.device
    Dh, Wh = _heads(D, H), _heads(W, H)
    R, _ = rat_anchor_rows(H, T_cap, Dh)
    WS, _ = rat_ring_rows(H, Wh)
    args = [
        _dtype_code(q), B, H, hd, _ptr(Dh), _ptr(Wh), float(scale), pos, T_cap,
        _dev(q, "q", (B, H, hd), st, dev), _dev(k, "k", (B, H, hd), st, dev),
        _dev(v, "v", (B, H, hd), st, dev), _dev(g, "g", (B, H, hd), st, dev),
        _dev(state_k, "state_k", (B, H, hd), torch.float32, dev),
        _dev(state_v, "state_v", (B, H, hd), torch.float32, dev),
        _opt(Kc, "Kc", (B, R, hd), st, dev), _opt(Vc, "Vc", (B, R, hd), st, dev),
        _opt(k_ring, "k_ring", (B, WS, hd), st, dev), _opt(v_ring, "v_ring", (B, WS, hd), st, dev),
        _dev(o, "o", (B, H, hd), st, dev), int(num_splits), _stream(stream, dev),
    ]
    _check("rat_decode_step_noalloc", lib().rat_decode_step_noalloc(*args))


def rat_topk_cache_build(hk, hv, hk_hist, hv_hist, block_means, t0: int = 0, stream=None):
    """History cache of a prefill (or of the chunk at positions t0 .. t0+T-1)
    for top-k decode: rows of hk, hv [B,H,T,hd] into hk_hist, hv_hist
    [B,H,T_cap,hd], block means [B,H,T_cap//64,hd] fp32."""
    torch = _torch()
    B, H, T, hd = hk.shape
    st = hk.dtype
    dev = hk.device
    T_cap = hk_hist.shape[2]
    NB = T_cap // TOPK_BLOCK
    args = [
        _dtype_code(hk), B, H, T, hd, T_cap, int(t0),
        _dev(hk, "hk", (B, H, T, hd), st, dev), _dev(hv, "hv", (B, H, T, hd), st, dev),
        _dev(hk_hist, "hk_hist", (B, H, T_cap, hd), st, dev),
        _dev(hv_hist, "hv_hist", (B, H, T_cap, hd), st, dev),
        _opt(block_means, "block_means", (B, H, NB, hd), torch.float32, dev),
        _stream(stream, dev),
    ]
    _check("rat_topk_cache_build", lib().rat_topk_cache_build(*args))


def rat_decode_step_topk(q, k, v, g, state_k, state_v, Kc, Vc, k_ring, v_ring, hk_hist, hv_hist,
                         block_means, o, D, W, pos: int, T_cap: int, k_blocks: int,
                         scale: float = 0.0, sel_out=None, stream=None):
    """One decode step at position pos with top-k block selection.
    q, k, v, g, o: [B,H,hd]; history [B,H,T_cap,hd]; sel_out [B,H,k_blocks] int32."""
    torch = _torch()
    B, H, hd = q.shape
    st = q.dtype
    dev = q.device
    Dh, Wh = _heads(D, H), _heads(W, H)
    R, _ = rat_anchor_rows(H, T_cap, Dh)
    WS, _ = rat_ring_rows(H, Wh)
    NB = T_cap // TOPK_BLOCK
    args = [
        _dtype_code(q), B, H, hd, _ptr(Dh), _ptr(Wh), float(scale), pos, T_cap, int(k_blocks),
        _dev(q, "q", (B, H, hd), st, dev), _dev(k, "k", (B, H, hd), st, dev),
        _dev(v, "v", (B, H, hd), st, dev), _dev(g, "g", (B, H, hd), st, dev),
        _dev(state_k, "state_k", (B, H, hd), torch.float32, dev),
        _dev(state_v, "state_v", (B, H, hd), torch.float32, dev),
        _opt(Kc, "Kc", (B, R, hd), st, dev), _opt(Vc, "Vc", (B, R, hd), st, dev),
        _opt(k_ring, "k_ring", (B, WS, hd), st, dev), _opt(v_ring, "v_ring", (B, WS, hd), st, dev),
        _dev(hk_hist, "hk_hist", (B, H, T_cap, hd), st, dev),
        _dev(hv_hist, "hv_hist", (B, H, T_cap, hd), st, dev),
        _opt(block_means, "block_means", (B, H, NB, hd), torch.float32, dev),
        _dev(o, "o", (B, H, hd), st, dev),
        _opt(sel_out, "sel_out", (B, H, int(k_blocks)), torch.int32, dev),
        _stream(stream, dev),
    ]
    _check("rat_decode_step_topk", lib().rat_decode_step_topk(*args))


def alloc_topk_history(B: int, H: int, hd: int, T_cap: int, dtype, device, fill=None):
    """State history [B,H,T_cap,hd] (k and v) and block means [B,H,T_cap//64,hd] fp32."""
    torch = _torch()

    def mk(shape, dt):
        if fill is None:
            return torch.empty(shape, dtype=dt, device=device)
        return torch.full(shape, fill, dtype=dt, device=device)

    return dict(hk_hist=mk((B, H, T_cap, hd), dtype), hv_hist=mk((B, H, T_cap, hd), dtype),
                block_means=mk((B, H, T_cap // TOPK_BLOCK, hd), torch.float32))


def rat_prefill_backward_workspace_bytes(B: int, H: int, T: int, hd: int, D, W) -> int:
    r = lib().rat_prefill_backward_workspace_bytes(B, H, T, hd, _ptr(_heads(D, H)),
                                                   _ptr(_heads(W, H)))
    if r < 0:
        raise RatError("rat_prefill_backward_workspace_bytes", int(r))
    return int(r)


def rat_prefill_backward(q, k, v, g, hk, hv, o, lse, dO, D, W, dq, dk, dv, dg, workspace,
                         scale: float = 0.0, stream=None):
    """Gradients dq, dk, dv, dg of the prefill for dL/do = dO.  All [B,H,T,hd]
    except lse [B,H,T] fp32."""
    torch = _torch()
    B, H, T, hd = q.shape
    st = q.dtype
    dev = q.device
    Dh, Wh = _heads(D, H), _heads(W, H)
    shp = (B, H, T, hd)
    args = [_dtype_code(q), B, H, T, hd, _ptr(Dh), _ptr(Wh), float(scale)]
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (hk, "hk"), (hv, "hv"), (o, "o")):
        args.append(_dev(t, n, shp, st, dev))
    args.append(_dev(lse, "lse", (B, H, T), torch.float32, dev))
    args.append(_dev(dO, "dO", shp, st, dev))
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (dg, "dg")):
        args.append(_dev(t, n, shp, st, dev))
    need = rat_prefill_backward_workspace_bytes(B, H, T, hd, Dh, Wh)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    args += [ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
             _stream(stream, dev)]
    _check("rat_prefill_backward", lib().rat_prefill_backward(*args))


def rat_layer_workspace_bytes(dtype_code: int, B: int, H: int, T: int, hd: int) -> int:
    r = lib().rat_layer_workspace_bytes(dtype_code, B, H, T, hd)
    if r < 0:
        raise RatError("rat_layer_workspace_bytes", int(r))
    return int(r)


def rat_layer_prefill(x, w_q, w_k, w_v, w_g, b_g, w_o, out, D, W, H: int, hd: int, T_cap: int,
                      cache, workspace, lse=None, scale: float = 0.0, stream=None):
    """One RAT+ layer over a prefill.  x, out: [B,T,dm]; w_*: [dm,H*hd]
    (w_o: [H*hd,dm]); b_g: [H*hd] fp32; cache: dict of alloc_cache."""
    torch = _torch()
    B, T, dm = x.shape
    st = x.dtype
    dev = x.device
    Dh, Wh = _heads(D, H), _heads(W, H)
    R, _ = rat_anchor_rows(H, T_cap, Dh)
    WS, _ = rat_ring_rows(H, Wh)
    HD = H * hd
    args = [_dtype_code(x), B, H, T, hd, dm, _ptr(Dh), _ptr(Wh), float(scale), T_cap,
            _dev(x, "x", (B, T, dm), st, dev)]
    for t, n in ((w_q, "w_q"), (w_k, "w_k"), (w_v, "w_v"), (w_g, "w_g")):
        args.append(_dev(t, n, (dm, HD), st, dev))
    args += [_dev(b_g, "b_g", (HD,), torch.float32, dev), _dev(w_o, "w_o", (HD, dm), st, dev),
             _dev(out, "out", (B, T, dm), st, dev),
             _opt(lse, "lse", (B, H, T), torch.float32, dev),
             _opt(cache["Kc"], "Kc", (B, R, hd), st, dev), _opt(cache["Vc"], "Vc", (B, R, hd), st, dev),
             _opt(cache["k_ring"], "k_ring", (B, WS, hd), st, dev),
             _opt(cache["v_ring"], "v_ring", (B, WS, hd), st, dev),
             _dev(cache["state_k"], "state_k", (B, H, hd), torch.float32, dev),
             _dev(cache["state_v"], "state_v", (B, H, hd), torch.float32, dev)]
    need = rat_layer_workspace_bytes(_dtype_code(x), B, H, T, hd)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    args += [ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
             _stream(stream, dev)]
    _check("rat_layer_prefill", lib().rat_layer_prefill(*args))


def rat_stack_workspace_bytes(dtype_code: int, B: int, H: int, T: int, hd: int, dm: int) -> int:
    r = lib().rat_stack_workspace_bytes(dtype_code, B, H, T, hd, dm)
    if r < 0:
        raise RatError("rat_stack_workspace_bytes", int(r))
    return int(r)


def rat_stack_prefill(x, layers, out, H: int, hd: int, T_cap: int, caches, workspace,
                      scale: float = 0.0, stream=None):
    """A stack of RAT+ layers over a prefill (layer-wise hybrid).  x, out:
    [B,T,dm]; layers: one dict per layer with D, W (per head) and w_q, w_k,
    w_v, w_g, b_g, w_o as for rat_layer_prefill; caches: one alloc_cache dict
    per layer (sized by that layer's D and W)."""
    torch = _torch()
    B, T, dm = x.shape
    st = x.dtype
    dev = x.device
    n = len(layers)
    if n < 1 or len(caches) != n:
        raise ValueError("one cache per layer, at least one layer")
    HD = H * hd
    D = np.ascontiguousarray(np.stack([_heads(l["D"], H) for l in layers]).astype(np.int32))
    W = np.ascontiguousarray(np.stack([_heads(l["W"], H) for l in layers]).astype(np.int32))
    arrs = {k: (ctypes.c_void_p * n)() for k in
            ("w_q", "w_k", "w_v", "w_g", "b_g", "w_o", "Kc", "Vc", "k_ring", "v_ring",
             "state_k", "state_v")}
    for i, (ly, c) in enumerate(zip(layers, caches)):
        R, _ = rat_anchor_rows(H, T_cap, D[i])
        WS, _ = rat_ring_rows(H, W[i])
        for k in ("w_q", "w_k", "w_v", "w_g"):
            arrs[k][i] = _dev(ly[k], k, (dm, HD), st, dev)
        arrs["b_g"][i] = _dev(ly["b_g"], "b_g", (HD,), torch.float32, dev)
        arrs["w_o"][i] = _dev(ly["w_o"], "w_o", (HD, dm), st, dev)
        arrs["Kc"][i] = _opt(c["Kc"], "Kc", (B, R, hd), st, dev)
        arrs["Vc"][i] = _opt(c["Vc"], "Vc", (B, R, hd), st, dev)
        arrs["k_ring"][i] = _opt(c["k_ring"], "k_ring", (B, WS, hd), st, dev)
        arrs["v_ring"][i] = _opt(c["v_ring"], "v_ring", (B, WS, hd), st, dev)
        arrs["state_k"][i] = _dev(c["state_k"], "state_k", (B, H, hd), torch.float32, dev)
        arrs["state_v"][i] = _dev(c["state_v"], "state_v", (B, H, hd), torch.float32, dev)
    need = rat_stack_workspace_bytes(_dtype_code(x), B, H, T, hd, dm)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    args = [_dtype_code(x), n, B, H, T, hd, dm, _ptr(D), _ptr(W), float(scale), T_cap,
            _dev(x, "x", (B, T, dm), st, dev)]
    args += [ctypes.cast(arrs[k], ctypes.c_void_p) for k in ("w_q", "w_k", "w_v", "w_g", "b_g", "w_o")]
    args += [_dev(out, "out", (B, T, dm), st, dev)]
    args += [ctypes.cast(arrs[k], ctypes.c_void_p)
             for k in ("Kc", "Vc", "k_ring", "v_ring", "state_k", "state_v")]
    args += [ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
             _stream(stream, dev)]
    _check("rat_stack_prefill", lib().rat_stack_prefill(*args))


def stack_workspace(dtype_code: int, B: int, H: int, T: int, hd: int, dm: int, device):
    """Zero-filled stack workspace (zero it again only after a failed call)."""
    torch = _torch()
    n = rat_stack_workspace_bytes(dtype_code, B, H, T, hd, dm)
    return torch.zeros(((n + 15) // 16) * 4, dtype=torch.int32, device=device)


def layer_workspace(dtype_code: int, B: int, H: int, T: int, hd: int, device):
    """Zero-filled layer workspace (zero it again only after a failed call)."""
    torch = _torch()
    n = rat_layer_workspace_bytes(dtype_code, B, H, T, hd)
    return torch.zeros(((n + 15) // 16) * 4, dtype=torch.int32, device=device)


# ---------------------------------------------------------------------------
# allocation helpers (plumbing: device buffers in the layouts of rat.h)
# ---------------------------------------------------------------------------
def alloc_cache(B: int, H: int, hd: int, T_cap: int, D, W, dtype, device,
                fill=None):
    """Anchor cache, window ring and fp32 state for one layer."""
    torch = _torch()
    R, _ = rat_anchor_rows(H, T_cap, D)
    WS, _ = rat_ring_rows(H, W)

    def mk(shape, dt):
        if fill is None:
            return torch.empty(shape, dtype=dt, device=device)
        return torch.full(shape, fill, dtype=dt, device=device)

    return dict(
        Kc=mk((B, R, hd), dtype), Vc=mk((B, R, hd), dtype),
        k_ring=mk((B, WS, hd), dtype) if WS > 0 else None,
        v_ring=mk((B, WS, hd), dtype) if WS > 0 else None,
        state_k=torch.zeros((B, H, hd), dtype=torch.float32, device=device),
        state_v=torch.zeros((B, H, hd), dtype=torch.float32, device=device),
    )


def scan_workspace(B: int, H: int, T: int, hd: int, device):
    """Zero-filled scan workspace (zero it again only after a failed call)."""
    torch = _torch()
    n = rat_scan_workspace_bytes(B, H, T, hd)
    return torch.zeros(((n + 15) // 16) * 4, dtype=torch.int32, device=device)


def decode_workspace(B: int, H: int, hd: int, T_cap: int, D, W, device,
                     num_splits: int = 0):
    torch = _torch()
    n = rat_decode_workspace_bytes(B, H, hd, T_cap, D, W, num_splits)
    if n == 0:
        return None
    return torch.empty(((n + 15) // 16) * 4, dtype=torch.int32, device=device)


def backward_workspace(B: int, H: int, T: int, hd: int, D, W, device):
    """Zero-filled backward workspace (zero it again only after a failed
    call: uint32 word 2 set)."""
    torch = _torch()
    n = rat_prefill_backward_workspace_bytes(B, H, T, hd, D, W)
    return torch.zeros(((n + 15) // 16) * 4, dtype=torch.int32, device=device)
