"""Python wrappers over the C oracle (``rat_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.

Every function takes and returns float64 numpy arrays in the layouts of the
method: activations ``[B, H, T, hd]``, recurrent state ``[B, H, hd]``,
anchor cache ``[B, R, hd]`` with heads packed at ``off[h]``, window ring
``[B, sum(W), hd]``.  Arithmetic is IEEE double; see ``rat_oracle.c`` for
the definitions and the passages of the pages each one follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rat_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no FP contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
            "-std=c11", "-shared", "-fPIC", "-Wall", "-Wno-unknown-pragmas",
            _SRC, "-o", tmp, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


def load(path: str) -> ctypes.CDLL:
    """Load an oracle shared library and declare its signatures."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    L.rat_oracle_round_bf16.argtypes = [f64]
    L.rat_oracle_round_bf16.restype = f64
    L.rat_oracle_round_bf16_array.argtypes = [i64, P]
    L.rat_oracle_scan.argtypes = [i32, i32, i32, i32, P, P, P, P]
    L.rat_oracle_in_keyset.argtypes = [i64, i64, i32, i32]
    L.rat_oracle_in_keyset.restype = i32
    L.rat_oracle_keyset_size.argtypes = [i64, i32, i32]
    L.rat_oracle_keyset_size.restype = i64
    L.rat_oracle_attention.argtypes = [i32, i32, i32, i32, P, P, f64,
                                       P, P, P, P, P]
    L.rat_oracle_attention_rows.argtypes = [i32, i32, i32, i32, P, P, f64,
                                            P, P, P, i64, P, P, P]
    L.rat_oracle_anchor_offsets.argtypes = [i32, i64, P, P]
    L.rat_oracle_anchor_offsets.restype = i64
    L.rat_oracle_build_cache.argtypes = [i32, i32, i32, i32, P, P, i64,
                                         P, P, P]
    L.rat_oracle_decode_step.argtypes = [i32, i32, i32, P, P, f64, i64,
                                         P, P, P, P, P, P, P, P, i32,
                                         P, P, P]
    L.rat_oracle_backward.argtypes = [i32, i32, i32, i32, P, P, f64, P, P, P,
                                      P, P, i32, P, P, P, P]
    L.rat_oracle_num_threads.restype = i32
    L.rat_oracle_set_threads.argtypes = [i32]
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = load(_LIB)
    return _lib


def build_variant(src_text: str, out_path: str) -> str:
    """Compile an edited copy of the oracle source (used by the tests that
    plant mistakes in the oracle to show that its pins catch them)."""
    c_path = out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp",
                           "-std=c11", "-shared", "-fPIC", "-w", c_path,
                           "-o", out_path, "-lm"])
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().rat_oracle_num_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's loops over (b, h) from here on (timing only)."""
    lib().rat_oracle_set_threads(int(n))


def round_bf16(x) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even), returned as float64."""
    out = np.array(x, dtype=np.float64, copy=True, order="C")
    lib().rat_oracle_round_bf16_array(out.size, _p(out))
    return out


def scan(g, x, want_h: bool = True):
    """Full-sequence gated recurrence over x with gate g ([B,H,T,hd]).

    Returns (h [B,H,T,hd] or None, state [B,H,hd])."""
    g = _f64(g)
    x = _f64(x)
    assert g.shape == x.shape and g.ndim == 4
    B, H, T, hd = g.shape
    h = np.empty_like(x) if want_h else None
    st = np.empty((B, H, hd), dtype=np.float64)
    lib().rat_oracle_scan(B, H, T, hd, _p(g), _p(x), _p(h), _p(st))
    return h, st


def in_keyset(t: int, j: int, D: int, W: int) -> bool:
    return bool(lib().rat_oracle_in_keyset(t, j, D, W))


def keyset_size(t: int, D: int, W: int) -> int:
    return int(lib().rat_oracle_keyset_size(t, D, W))


def attention(q, hk, hv, D, W, scale):
    """Dilated causal softmax attention for all queries.  Returns (o, lse)."""
    q, hk, hv = _f64(q), _f64(hk), _f64(hv)
    B, H, T, hd = q.shape
    D, W = _i32(D), _i32(W)
    assert D.shape == (H,) and W.shape == (H,)
    o = np.empty_like(q)
    lse = np.empty((B, H, T), dtype=np.float64)
    lib().rat_oracle_attention(B, H, T, hd, _p(D), _p(W), float(scale), _p(q),
                               _p(hk), _p(hv), _p(o), _p(lse))
    return o, lse


def attention_rows(q, hk, hv, D, W, scale, rows):
    """Attention for selected (b, h, t) triples only.  Returns (o, lse)."""
    q, hk, hv = _f64(q), _f64(hk), _f64(hv)
    B, H, T, hd = q.shape
    D, W = _i32(D), _i32(W)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    n = rows.shape[0]
    o = np.empty((n, hd), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    lib().rat_oracle_attention_rows(B, H, T, hd, _p(D), _p(W), float(scale),
                                    _p(q), _p(hk), _p(hv), n, _p(rows), _p(o),
                                    _p(lse))
    return o, lse


def anchor_offsets(H: int, T_cap: int, D):
    """Returns (R, off[H+1]) of the packed anchor-only cache."""
    D = _i32(D)
    off = np.zeros(H + 1, dtype=np.int64)
    R = lib().rat_oracle_anchor_offsets(H, T_cap, _p(D), _p(off))
    return int(R), off


def build_cache(hs, D, W, T_cap: int, Kc=None, ring=None):
    """Anchor cache (and window ring) after a prefill of hs ([B,H,T,hd]).

    Rows the definition does not name keep the values of the given arrays
    (NaN-filled by default)."""
    hs = _f64(hs)
    B, H, T, hd = hs.shape
    D, W = _i32(D), _i32(W)
    R, _ = anchor_offsets(H, T_cap, D)
    WS = int(W.sum())
    if Kc is None:
        Kc = np.full((B, R, hd), np.nan)
    Kc = _f64(Kc).copy()
    if WS > 0:
        ring = np.full((B, WS, hd), np.nan) if ring is None else _f64(ring).copy()
    else:
        ring = None
    lib().rat_oracle_build_cache(B, H, T, hd, _p(D), _p(W), T_cap, _p(hs),
                                 _p(Kc), _p(ring))
    return Kc, ring


def prefill(q, k, v, g, D, W, scale, st_bf16: bool):
    """Scan over k and v, optional bf16 storage rounding of the states, then
    dilated attention.  Returns a dict of float64 arrays."""
    hk, sk = scan(g, k)
    hv, sv = scan(g, v)
    if st_bf16:
        hk, hv = round_bf16(hk), round_bf16(hv)
    o, lse = attention(q, hk, hv, D, W, scale)
    return dict(hk=hk, hv=hv, state_k=sk, state_v=sv, o=o, lse=lse)


def decode_step(q, k, v, g, state_k, state_v, hk_hist, hv_hist, D, W, scale,
                pos: int, st_bf16: bool):
    """One decode step at position pos.  q,k,v,g: [B,H,hd]; state: [B,H,hd]
    (not modified); history: [B,H,pos,hd] stored states of positions < pos.
    Returns (o, new_state_k, new_state_v, hat_k, hat_v)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, H, hd = q.shape
    sk = _f64(state_k).copy()
    sv = _f64(state_v).copy()
    hk_hist = _f64(hk_hist)
    hv_hist = _f64(hv_hist)
    assert hk_hist.shape == (B, H, pos, hd)
    D, W = _i32(D), _i32(W)
    o = np.empty((B, H, hd))
    hk_new = np.empty((B, H, hd))
    hv_new = np.empty((B, H, hd))
    lib().rat_oracle_decode_step(B, H, hd, _p(D), _p(W), float(scale), pos,
                                 _p(q), _p(k), _p(v), _p(g), _p(sk), _p(sv),
                                 _p(hk_hist), _p(hv_hist), int(st_bf16), _p(o),
                                 _p(hk_new), _p(hv_new))
    return o, sk, sv, hk_new, hv_new


def backward(q, k, v, g, dO, D, W, scale, st_bf16: bool):
    """Gradients (dq, dk, dv, dg) of a loss whose gradient with respect to
    the prefill output o is dO; all [B,H,T,hd].  See rat_oracle_backward."""
    q, k, v, g, dO = _f64(q), _f64(k), _f64(v), _f64(g), _f64(dO)
    B, H, T, hd = q.shape
    D, W = _i32(D), _i32(W)
    out = [np.empty_like(q) for _ in range(4)]
    lib().rat_oracle_backward(B, H, T, hd, _p(D), _p(W), float(scale), _p(q), _p(k),
                              _p(v), _p(g), _p(dO), int(st_bf16), *[_p(a) for a in out])
    return dict(dq=out[0], dk=out[1], dv=out[2], dg=out[3])


def layer_prefill(x, w_q, w_k, w_v, w_g, b_g, w_o, H: int, hd: int, D, W, scale, st_bf16: bool):
    """One layer over a prefill: projections (numpy matmul in float64; each
    projection output rounded to the storage type, as stored), the gate
    sigmoid(x W_g + b_g), the prefill of this module, and out = o W_o with o
    rounded to the storage type and the heads concatenated.  x: [B,T,dm]."""
    x = _f64(x)
    B, T, dm = x.shape

    def heads(y):  # [B,T,H*hd] -> [B,H,T,hd]
        return np.ascontiguousarray(y.reshape(B, T, H, hd).transpose(0, 2, 1, 3))

    rnd = round_bf16 if st_bf16 else (lambda a: a)
    q = heads(rnd(x @ _f64(w_q)))
    k = heads(rnd(x @ _f64(w_k)))
    v = heads(rnd(x @ _f64(w_v)))
    gpre = heads(rnd(x @ _f64(w_g)))
    g = 1.0 / (1.0 + np.exp(-(gpre + _f64(b_g).reshape(1, H, 1, hd))))
    r = prefill(q, k, v, g, D, W, scale, st_bf16)
    o = rnd(r["o"]).transpose(0, 2, 1, 3).reshape(B, T, H * hd)
    r["out"] = o @ _f64(w_o)
    return r


def stack_prefill(x, layers, H: int, hd: int, scale, st_bf16: bool):
    """A stack of layers over a prefill (the layer-wise hybrid: each layer
    has its own per-head D and W).  layers: one dict per layer with D, W,
    w_q, w_k, w_v, w_g, b_g, w_o.  The input of layer l+1 is the out of
    layer l rounded to the storage type, as stored between layers; nothing
    else (no residual, no normalisation) joins them.  Returns the list of
    per-layer results of layer_prefill; the last one's "out" is the stack's
    output (not rounded)."""
    rnd = round_bf16 if st_bf16 else (lambda a: a)
    res = []
    h = _f64(x)
    for i, ly in enumerate(layers):
        if i > 0:
            h = rnd(res[-1]["out"])
        res.append(layer_prefill(h, ly["w_q"], ly["w_k"], ly["w_v"], ly["w_g"], ly["b_g"],
                                 ly["w_o"], H, hd, ly["D"], ly["W"], scale, st_bf16))
    return res
