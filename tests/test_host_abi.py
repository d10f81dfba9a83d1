"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

Every call here fails validation, or has an empty batch, before anything is
enqueued, so only host code runs.  Fake device pointers are used only in
calls that are rejected by validation.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from dilated_sparse_attention_rat_amd import binding as rb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rat.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rb.LIB_PATH):
        from dilated_sparse_attention_rat_amd import build
        build.build_library(verbose=False)
    return rb.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rat_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(rb.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", rb.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in _declared():
        assert name in syms, name
        assert hasattr(L, name)


def test_version_and_status_strings(L):
    assert "gfx950" in rb.rat_version()
    for code in (0, -1, -2, -3, -4, -5):
        assert rb.rat_status_string(code) not in ("", "unknown status")
    assert rb.rat_status_string(-99) == "unknown status"


@pytest.mark.parametrize("seed", range(5))
def test_anchor_rows_match_oracle(L, seed):
    rng = np.random.default_rng(seed)
    H = int(rng.integers(1, 40))
    D = rng.integers(1, 70, size=H).astype(np.int32)
    T_cap = int(rng.integers(0, 100000))
    R, off = rb.rat_anchor_rows(H, T_cap, D)
    R2, off2 = oracle.anchor_offsets(H, T_cap, D)
    assert R == R2
    np.testing.assert_array_equal(off, off2)


def test_ring_rows(L):
    W = np.array([0, 5, 128, 0, 7], dtype=np.int32)
    S, off = rb.rat_ring_rows(5, W)
    assert S == 140
    assert list(off) == [0, 0, 5, 133, 133, 140]


def test_layout_functions_reject_bad_tables(L):
    D = np.array([4, 0], dtype=np.int32)
    assert L.rat_anchor_rows(2, 100, D.ctypes.data_as(ctypes.c_void_p), None) == rb.RAT_ERR_INVALID_ARG
    W = np.array([4, -1], dtype=np.int32)
    assert L.rat_ring_rows(2, W.ctypes.data_as(ctypes.c_void_p), None) == rb.RAT_ERR_INVALID_ARG
    assert L.rat_anchor_rows(-1, 100, None, None) == rb.RAT_ERR_INVALID_ARG


def test_workspace_sizes(L):
    assert rb.rat_scan_workspace_bytes(4, 16, 4096, 128) > 0
    assert rb.rat_scan_workspace_bytes(1, 1, 0, 64) > 0
    a = rb.rat_scan_workspace_bytes(1, 16, 16384, 128)
    b = rb.rat_scan_workspace_bytes(2, 16, 16384, 128)
    assert b > a
    assert L.rat_scan_workspace_bytes(1, 1, 10, 96) == rb.RAT_ERR_UNSUPPORTED
    D = np.full(32, 64, np.int32)
    W = np.full(32, 128, np.int32)
    assert rb.rat_decode_workspace_bytes(64, 32, 128, 33024, D, W) == 0  # one split
    assert rb.rat_decode_workspace_bytes(1, 2, 128, 33024, D[:2], W[:2]) > 0
    assert rb.rat_decode_workspace_bytes(1, 2, 128, 1000, D[:2], W[:2], num_splits=4) == 2 * 4 * 130 * 4


# -------------------------------------------------------------------------
# validation paths of the three compute entry points (rejected before any
# launch; fake pointers are never dereferenced)
# -------------------------------------------------------------------------
FAKE = 1 << 20  # 16-byte aligned, never dereferenced


def _p(x=FAKE):
    return ctypes.c_void_p(x)


def _tables(H, D=4, W=0):
    d = np.full(H, D, np.int32)
    w = np.full(H, W, np.int32)
    return d, w, d.ctypes.data_as(ctypes.c_void_p), w.ctypes.data_as(ctypes.c_void_p)


def _scan(L, dtype=0, B=1, H=2, T=16, hd=64, D=4, W=0, T_cap=16, kptr=FAKE, ws=FAKE,
          ws_bytes=1 << 30, state=FAKE, hk=FAKE, hv=FAKE, ring=FAKE):
    d, w, dp, wp = _tables(H, D, W)
    return L.rat_scan_prefill(dtype, B, H, T, hd, dp, wp, T_cap, _p(kptr), _p(), _p(), _p(hk),
                              _p(hv), _p(), _p(), _p(ring), _p(ring), _p(state), _p(state),
                              _p(ws), ws_bytes, None)


def test_scan_validation(L):
    assert _scan(L, dtype=7) == rb.RAT_ERR_UNSUPPORTED
    assert _scan(L, hd=96) == rb.RAT_ERR_UNSUPPORTED
    assert _scan(L, D=0) == rb.RAT_ERR_INVALID_ARG
    assert _scan(L, W=-3) == rb.RAT_ERR_INVALID_ARG
    assert _scan(L, T=17, T_cap=16) == rb.RAT_ERR_CAPACITY
    assert _scan(L, kptr=FAKE + 8) == rb.RAT_ERR_INVALID_ARG       # misaligned
    assert _scan(L, kptr=0) == rb.RAT_ERR_INVALID_ARG              # null input
    assert _scan(L, state=0) == rb.RAT_ERR_INVALID_ARG
    assert _scan(L, hk=0) == rb.RAT_ERR_INVALID_ARG                # hk without hv
    assert _scan(L, W=4, ring=0) == rb.RAT_ERR_INVALID_ARG         # window needs a ring
    assert _scan(L, ws=0) == rb.RAT_ERR_WORKSPACE
    assert _scan(L, ws_bytes=64) == rb.RAT_ERR_WORKSPACE
    assert _scan(L, H=129) == rb.RAT_ERR_UNSUPPORTED
    assert _scan(L, B=-1) == rb.RAT_ERR_INVALID_ARG
    assert _scan(L, B=0) == rb.RAT_OK                              # empty batch: no-op


def _attn(L, dtype=0, B=1, H=2, T=16, hd=64, D=4, W=0, T_cap=16, scale=0.0, q=FAKE, lse=0):
    d, w, dp, wp = _tables(H, D, W)
    return L.rat_dilated_attn_prefill(dtype, B, H, T, hd, dp, wp, scale, T_cap, _p(q), _p(), _p(),
                                      _p(), _p(), _p(), _p(lse) if lse else None, None)


def test_attention_validation(L):
    assert _attn(L, dtype=3) == rb.RAT_ERR_UNSUPPORTED
    assert _attn(L, hd=32) == rb.RAT_ERR_UNSUPPORTED
    assert _attn(L, D=-1) == rb.RAT_ERR_INVALID_ARG
    assert _attn(L, T=20, T_cap=16) == rb.RAT_ERR_CAPACITY
    assert _attn(L, q=0) == rb.RAT_ERR_INVALID_ARG
    assert _attn(L, q=FAKE + 4) == rb.RAT_ERR_INVALID_ARG
    assert _attn(L, lse=FAKE + 4) == rb.RAT_ERR_INVALID_ARG
    assert _attn(L, scale=float("inf")) == rb.RAT_ERR_INVALID_ARG
    assert _attn(L, T=0) == rb.RAT_OK
    assert _attn(L, B=0) == rb.RAT_OK


def _scan_c(L, B=1, H=2, T=8, hd=64, D=4, W=0, T_cap=16, t0=8, sin=FAKE + 4096, sout=FAKE,
            rin=0, ring=FAKE):
    d, w, dp, wp = _tables(H, D, W)
    return L.rat_scan_prefill_continue(0, B, H, T, hd, dp, wp, T_cap, t0, _p(), _p(), _p(),
                                       _p(sin), _p(sin), _p(), _p(), _p(), _p(),
                                       _p(rin) if rin else None, _p(rin) if rin else None,
                                       _p(ring), _p(ring), _p(sout), _p(sout), _p(), 1 << 30,
                                       None)


def test_scan_continue_validation(L):
    assert _scan_c(L, t0=-1) == rb.RAT_ERR_INVALID_ARG
    assert _scan_c(L, t0=10) == rb.RAT_ERR_CAPACITY                # t0 + T > T_cap
    assert _scan_c(L, sin=0) == rb.RAT_ERR_INVALID_ARG             # input state required
    assert _scan_c(L, sin=FAKE) == rb.RAT_ERR_INVALID_ARG          # aliases the output state
    assert _scan_c(L, sin=FAKE + 4100) == rb.RAT_ERR_INVALID_ARG   # misaligned
    assert _scan_c(L, W=4, rin=FAKE + 8) == rb.RAT_ERR_INVALID_ARG
    assert _scan_c(L, B=0) == rb.RAT_OK


def _attn_c(L, B=1, H=2, T=8, hd=64, D=4, W=0, T_cap=16, t0=8, rprev=0):
    d, w, dp, wp = _tables(H, D, W)
    return L.rat_dilated_attn_prefill_continue(0, B, H, T, hd, dp, wp, 0.0, T_cap, t0, _p(),
                                               _p(), _p(), _p(), _p(),
                                               _p(rprev) if rprev else None,
                                               _p(rprev) if rprev else None, _p(), None, None)


def test_attention_continue_validation(L):
    assert _attn_c(L, t0=-2) == rb.RAT_ERR_INVALID_ARG
    assert _attn_c(L, t0=9) == rb.RAT_ERR_CAPACITY
    assert _attn_c(L, W=4) == rb.RAT_ERR_INVALID_ARG               # window keys before t0
    assert _attn_c(L, W=4, rprev=FAKE + 2) == rb.RAT_ERR_INVALID_ARG
    assert _attn_c(L, T=0) == rb.RAT_OK
    assert _attn_c(L, B=0) == rb.RAT_OK


def test_backward_validation(L):
    d, w, dp, wp = _tables(2, 4, 0)
    assert L.rat_prefill_backward_workspace_bytes(1, 2, 100, 128, dp, wp) > 0
    assert L.rat_prefill_backward_workspace_bytes(1, 2, 100, 96, dp, wp) == rb.RAT_ERR_UNSUPPORTED
    assert L.rat_prefill_backward_workspace_bytes(1, 2, -1, 128, dp, wp) == rb.RAT_ERR_INVALID_ARG

    def bwd(dtype=0, T=16, hd=64, ptr=FAKE, ws=FAKE, ws_bytes=1 << 30, B=1):
        return L.rat_prefill_backward(dtype, B, 2, T, hd, dp, wp, 0.0, *([_p(ptr)] * 13),
                                      _p(ws), ws_bytes, None)

    assert bwd(dtype=5) == rb.RAT_ERR_UNSUPPORTED
    assert bwd(hd=32) == rb.RAT_ERR_UNSUPPORTED
    assert bwd(ptr=0) == rb.RAT_ERR_INVALID_ARG
    assert bwd(ptr=FAKE + 2) == rb.RAT_ERR_INVALID_ARG
    assert bwd(ws=0) == rb.RAT_ERR_WORKSPACE
    assert bwd(ws_bytes=64) == rb.RAT_ERR_WORKSPACE
    assert bwd(T=0) == rb.RAT_OK
    assert bwd(B=0) == rb.RAT_OK


def test_layer_validation(L):
    d, w, dp, wp = _tables(2, 4, 0)
    assert L.rat_layer_workspace_bytes(0, 1, 2, 100, 128) > 0
    assert L.rat_layer_workspace_bytes(0, 1, 2, 100, 96) == rb.RAT_ERR_UNSUPPORTED
    assert L.rat_layer_workspace_bytes(3, 1, 2, 100, 128) == rb.RAT_ERR_UNSUPPORTED

    def layer(dm=64, T=16, T_cap=16, ptr=FAKE, ws=FAKE, ws_bytes=1 << 30, B=1, hd=64):
        return L.rat_layer_prefill(0, B, 2, T, hd, dm, dp, wp, 0.0, T_cap, *([_p(ptr)] * 16),
                                   ws_bytes, None) if ws == FAKE else \
            L.rat_layer_prefill(0, B, 2, T, hd, dm, dp, wp, 0.0, T_cap, *([_p(ptr)] * 15),
                                _p(ws) if ws else None, ws_bytes, None)

    assert layer(dm=0) == rb.RAT_ERR_INVALID_ARG
    assert layer(hd=96) == rb.RAT_ERR_UNSUPPORTED
    assert layer(T=17) == rb.RAT_ERR_CAPACITY
    assert layer(ptr=0) == rb.RAT_ERR_INVALID_ARG
    assert layer(ws=0) == rb.RAT_ERR_WORKSPACE
    assert layer(ws_bytes=64) == rb.RAT_ERR_WORKSPACE
    assert layer(B=0) == rb.RAT_OK



def test_stack_validation(L):
    """The stack checks every layer before its first launch: a bad second
    layer (a zero D, a missing weight) is an error with nothing run."""
    H, n = 2, 2
    assert L.rat_stack_workspace_bytes(0, 1, H, 100, 128, 64) > \
        L.rat_layer_workspace_bytes(0, 1, H, 100, 128)
    assert L.rat_stack_workspace_bytes(0, 1, H, 100, 128, 0) == rb.RAT_ERR_INVALID_ARG
    assert L.rat_stack_workspace_bytes(0, 1, H, 100, 96, 64) == rb.RAT_ERR_UNSUPPORTED

    def stack(nl=n, D=4, D2=4, T=16, T_cap=16, ws_bytes=1 << 30, B=1, null_wo2=False,
              null_arr=False):
        d = np.full((max(nl, 1), H), D, np.int32)
        d[-1] = D2
        w = np.zeros((max(nl, 1), H), np.int32)
        arr = (ctypes.c_void_p * max(nl, 1))(*([FAKE] * max(nl, 1)))
        wo = (ctypes.c_void_p * max(nl, 1))(*([FAKE] * max(nl, 1)))
        if null_wo2:
            wo[nl - 1] = None
        a = None if null_arr else arr
        return L.rat_stack_prefill(0, nl, B, H, T, 64, 64, d.ctypes.data_as(ctypes.c_void_p),
                                   w.ctypes.data_as(ctypes.c_void_p), 0.0, T_cap, _p(),
                                   a, arr, arr, arr, arr, wo, _p(), arr, arr, arr, arr, arr, arr,
                                   _p(), ws_bytes, None)

    assert stack(nl=0) == rb.RAT_ERR_INVALID_ARG
    assert stack(null_arr=True) == rb.RAT_ERR_INVALID_ARG
    assert stack(D2=0) == rb.RAT_ERR_INVALID_ARG
    assert stack(null_wo2=True) == rb.RAT_ERR_INVALID_ARG
    assert stack(T=17) == rb.RAT_ERR_CAPACITY
    assert stack(ws_bytes=64) == rb.RAT_ERR_WORKSPACE
    assert stack(B=0) == rb.RAT_OK
    assert stack(B=0, D2=0) == rb.RAT_ERR_INVALID_ARG

def _dec(L, dtype=0, B=1, H=2, hd=64, D=4, W=0, pos=5, T_cap=16, splits=0, ws=0, ws_bytes=0,
         q=FAKE):
    d, w, dp, wp = _tables(H, D, W)
    return L.rat_decode_step(dtype, B, H, hd, dp, wp, 0.0, pos, T_cap, _p(q), _p(), _p(), _p(),
                             _p(), _p(), _p(), _p(), _p(), _p(), _p(), splits,
                             _p(ws) if ws else None, ws_bytes, None)


def test_decode_validation(L):
    assert _dec(L, pos=16, T_cap=16) == rb.RAT_ERR_CAPACITY
    assert _dec(L, pos=-1) == rb.RAT_ERR_INVALID_ARG
    assert _dec(L, dtype=9) == rb.RAT_ERR_UNSUPPORTED
    assert _dec(L, hd=256) == rb.RAT_ERR_UNSUPPORTED
    assert _dec(L, q=0) == rb.RAT_ERR_INVALID_ARG
    assert _dec(L, splits=4) == rb.RAT_ERR_WORKSPACE               # 4 splits need a workspace
    assert _dec(L, splits=4, ws=FAKE, ws_bytes=16) == rb.RAT_ERR_WORKSPACE
    assert _dec(L, splits=-2) == rb.RAT_ERR_INVALID_ARG
    assert _dec(L, B=0) == rb.RAT_OK


def test_decode_noalloc_validation(L):
    """The no-allocation decode validates like rat_decode_step and rejects
    split-K partials beyond its device array before anything is launched."""
    def dec(dtype=0, B=1, H=2, hd=64, pos=5, T_cap=16, splits=0, q=FAKE):
        d, w, dp, wp = _tables(H, 4, 0)
        return L.rat_decode_step_noalloc(dtype, B, H, hd, dp, wp, 0.0, pos, T_cap, _p(q), _p(),
                                         _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(),
                                         splits, None)

    assert dec(pos=16, T_cap=16) == rb.RAT_ERR_CAPACITY
    assert dec(dtype=9) == rb.RAT_ERR_UNSUPPORTED
    assert dec(q=0) == rb.RAT_ERR_INVALID_ARG
    assert dec(splits=-2) == rb.RAT_ERR_INVALID_ARG
    # 64 * 64 (b, h) x 64 splits x (128 + 2) fp32 = 136 MB > the 16 MiB array
    assert 64 * 64 * 64 * 130 * 4 > rb.NOALLOC_SCRATCH_BYTES
    assert dec(B=64, H=64, hd=128, T_cap=1 << 16, splits=64) == rb.RAT_ERR_WORKSPACE
    assert dec(B=0) == rb.RAT_OK


def _tk_build(L, dtype=0, B=1, H=2, T=64, hd=64, T_cap=128, t0=0, ptr=FAKE, means=FAKE):
    return L.rat_topk_cache_build(dtype, B, H, T, hd, T_cap, t0, _p(ptr), _p(ptr), _p(ptr),
                                  _p(ptr), _p(means) if means else None, None)


def test_topk_cache_build_validation(L):
    assert _tk_build(L, dtype=4) == rb.RAT_ERR_UNSUPPORTED
    assert _tk_build(L, hd=32) == rb.RAT_ERR_UNSUPPORTED
    assert _tk_build(L, T=129) == rb.RAT_ERR_CAPACITY
    assert _tk_build(L, T=64, t0=65) == rb.RAT_ERR_CAPACITY        # t0 + T > T_cap
    assert _tk_build(L, T=-1) == rb.RAT_ERR_INVALID_ARG
    assert _tk_build(L, t0=-1) == rb.RAT_ERR_INVALID_ARG
    assert _tk_build(L, T=10, t0=60, means=0) == rb.RAT_ERR_INVALID_ARG  # block 0 ends here

    assert _tk_build(L, ptr=0) == rb.RAT_ERR_INVALID_ARG
    assert _tk_build(L, ptr=FAKE + 4) == rb.RAT_ERR_INVALID_ARG
    assert _tk_build(L, means=0) == rb.RAT_ERR_INVALID_ARG          # a complete block needs means
    assert _tk_build(L, means=FAKE + 8) == rb.RAT_ERR_INVALID_ARG
    assert _tk_build(L, B=0) == rb.RAT_OK
    assert _tk_build(L, T=0) == rb.RAT_OK


def _tk_dec(L, dtype=0, B=1, H=2, hd=64, D=4, W=0, pos=70, T_cap=128, k=4, scale=0.0, q=FAKE,
            hist=FAKE, means=FAKE, ring=FAKE):
    d, w, dp, wp = _tables(H, D, W)
    return L.rat_decode_step_topk(dtype, B, H, hd, dp, wp, scale, pos, T_cap, k, _p(q), _p(),
                                  _p(), _p(), _p(), _p(), _p(), _p(), _p(ring), _p(ring),
                                  _p(hist), _p(hist), _p(means) if means else None, _p(), None,
                                  None)


def test_topk_decode_validation(L):
    assert _tk_dec(L, pos=128) == rb.RAT_ERR_CAPACITY
    assert _tk_dec(L, pos=-1) == rb.RAT_ERR_INVALID_ARG
    assert _tk_dec(L, k=-1) == rb.RAT_ERR_INVALID_ARG
    assert _tk_dec(L, k=rb.TOPK_MAX_K + 1) == rb.RAT_ERR_UNSUPPORTED
    assert _tk_dec(L, T_cap=64 * 8192 + 64, pos=5) == rb.RAT_ERR_UNSUPPORTED  # block table limit
    assert _tk_dec(L, dtype=2) == rb.RAT_ERR_UNSUPPORTED
    assert _tk_dec(L, hd=16) == rb.RAT_ERR_UNSUPPORTED
    assert _tk_dec(L, D=0) == rb.RAT_ERR_INVALID_ARG
    assert _tk_dec(L, scale=float("nan")) == rb.RAT_ERR_INVALID_ARG
    assert _tk_dec(L, q=0) == rb.RAT_ERR_INVALID_ARG
    assert _tk_dec(L, hist=0) == rb.RAT_ERR_INVALID_ARG
    assert _tk_dec(L, hist=FAKE + 2) == rb.RAT_ERR_INVALID_ARG
    assert _tk_dec(L, means=0) == rb.RAT_ERR_INVALID_ARG
    assert _tk_dec(L, W=8, ring=0) == rb.RAT_ERR_INVALID_ARG         # window needs a ring
    assert _tk_dec(L, B=0) == rb.RAT_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(rb, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(rb, "_lib", None)
    with pytest.raises(ImportError):
        rb.lib()
