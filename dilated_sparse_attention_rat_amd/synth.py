"""Seeded synthetic workloads for the RAT+ hot path.

This module only draws and stores inputs; it performs none of the method's
arithmetic.  Both the parity tests (which feed the CPU oracle) and the
benchmark draw their inputs from here, so the two sides see identical
values.

Workloads.  The pages evaluate on public text suites that are not used here;
these synthetic tensors stand in for them in shape only: sequence lengths of
4K-32K tokens and dilations 4-64, which is the operating range the pages
discuss (RAT+ abstract; zhichai.net deep dive, sections 7.1 and 7.3), and
the head-wise hybrid of section 六 (two dense heads, the rest at D = 4).

Recipe.  ``numpy.random.default_rng(seed)`` (PCG64) standard normals in
float32, drawn in the order q, k, v, g over the full ``[B, H, T, hd]``
shape; q, k, v are scaled by ``qkv_std``; ``g = sigmoid(z + g_bias)``; bf16
workloads are then rounded to bfloat16 (nearest, ties to even).  The decode
workload's 16 GiB-per-tensor context is drawn on the device with
``torch.Generator`` one batch row at a time (seed ``1000*seed + b``, order k,
v, g), and its per-step inputs likewise (seed ``1000*seed + 500 + step``,
order q, k, v, g over ``[B, H, hd]``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    hd: int
    T: int                 # prefill length (context length for decode)
    D: tuple               # per-head dilation
    W: tuple               # per-head window
    dtype: str             # "bf16" or "f32"
    qkv_std: float
    g_bias: float
    seed: int
    decode_steps: int = 0  # > 0 for the decode workload
    note: str = field(default="", compare=False)

    @property
    def T_cap(self) -> int:
        return self.T + self.decode_steps

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.hd)


def _heads(v, H):
    return tuple(int(x) for x in (v if isinstance(v, (list, tuple)) else [v] * H))


WORKLOADS = {
    0: Workload("tiny-f32", 1, 2, 64, 256, _heads(4, 2), _heads(0, 2), "f32",
                1.0, 2.0, 0),
    1: Workload("prefill-1.5B-like", 4, 16, 128, 4096, _heads(16, 16),
                _heads(0, 16), "bf16", 1.0 / math.sqrt(128), 3.0, 1),
    2: Workload("long-prefill-window", 1, 16, 128, 16384, _heads(64, 16),
                _heads(256, 16), "bf16", 1.0 / math.sqrt(128), 3.0, 2),
    3: Workload("decode", 64, 32, 128, 32768, _heads(64, 32), _heads(128, 32),
                "bf16", 1.0 / math.sqrt(128), 3.0, 3, decode_steps=256),
    4: Workload("headwise-hybrid-7.6B-like", 2, 32, 128, 8192,
                _heads([1, 1] + [4] * 30, 32), _heads(0, 32), "bf16",
                1.0 / math.sqrt(128), 3.0, 4),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _sigmoid32(z: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-z, dtype=np.float32))).astype(np.float32)


def draw(shape, seed: int, qkv_std: float, g_bias: float, dtype: str,
         names=("q", "k", "v", "g")):
    """Draw q, k, v, g of ``shape`` with the recipe above.

    Returns a dict name -> float32 array holding exactly the stored values
    (bf16-representable when dtype == "bf16")."""
    rng = np.random.default_rng(seed)
    out = {}
    for n in names:
        z = rng.standard_normal(shape, dtype=np.float32)
        if n == "g":
            a = _sigmoid32(z + np.float32(g_bias))
        else:
            a = z * np.float32(qkv_std)
        if dtype == "bf16":
            a = bf16_to_f32(bf16_bits(a))
        out[n] = np.ascontiguousarray(a, dtype=np.float32)
    return out


def prefill_inputs(w: Workload, B=None, H=None, T=None):
    """Inputs for a prefill workload (optionally at reduced B/H/T, drawn with
    the workload's own law and seed)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    return draw((B, H, T, w.hd), w.seed, w.qkv_std, w.g_bias, w.dtype)


def random_case(seed: int, B: int, H: int, T: int, hd: int, dtype: str,
                qkv_std: float = 1.0, g_bias: float = 2.0):
    """Small random case for parity tests (same recipe, arbitrary shape)."""
    return draw((B, H, T, hd), seed, qkv_std, g_bias, dtype)


# ---------------------------------------------------------------------------
# device-side drawing for the decode workload (torch is plumbing only here)
# ---------------------------------------------------------------------------
def _torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def draw_device(shape, seed: int, qkv_std: float, g_bias: float, dtype: str,
                names, device="cuda"):
    """Draw tensors on the device with torch.Generator (order = names)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = {}
    for n in names:
        z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        a = torch.sigmoid(z + g_bias) if n == "g" else z * qkv_std
        out[n] = a.to(_torch_dtype(dtype)).contiguous()
    return out


def decode_context_row(w: Workload, b: int, device="cuda", T=None):
    """k, v, g of batch row b of the decode workload's context ([1,H,T,hd])."""
    T = w.T if T is None else T
    return draw_device((1, w.H, T, w.hd), 1000 * w.seed + b, w.qkv_std,
                       w.g_bias, w.dtype, ("k", "v", "g"), device)


def decode_step_inputs(w: Workload, step: int, device="cuda", B=None):
    """q, k, v, g ([B,H,hd]) for decode step ``step`` (position T + step)."""
    B = w.B if B is None else B
    return draw_device((B, w.H, w.hd), 1000 * w.seed + 500 + step, w.qkv_std,
                       w.g_bias, w.dtype, ("q", "k", "v", "g"), device)
