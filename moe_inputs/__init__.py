"""Seeded synthetic inputs for one GPU's share of an expert-parallel MoE layer.

This module draws random numbers and stores them in the layer's storage dtypes. It holds none of the layer's
arithmetic: no routing, no sorting, no expert FFN, no combine. The CPU oracle and the HIP path both consume the
exact bytes it returns, so the two implementations see identical inputs.

Workloads (the five layer shapes of the benchmark and the parity tests):

=================  =====  ====  ===  ==  =====  ======  =========================================
name               T      H     E    k   F      dtype   logits
=================  =====  ====  ===  ==  =====  ======  =========================================
tiny_fp32          256    128   8    2   256    f32     x @ W_r, W_r ~ N(0, 1/H)
mixtral_bf16       2048   4096  8    2   14336  bf16    x @ W_r, W_r ~ N(0, 1/H)
decode_bf16        64     7168  32   8   2048   bf16    N(0, 1) per token x expert
dsv3_fp8           8192   7168  32   8   2048   fp8     N(0, 1) per token x expert
skewed_bf16        16384  4096  64   4   1536   bf16    N(0, 1) + b_e, b_e = 2 ln((e+1)^-1.2)
=================  =====  ====  ===  ==  =====  ======  =========================================

Recipe (numpy PCG64, ``default_rng(seed)``; draws happen in this order):

1. ``x ~ N(0, 1)`` of shape [T, H] in fp32, stored as the layer dtype.  fp8 rows are stored as OCP e4m3
   codes with one fp32 scale per row per 128 columns, ``scale = amax / 448`` (1 when the group is all zero).
2. Router logits [T, E] fp32, per the table.  For the ``x @ W_r`` kind, ``W_r ~ N(0, 1) / sqrt(H)`` is drawn
   as [H, E] fp32 and the logits are the fp64 product of the *stored* x values with ``W_r``, rounded once to
   fp32.
3. For each local expert e in order: ``W_gate[e]``, ``W_up[e] ~ N(0, 1) / sqrt(H)`` of shape [H, F], then
   ``W_down[e] ~ N(0, 1) / sqrt(F)`` of shape [F, H], drawn in fp32 and stored as the layer dtype.  fp8
   weights carry one fp32 scale per 128 x 128 block, ``scale = amax / 448``.

Rounding to bf16 and fp8 uses torch's dtype casts (round to nearest even); the generator only decides what the
stored bytes are, and both consumers read those bytes.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_inputs", "Inputs", "ELEM_BYTES"]

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
FP8_MAX = 448.0
QBLOCK = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int  # experts the router chooses among
    k: int
    F: int
    dtype: str  # "f32" | "bf16" | "fp8"
    logits: str  # "router" | "gauss" | "zipf"
    seed: int
    e_lo: int = 0  # first local expert of the window
    E_local: int | None = None  # local experts (default: all E)

    @property
    def n_local(self) -> int:
        return self.E if self.E_local is None else self.E_local

    @property
    def out_dtype(self) -> str:
        return "f32" if self.dtype == "f32" else "bf16"

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", T=256, H=128, E=8, k=2, F=256, dtype="f32", logits="router", seed=1001),
        Workload("mixtral_bf16", T=2048, H=4096, E=8, k=2, F=14336, dtype="bf16", logits="router", seed=1002),
        Workload("decode_bf16", T=64, H=7168, E=32, k=8, F=2048, dtype="bf16", logits="gauss", seed=1003),
        Workload("dsv3_fp8", T=8192, H=7168, E=32, k=8, F=2048, dtype="fp8", logits="gauss", seed=1004),
        Workload("skewed_bf16", T=16384, H=4096, E=64, k=4, F=1536, dtype="bf16", logits="zipf", seed=1005),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


@dataclasses.dataclass
class Inputs:
    """Host arrays of one workload.  Storage dtypes: f32 -> float32, bf16 -> uint16 bit patterns,
    fp8 -> uint8 OCP e4m3 codes (plus float32 scales)."""

    wl: Workload
    x: np.ndarray  # [T, H]
    x_scales: np.ndarray | None  # fp8: [T, H/128] float32
    logits: np.ndarray  # [T, E] float32
    w_gate: np.ndarray  # [E_local, H, F]
    w_up: np.ndarray  # [E_local, H, F]
    w_down: np.ndarray  # [E_local, F, H]
    s_gate: np.ndarray | None  # fp8: [E_local, H/128, F/128]
    s_up: np.ndarray | None
    s_down: np.ndarray | None  # fp8: [E_local, F/128, H/128]
    w_router: np.ndarray | None = None  # "router" logits kind: W_r [H, E] float32


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Stored bf16 bit patterns -> float32 values (exact widening)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def _to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def e4m3_codes_to_f32(c: np.ndarray) -> np.ndarray:
    import torch

    return torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def _group_scale(amax: np.ndarray) -> np.ndarray:
    s = (amax.astype(np.float32) / np.float32(FP8_MAX)).astype(np.float32)
    s[amax == 0] = 1.0
    return s


def _quant_rows(a: np.ndarray):
    """[R, C] fp32 -> e4m3 codes [R, C] + scales [R, C/128]: one scale per row per 128 columns."""
    R, C = a.shape
    g = a.reshape(R, C // QBLOCK, QBLOCK)
    s = _group_scale(np.abs(g).max(axis=2))
    codes = _to_e4m3_codes(g / s[:, :, None])
    return codes.reshape(R, C), s


def _quant_blocks(a: np.ndarray):
    """[K, N] fp32 -> e4m3 codes [K, N] + scales [K/128, N/128]: one scale per 128 x 128 block."""
    K, N = a.shape
    g = a.reshape(K // QBLOCK, QBLOCK, N // QBLOCK, QBLOCK)
    s = _group_scale(np.abs(g).max(axis=(1, 3)))
    codes = _to_e4m3_codes(g / s[:, None, :, None])
    return codes.reshape(K, N), s


def _store(a: np.ndarray, dtype: str):
    if dtype == "f32":
        return a.astype(np.float32), None
    if dtype == "bf16":
        return _to_bf16_bits(a), None
    raise ValueError(dtype)


def stored_x_values(inp: Inputs) -> np.ndarray:
    """float64 values of the stored x (exact decode of the stored bytes, scales applied)."""
    wl = inp.wl
    if wl.dtype == "f32":
        return inp.x.astype(np.float64)
    if wl.dtype == "bf16":
        return bf16_bits_to_f32(inp.x).astype(np.float64)
    v = e4m3_codes_to_f32(inp.x).astype(np.float64).reshape(wl.T, wl.H // QBLOCK, QBLOCK)
    return (v * inp.x_scales.astype(np.float64)[:, :, None]).reshape(wl.T, wl.H)


def make_inputs(wl: Workload, seed: int | None = None, with_weights: bool = True) -> Inputs:
    """Draw one workload's inputs (see the module docstring for the recipe)."""
    if wl.H % QBLOCK or wl.F % QBLOCK:
        raise ValueError("H and F must be multiples of 128")
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    T, H, E, F = wl.T, wl.H, wl.E, wl.F
    dt = wl.dtype

    # 1. activations
    x32 = rng.standard_normal((T, H), dtype=np.float32)
    if dt == "fp8":
        x, x_scales = _quant_rows(x32) if T else (np.zeros((0, H), np.uint8), np.zeros((0, H // QBLOCK), np.float32))
    else:
        x, x_scales = _store(x32, dt)
    del x32

    # 2. router logits
    w_r = None
    if wl.logits == "router":
        w_r = (rng.standard_normal((H, E), dtype=np.float32) / np.float32(math.sqrt(H))).astype(np.float32)
        tmp = Inputs(wl, x, x_scales, None, None, None, None, None, None, None)
        logits = (stored_x_values(tmp) @ w_r.astype(np.float64)).astype(np.float32)
    elif wl.logits == "gauss":
        logits = rng.standard_normal((T, E), dtype=np.float32)
    elif wl.logits == "zipf":
        bias = np.array([2.0 * math.log(1.0 / (e + 1) ** 1.2) for e in range(E)], dtype=np.float32)
        logits = (rng.standard_normal((T, E), dtype=np.float32) + bias[None, :]).astype(np.float32)
    else:
        raise ValueError(wl.logits)

    # 3. expert weights (local experts only)
    El = wl.n_local
    if not with_weights:
        return Inputs(wl, x, x_scales, logits, None, None, None, None, None, None, w_r)
    ebytes = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dt]
    w_gate = np.empty((El, H, F), ebytes)
    w_up = np.empty((El, H, F), ebytes)
    w_down = np.empty((El, F, H), ebytes)
    s_gate = s_up = s_down = None
    if dt == "fp8":
        s_gate = np.empty((El, H // QBLOCK, F // QBLOCK), np.float32)
        s_up = np.empty_like(s_gate)
        s_down = np.empty((El, F // QBLOCK, H // QBLOCK), np.float32)
    inv_h = np.float32(1.0 / math.sqrt(H))
    inv_f = np.float32(1.0 / math.sqrt(F))
    for e in range(El):
        g = rng.standard_normal((H, F), dtype=np.float32) * inv_h
        u = rng.standard_normal((H, F), dtype=np.float32) * inv_h
        d = rng.standard_normal((F, H), dtype=np.float32) * inv_f
        if dt == "fp8":
            w_gate[e], s_gate[e] = _quant_blocks(g)
            w_up[e], s_up[e] = _quant_blocks(u)
            w_down[e], s_down[e] = _quant_blocks(d)
        else:
            w_gate[e] = _store(g, dt)[0]
            w_up[e] = _store(u, dt)[0]
            w_down[e] = _store(d, dt)[0]
    return Inputs(wl, x, x_scales, logits, w_gate, w_up, w_down, s_gate, s_up, s_down, w_r)
