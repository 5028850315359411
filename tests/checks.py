"""Comparison rules shared by the GPU parity tests and their CPU self-tests (no GPU, no library code).

check_h: the stored SwiGLU intermediate h (as the grouped FFN's gate/up product leaves it in its workspace)
against the oracle's values for the same (token, pick) pairs.  h is a rounding of a = silu(g) u to the layer
dtype, so its elements are integers decided by floating point: away from a rounding midpoint the stored element
is unique and must equal the oracle's bit for bit; within the GPU arithmetic's error of a midpoint either
neighbour is correct, and the element must be one of the two.  The GPU's error in a is bounded from the oracle's
own sums of |terms|:
  |a_gpu - a| <= kappa (|u silu'(g)| gabs + |silu(g)| uabs) + 8 2^-24 |a|,
kappa = 2^-14 for fp8 products: gfx950's fp8 MFMA sums the 128 products of an instruction with a precision of its
own, then the block scales multiply and the blocks accumulate in fp32; on the parity shapes the stored codes
needed at most 1.1e-5 (about 2^-16.5) of the sums of |terms|, and the bound keeps a factor of 5 above that.
(H + 16) 2^-24 for bf16 / fp32 products: the worst case of fp32 accumulation over H terms (the codes needed
2e-8).  The 8 ulps cover silu(g) u in fp32.  For fp8 the scale of a group,
max|a| / 448, may differ by the bound of its largest element, and the code of a / scale then by that relative
change as well.
"""
from __future__ import annotations

import numpy as np
import torch

KAPPA_FP8 = 2.0**-14


def kappa(dtype: str, H: int) -> float:
    return KAPPA_FP8 if dtype == "fp8" else (H + 16) * 2.0**-24


def a_bound(ref: dict, dtype: str, H: int) -> np.ndarray:
    """Bound on |a_gpu - a| per element, from the oracle's g, u and their sums of |terms|."""
    g, u = ref["g"], ref["u"]
    sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = sig * (1.0 + g * (1.0 - sig))
    k = kappa(dtype, H)
    return k * (np.abs(u * dsilu) * ref["gabs"] + np.abs(silu) * ref["uabs"]) + 8 * 2.0**-24 * np.abs(ref["a"])


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    """Values of OCP e4m3 codes through torch's float8_e4m3fn type (a library decode)."""
    c = torch.from_numpy(np.ascontiguousarray(codes.astype(np.uint8)))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_values(bits: np.ndarray) -> np.ndarray:
    b = torch.from_numpy(np.ascontiguousarray(bits.astype(np.uint16)).view(np.int16))
    return b.view(torch.bfloat16).to(torch.float64).numpy()


def midpoint_window(dtype: str, H: int, ref: dict):
    """Elements of the oracle's h whose exact value lies within the GPU's error bound of a rounding midpoint
    (either neighbour is then a correct stored value), and for those the change of the stored value (scale
    applied) if the other neighbour is stored: (mask [n, F] bool, delta [n, F] float64, 0 outside the mask)."""
    a = ref["a"]
    da = a_bound(ref, dtype, H)
    rb = ref["h_bits"].astype(np.uint32)
    if dtype == "fp8":
        n, F = a.shape
        sr = np.repeat(ref["h_scales"].astype(np.float64), 128, axis=1)
        # the GPU's scale lies in [max(|a| - bound), max(|a| + bound)] / 448 over the group
        ga, gd = np.abs(a).reshape(n, F // 128, 128), da.reshape(n, F // 128, 128)
        srel = ((ga + gd).max(axis=2) - np.maximum(ga - gd, 0).max(axis=2)) / np.maximum(ga.max(axis=2), 1e-300)
        v = a / sr
        dv = da / sr + np.abs(v) * (np.repeat(srel, 128, axis=1) + 2.0**-22)
        dec, mag_mask, top = e4m3_values, 0x7F, 0x7E
    elif dtype == "bf16":
        sr = 1.0
        v, dv = a, da
        dec, mag_mask, top = bf16_values, 0x7FFF, 0x7F7F
    else:
        return np.zeros(a.shape, bool), np.zeros(a.shape)
    rmag = rb & mag_mask
    rval = np.abs(dec(rb))
    above = np.abs(dec(np.where(rmag < top, rb + 1, rb)))
    below = np.abs(dec(np.where(rmag > 0, rb - 1, rb)))
    d_up = np.abs(np.abs(v) - (rval + above) / 2)
    d_dn = np.abs(np.abs(v) - (rval + below) / 2)
    up = d_up <= d_dn
    mask = np.minimum(d_up, d_dn) <= dv
    delta = np.where(up, above - rval, rval - below) * sr
    return mask, np.where(mask, delta, 0.0)


def check_h(dtype: str, H: int, ref: dict, got_bits: np.ndarray, got_scales: np.ndarray | None = None) -> dict:
    """Raise AssertionError unless every stored element satisfies the rule above; return statistics (elements,
    elements within their bound of a midpoint, differing elements, and the largest |v - midpoint| / bound among
    the differing ones)."""
    a = ref["a"]
    da = a_bound(ref, dtype, H)
    rb = ref["h_bits"].astype(np.uint32)
    got_bits = got_bits.astype(np.uint32)
    if dtype != "f32":  # -0 and +0 are the same value
        neg0 = np.uint32(0x80 if dtype == "fp8" else 0x8000)
        rb = np.where(rb == neg0, np.uint32(0), rb)
        got_bits = np.where(got_bits == neg0, np.uint32(0), got_bits)
    stats = dict(elements=int(a.size))
    if dtype == "f32":
        gv = got_bits.astype(np.uint32).view(np.float32).astype(np.float64)
        ulp = np.spacing(np.abs(a).astype(np.float32)).astype(np.float64)
        bad = np.abs(gv - a) > da + ulp
        assert not bad.any(), f"{int(bad.sum())} fp32 h elements outside their bound"
        stats.update(window=0, differing=int((got_bits != rb).sum()), worst=0.0, kappa_needed=0.0)
        return stats
    if dtype == "bf16":
        v = a
        dv = da
        gval, rval = bf16_values(got_bits), bf16_values(rb)
        gmag, rmag = got_bits & 0x7FFF, rb & 0x7FFF
        gsgn, rsgn = got_bits >> 15, rb >> 15
        step_up = bf16_values(np.where(rmag < 0x7F7F, rb + 1, rb)) - rval  # spacing above |ref| (same sign)
    else:
        s_ref = ref["h_scales"].astype(np.float64)
        s_got = got_scales.astype(np.float64)
        F = a.shape[1]
        # the GPU's group maximum lies in [max(|a| - bound), max(|a| + bound)] over the group's elements
        ga = np.abs(a).reshape(len(a), F // 128, 128)
        gd = da.reshape(len(a), F // 128, 128)
        s_lo = np.maximum(ga - gd, 0).max(axis=2) / 448.0
        s_hi = (ga + gd).max(axis=2) / 448.0
        ulp2 = 2.0 * np.spacing(s_ref.astype(np.float32)).astype(np.float64)
        zero = ga.max(axis=2) == 0
        bad_s = ~zero & ((s_got < s_lo - ulp2) | (s_got > s_hi + ulp2))
        bad_s |= zero & (s_got != 1.0)
        assert not bad_s.any(), f"{int(bad_s.sum())} fp8 h scales outside their bound"
        sr = np.repeat(s_ref, 128, axis=1)
        sg = np.repeat(s_got, 128, axis=1)
        v = a / sr
        dv = da / sr + np.abs(v) * np.abs(sg - sr) / sr + 2.0**-22 * np.abs(v)
        gval, rval = e4m3_values(got_bits), e4m3_values(rb)
        gmag, rmag = got_bits & 0x7F, rb & 0x7F
        gsgn, rsgn = got_bits >> 7, rb >> 7
        step_up = e4m3_values(np.where(rmag < 0x7E, rb + 1, rb)) - rval
    # elements within their bound of a midpoint (where either neighbour is a correct rounding)
    below = np.where(rmag > 0, rb - 1, rb)  # the next smaller magnitude (same sign)
    step_dn = np.abs(rval) - np.abs(e4m3_values(below) if dtype == "fp8" else bf16_values(below))
    d_up = np.abs(np.abs(v) - (np.abs(rval) + np.abs(step_up) / 2))  # to the midpoint above |ref|
    d_dn = np.abs(np.abs(v) - (np.abs(rval) - step_dn / 2))  # to the midpoint below |ref|
    window = np.minimum(d_up, d_dn) <= dv
    diff = got_bits != rb
    stats["window"] = int(window.sum())
    stats["differing"] = int(diff.sum())
    if not diff.any():
        stats["worst"] = stats["kappa_needed"] = 0.0
        return stats
    # a differing element is correct when its code is the rounding of some value within the bound of the exact
    # value: the code's rounding interval (half a step to either side) comes within dv of v
    dec = e4m3_values if dtype == "fp8" else bf16_values
    gb = got_bits[diff]
    top = 0x7E if dtype == "fp8" else 0x7F7F
    gm = gb & (0x7F if dtype == "fp8" else 0x7FFF)
    g_up = np.abs(dec(np.where(gm < top, gb + 1, gb)))
    g_dn = np.abs(dec(np.where(gm > 0, gb - 1, gb)))
    gv = np.abs(gval[diff])
    lo = np.where(gm > 0, (gv + g_dn) / 2, 0.0)  # the code's rounding interval in magnitude
    hi = np.where(gm < top, (gv + g_up) / 2, np.inf)
    sgn_ok = (gsgn[diff] == (v[diff] < 0)) | (gm == 0)
    av = np.abs(v[diff])
    dist = np.where(av < lo, lo - av, np.where(av > hi, av - hi, 0.0))  # |v| to the interval
    dist = np.where(sgn_ok, dist, av + lo)
    ok = dist <= dv[diff]
    # the smallest kappa that would admit each differing element (the measured size of the GPU's error)
    w = dv[diff] / kappa(dtype, H)
    stats["kappa_needed"] = float(np.max(dist / np.maximum(w, 1e-300)))
    n_bad = int((~ok).sum())
    if n_bad:
        i = np.nonzero(~ok)[0][:5]
        raise AssertionError(f"{n_bad} of {int(diff.sum())} differing h elements are not roundings of a value "
                             f"within the bound: v {v[diff][i]}, gpu {gval[diff][i]}, oracle {rval[diff][i]}, "
                             f"distance / bound {dist[i] / dv[diff][i]}")
    stats["worst"] = float(np.max(dist / dv[diff]))
    return stats


# ------------------------------------------------------------------------------------------------------------
# rounding noise of a sum of terms that each carry one operand rounded to the layer dtype
# ------------------------------------------------------------------------------------------------------------
UNIT = {"f32": 2.0**-24, "bf16": 2.0**-8}


def noise_ratio(got: np.ndarray, ref: np.ndarray, sq: np.ndarray, K: int, dtype: str, out_rounded: bool) -> float:
    """sqrt(sum err^2 / sum var) over the elements, var = (u^2 / 3 + K 2^-48 / 6) S + (u_out^2 / 3) ref^2 with S
    the oracle's sum of squared terms of the element: a rounding to a p-bit significand has relative RMS at most
    2^(1-p) / sqrt(12) = u / sqrt(3), independent per term; K fp32 additions add a random-walk share; u_out is the
    output's own rounding (u when the output is stored in the layer dtype, else 2^-24).  A correct result sits
    below 1 (the model takes the largest relative RMS); a dropped term of typical size, repeated over a tile
    edge or a reduction stage, lifts it far above, also where the elementwise worst-case bound (which grows with
    the sum of |terms|) still holds."""
    u = UNIT[dtype]
    uo = u if out_rounded else 2.0**-24
    var = (u * u / 3.0 + K * 2.0**-48 / 6.0) * sq + (uo * uo / 3.0) * ref * ref
    s = float(np.sum(var))
    e = float(np.sum((got - ref) ** 2))
    return float(np.sqrt(e / s)) if s > 0 else (0.0 if e == 0 else float("inf"))
