"""CPU oracle for one GPU's share of an expert-parallel MoE layer -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this package.
It wraps ``moe_oracle.c`` (plain C, fp64, a per-token loop) with ctypes and numpy arrays.  It shares no code
with the HIP library and imports nothing from it.

Every function cites the page passage it follows in ``moe_oracle.c``.  Parity status: routing, counts,
offsets and the permutation are pinned by library routines and closed forms; the expert FFN is pinned by
special cases (a dense layer through a library matmul, linearity, label permutation, zero input) and by brute
force against an independent vectorised formulation on tiny inputs (see ``tests/test_oracle_pins.py``).  The
backward pass (training gradients of x, the expert weights, the routing weights and the logits) is pinned by
fp64 torch autograd of an independently written forward, by central differences of the forward oracle, and by
the softmax-Jacobian invariant.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_DT = {"f32": 0, "bf16": 1, "fp8": 2}
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (-O2, no fast-math, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", _SRC, "-lm", "-o", tmp],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.orc_bf16_decode.restype = ctypes.c_double
        L.orc_bf16_decode.argtypes = [ctypes.c_uint16]
        L.orc_bf16_encode.restype = ctypes.c_uint16
        L.orc_bf16_encode.argtypes = [ctypes.c_double]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_payload_bytes.restype = ctypes.c_uint64
        L.orc_payload_bytes.argtypes = [i64, i32, i32, i32]
        L.orc_route_topk.restype = ctypes.c_int
        L.orc_route_topk.argtypes = [P, i64, i32, i32, P, P]
        L.orc_dispatch.restype = ctypes.c_int
        L.orc_dispatch.argtypes = [P, i64, i32, i32, P, P, P, P]
        L.orc_moe_tokens.restype = ctypes.c_int
        L.orc_moe_tokens.argtypes = [i32, P, P, i64, i32, P, P, i32, i32, i32, i32, P, P, P, P, P, P, P, i64, P, P]
        L.orc_router_logits.restype = ctypes.c_int
        L.orc_router_logits.argtypes = [i32, P, P, i64, i32, P, i32, P, P]
        L.orc_dispatch_capacity.restype = ctypes.c_int
        L.orc_dispatch_capacity.argtypes = [P, i64, i32, i32, i32, P, P, P, P, P]
        L.orc_combine.restype = ctypes.c_int
        L.orc_combine.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, P]
        bwd_in = [i32, P, i64, i32, P, P, i32, i32, i32, i32, i32, P, P, P, P, P]
        L.orc_bwd_rows.restype = ctypes.c_int
        L.orc_bwd_rows.argtypes = bwd_in + [P, i64, P, P, P, P, P]
        L.orc_bwd_weight_elems.restype = ctypes.c_int
        L.orc_bwd_weight_elems.argtypes = bwd_in + [P, P, P, P, i64, P, P, P]
        L.orc_bwd_weights.restype = ctypes.c_int
        L.orc_bwd_weights.argtypes = bwd_in + [P, P, P, P, P, P, P, P, P]
        L.orc_pair_h.restype = ctypes.c_int
        L.orc_pair_h.argtypes = [i32, P, P, i64, i32, P, i32, i32, i32, i32, P, P, P, P, P, i64, P, P, P, P, P, P, P]
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().orc_num_threads()


def bf16_decode(bits: int) -> float:
    return lib().orc_bf16_decode(bits)


def bf16_encode(v: float) -> int:
    return lib().orc_bf16_encode(v)


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(code)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def payload_bytes(tokens: int, k: int, H: int, bytes_per_elem: int) -> int:
    return lib().orc_payload_bytes(tokens, k, H, bytes_per_elem)


def route_topk(logits: np.ndarray, k: int):
    """-> (topk_idx int32 [T,k], topk_w float64 [T,k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    if lib().orc_route_topk(_p(logits), T, E, k, _p(idx), _p(w)) != 0:
        raise ValueError("oracle route: bad arguments")
    return idx, w


def dispatch(topk_idx: np.ndarray, E: int):
    """-> (counts [E], offsets [E+1], row_of_pair [T*k], token_of_row [T*k]), all int32."""
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = topk_idx.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    rop = np.zeros(T * k, np.int32)
    tor = np.zeros(T * k, np.int32)
    if lib().orc_dispatch(_p(topk_idx), T, k, E, _p(counts), _p(offsets), _p(rop), _p(tor)) != 0:
        raise ValueError("oracle dispatch: bad arguments")
    return counts, offsets, rop, tor


def router_logits(inp, w_router=None):
    """fp64 router logits x W_r [T, E] from the stored x, and sum |x_h W_r[h, e]| [T, E] (for error bounds)."""
    wl = inp.wl
    w = np.ascontiguousarray(inp.w_router if w_router is None else w_router, dtype=np.float32)
    E = w.shape[1]
    logits = np.zeros((wl.T, E), np.float64)
    absdot = np.zeros((wl.T, E), np.float64)
    c = np.ascontiguousarray
    if lib().orc_router_logits(_DT[wl.dtype], _p(c(inp.x)), _p(None if inp.x_scales is None else c(inp.x_scales)),
                               wl.T, wl.H, _p(w), E, _p(logits), _p(absdot)) != 0:
        raise ValueError("oracle router_logits: bad arguments")
    return logits, absdot


def dispatch_capacity(topk_idx: np.ndarray, E: int, capacity: int):
    """Fixed-capacity dispatch: each expert keeps its first ``capacity`` pairs in ascending pair order.

    -> (counts [E] kept, offsets [E+1], row_of_pair [T*k] (-1 = dropped), token_of_row [sum kept], keep [T*k] u8)"""
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = topk_idx.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    rop = np.zeros(T * k, np.int32)
    tor = np.zeros(T * k, np.int32)
    keep = np.zeros(T * k, np.uint8)
    if lib().orc_dispatch_capacity(_p(topk_idx), T, k, E, capacity, _p(counts), _p(offsets), _p(rop), _p(tor),
                                   _p(keep)) != 0:
        raise ValueError("oracle dispatch_capacity: bad arguments")
    return counts, offsets, rop, tor[: int(offsets[E])], keep


def moe_tokens(inp, topk_idx, topk_w, tokens=None, e_lo=None, E_local=None, keep=None) -> np.ndarray:
    """fp64 layer output rows [len(tokens), H] for the given token ids (all tokens by default).

    ``inp`` is a ``moe_inputs.Inputs``; weights are the local experts [e_lo, e_lo + E_local).  ``keep``
    ([T*k] uint8, from dispatch_capacity) drops the pairs marked 0."""
    wl = inp.wl
    if tokens is None:
        tokens = np.arange(wl.T, dtype=np.int64)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    e_lo = wl.e_lo if e_lo is None else e_lo
    E_local = wl.n_local if E_local is None else E_local
    out = np.zeros((len(tokens), wl.H), np.float64)
    c = np.ascontiguousarray
    rc = lib().orc_moe_tokens(
        _DT[wl.dtype], _p(c(inp.x)), _p(None if inp.x_scales is None else c(inp.x_scales)), wl.T, wl.H,
        _p(c(topk_idx, dtype=np.int32)), _p(c(topk_w, dtype=np.float64)), wl.k, e_lo, E_local, wl.F,
        _p(c(inp.w_gate)), _p(c(inp.w_up)), _p(c(inp.w_down)),
        _p(None if inp.s_gate is None else c(inp.s_gate)), _p(None if inp.s_up is None else c(inp.s_up)),
        _p(None if inp.s_down is None else c(inp.s_down)), _p(tokens), len(tokens), _p(out),
        _p(None if keep is None else c(keep, dtype=np.uint8)))
    if rc != 0:
        raise ValueError("oracle moe: bad arguments")
    return out


def pair_h(inp, topk_idx, pairs, e_lo=None, E_local=None) -> dict:
    """The SwiGLU intermediate of the listed pairs p = t*k + j, before and after its storage in the layer dtype.

    -> dict of fp64 [n, F] arrays g, u, gabs, uabs (sums of |terms| of g and u), a = silu(g) * u; h_bits uint32
    [n, F] (fp32 bits, bf16 bits or e4m3 codes); h_scales fp32 [n, F/128] (fp8; None otherwise)."""
    wl = inp.wl
    pairs = np.ascontiguousarray(pairs, dtype=np.int64)
    n, F = len(pairs), wl.F
    e_lo = wl.e_lo if e_lo is None else e_lo
    E_local = wl.n_local if E_local is None else E_local
    res = {name: np.zeros((n, F), np.float64) for name in ("g", "u", "gabs", "uabs", "a")}
    res["h_bits"] = np.zeros((n, F), np.uint32)
    res["h_scales"] = np.zeros((n, F // 128), np.float32) if wl.dtype == "fp8" else None
    c = np.ascontiguousarray
    rc = lib().orc_pair_h(
        _DT[wl.dtype], _p(c(inp.x)), _p(None if inp.x_scales is None else c(inp.x_scales)), wl.T, wl.H,
        _p(c(topk_idx, dtype=np.int32)), wl.k, e_lo, E_local, F, _p(c(inp.w_gate)), _p(c(inp.w_up)),
        _p(None if inp.s_gate is None else c(inp.s_gate)), _p(None if inp.s_up is None else c(inp.s_up)),
        _p(pairs), n, *(_p(res[k]) for k in ("g", "u", "gabs", "uabs", "a", "h_bits")), _p(res["h_scales"]))
    if rc != 0:
        raise ValueError("oracle pair_h: bad arguments")
    return res


def combine(y: np.ndarray, row_of_pair, topk_idx, topk_w, e_lo: int, E_local: int) -> np.ndarray:
    """out [T,H] fp64 = per token, the slot-ordered weighted sum of the local expert-output rows y [R,H]."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = topk_idx.shape
    H = y.shape[1]
    out = np.zeros((T, H), np.float64)
    lib().orc_combine(_p(y), _p(np.ascontiguousarray(row_of_pair, dtype=np.int32)), _p(topk_idx),
                      _p(np.ascontiguousarray(topk_w, dtype=np.float64)), T, k, H, e_lo, E_local, _p(out))
    return out


def layer(inp, tokens=None):
    """Route, dispatch and the expert FFN + weighted sum for one workload's inputs.

    Returns a dict with topk_idx, topk_w, counts, offsets, row_of_pair, token_of_row and out (fp64 rows of the
    requested tokens)."""
    wl = inp.wl
    idx, w = route_topk(inp.logits, wl.k)
    counts, offsets, rop, tor = dispatch(idx, wl.E)
    out = moe_tokens(inp, idx, w, tokens=tokens)
    return dict(topk_idx=idx, topk_w=w, counts=counts, offsets=offsets, row_of_pair=rop, token_of_row=tor, out=out)


def _bwd_common(inp, topk_idx, topk_w, dout, keep, e_lo, E_local):
    wl = inp.wl
    if wl.dtype == "fp8":
        raise ValueError("oracle backward: fp8 layers are not covered")
    c = np.ascontiguousarray
    e_lo = wl.e_lo if e_lo is None else e_lo
    E_local = wl.n_local if E_local is None else E_local
    keep_a = None if keep is None else c(keep, dtype=np.uint8)
    arrs = dict(x=c(inp.x), idx=c(topk_idx, dtype=np.int32), w=c(topk_w, dtype=np.float64),
                wg=c(inp.w_gate), wu=c(inp.w_up), wd=c(inp.w_down), dout=c(dout, dtype=np.float64), keep=keep_a)
    head = [_DT[wl.dtype], _p(arrs["x"]), wl.T, wl.H, _p(arrs["idx"]), _p(arrs["w"]), wl.k, wl.E, e_lo, E_local, wl.F,
            _p(arrs["wg"]), _p(arrs["wu"]), _p(arrs["wd"]), _p(arrs["dout"]), _p(keep_a)]
    return head, arrs


def backward_rows(inp, topk_idx, topk_w, dout, tokens=None, keep=None, e_lo=None, E_local=None, with_abs=False,
                  with_sq=False):
    """Backward of the layer for the listed tokens: (dx [n, H], d_topk_w [n, k], d_logits [n, E]) in fp64, and
    with_abs: also dx_abs [n, H], the sum of |terms| of each dx element (for rounding-error bounds); with_sq: also
    dx_sq [n, H], the sum of the squared terms (for rounding-noise estimates).

    ``dout`` [T, H] is the loss gradient of the layer output; weights are the local experts (natural layouts)."""
    wl = inp.wl
    if tokens is None:
        tokens = np.arange(wl.T, dtype=np.int64)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    head, keepalive = _bwd_common(inp, topk_idx, topk_w, dout, keep, e_lo, E_local)
    n = len(tokens)
    dx = np.zeros((n, wl.H), np.float64)
    dtw = np.zeros((n, wl.k), np.float64)
    dl = np.zeros((n, wl.E), np.float64)
    dxa = np.zeros((n, wl.H), np.float64) if with_abs else None
    dxs = np.zeros((n, wl.H), np.float64) if with_sq else None
    if lib().orc_bwd_rows(*head, _p(tokens), n, _p(dx), _p(dtw), _p(dl), _p(dxa), _p(dxs)) != 0:
        raise ValueError("oracle backward_rows: bad arguments")
    del keepalive
    res = (dx, dtw, dl) + ((dxa,) if with_abs else ()) + ((dxs,) if with_sq else ())
    return res


def backward_weights(inp, topk_idx, topk_w, dout, keep=None, e_lo=None, E_local=None, with_abs=False,
                     with_sq=False):
    """All weight gradients (dWg, dWu [E_local, H, F], dWd [E_local, F, H]) in fp64 (small layers); with_abs:
    also the three arrays of sums of |terms|; with_sq: then the three arrays of sums of squared terms."""
    wl = inp.wl
    El = wl.n_local if E_local is None else E_local
    head, keepalive = _bwd_common(inp, topk_idx, topk_w, dout, keep, e_lo, E_local)
    dwg = np.zeros((El, wl.H, wl.F), np.float64)
    dwu = np.zeros((El, wl.H, wl.F), np.float64)
    dwd = np.zeros((El, wl.F, wl.H), np.float64)
    ab = [np.zeros_like(a) for a in (dwg, dwu, dwd)] if with_abs else [None, None, None]
    sq = [np.zeros_like(a) for a in (dwg, dwu, dwd)] if with_sq else [None, None, None]
    if lib().orc_bwd_weights(*head, _p(dwg), _p(dwu), _p(dwd), *(_p(a) for a in ab), *(_p(a) for a in sq)) != 0:
        raise ValueError("oracle backward_weights: bad arguments")
    del keepalive
    return (dwg, dwu, dwd) + (tuple(ab) if with_abs else ()) + (tuple(sq) if with_sq else ())


def backward_weight_elems(inp, topk_idx, topk_w, dout, which, ex, ii, jj, keep=None, e_lo=None, E_local=None,
                          with_abs=False, with_sq=False):
    """Sampled weight-gradient elements: which 0 dWg[e][c][f], 1 dWu[e][c][f] (ii=c, jj=f), 2 dWd[e][f][c]
    (ii=f, jj=c); e local.  -> fp64 [n] (with_abs: and the sums of |terms| [n]; with_sq: and the sums of squared
    terms [n])."""
    head, keepalive = _bwd_common(inp, topk_idx, topk_w, dout, keep, e_lo, E_local)
    c = lambda a: np.ascontiguousarray(a, dtype=np.int32)
    which, ex, ii, jj = c(which), c(ex), c(ii), c(jj)
    out = np.zeros(len(which), np.float64)
    oab = np.zeros(len(which), np.float64)
    osq = np.zeros(len(which), np.float64)
    if lib().orc_bwd_weight_elems(*head, _p(which), _p(ex), _p(ii), _p(jj), len(which), _p(out), _p(oab),
                                  _p(osq)) != 0:
        raise ValueError("oracle backward_weight_elems: bad arguments")
    del keepalive
    if not with_abs and not with_sq:
        return out
    return (out,) + ((oab,) if with_abs else ()) + ((osq,) if with_sq else ())
