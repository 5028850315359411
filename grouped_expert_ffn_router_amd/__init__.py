"""Python binding of libmoe_ep.so: one GPU's share of an expert-parallel MoE layer on MI355X.

Thin ctypes marshalling over the C ABI in ``include/moe_ep.h``; every step of the layer runs in the HIP
kernels of the library.  torch supplies device memory and streams only.  There is no fallback: if the
library is missing the import fails, and a non-OK status raises (``ValueError`` for invalid arguments,
``NotImplementedError`` for unsupported requests, ``RuntimeError`` otherwise).

Functions carry the C names:

    moe_route_topk        logits [T, E] fp32                  -> topk_idx [T, k] int32, topk_w [T, k] fp32
    moe_router_topk       x [T, H] (+ fp8 scales), W_r [H, E] -> logits [T, E] fp32, topk_idx, topk_w
    moe_dispatch_permute  x [T, H] (+ fp8 scales), topk_idx   -> counts, offsets, row_of_pair, token_of_row,
                                                                 x_perm [T*k, H] (+ fp8 scales)
    moe_pack_ffn_weights  natural-layout expert weights       -> PackedWeights (init time)
    moe_grouped_ffn       x_perm, offsets, PackedWeights      -> y_perm [T*k, H] fp32
    moe_combine           y_perm, row_of_pair, picks          -> out [T, H]
    moe_payload_bytes     the dispatch + combine closed form 2 * k * H * bytes * tokens
    moe_grouped_ffn_train     moe_grouped_ffn keeping h and the gate/up pre-activations (training)
    moe_grouped_ffn_backward  dout -> dx, expert weight gradients, routing-weight and logit gradients

``MoELayer`` chains the four calls with preallocated buffers for repeated use.

Streams: every call enqueues on ``stream`` (a ``torch.cuda.Stream``, a raw ``hipStream_t`` handle, or None for the
current stream).  Outputs and workspaces a wrapper allocates itself are allocated on that stream, as torch's own
ops allocate on the stream they run on; with a raw handle the caller passes every buffer.
"""
from __future__ import annotations

import contextlib
import ctypes
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_ep.so")

MOE_DTYPE_F32, MOE_DTYPE_BF16, MOE_DTYPE_FP8_E4M3 = 0, 1, 2
MOE_LAYOUT_NATURAL, MOE_LAYOUT_PACKED = 0, 1
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)

# every symbol include/moe_ep.h declares
EXPORTS = [
    "moe_status_string", "moe_abi_version", "moe_last_error", "moe_route_topk", "moe_dispatch_workspace_bytes",
    "moe_dispatch_permute", "moe_pack_ffn_weights_bytes", "moe_pack_ffn_weights", "moe_grouped_ffn_workspace_bytes",
    "moe_grouped_ffn", "moe_grouped_ffn_gate_up", "moe_grouped_ffn_down", "moe_combine", "moe_payload_bytes",
    "moe_grouped_ffn_gate_up_gather", "moe_grouped_ffn_down_scatter", "moe_grouped_ffn_fused", "moe_combine_slots",
    "moe_dispatch_permute_capacity", "moe_router_topk", "moe_grouped_ffn_train",
    "moe_grouped_ffn_backward_workspace_bytes", "moe_grouped_ffn_backward", "moe_dispatch_permute_noalloc",
]


class FfnWeights(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int), ("layout", ctypes.c_int), ("E_local", ctypes.c_int32), ("H", ctypes.c_int32),
        ("F", ctypes.c_int32), ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "moe_status_string": (ctypes.c_char_p, [st]),
        "moe_abi_version": (ctypes.c_int, []),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_route_topk": (st, [P, i64, i32, i32, P, P, P]),
        "moe_router_topk": (st, [P, P, st, i64, i32, P, i32, i32, P, P, P, P]),
        "moe_grouped_ffn_train": (st, [P, P, i32, i64, ctypes.POINTER(FfnWeights), P, P, P, P, sz, P]),
        "moe_grouped_ffn_backward_workspace_bytes": (sz, [ctypes.POINTER(FfnWeights), i64]),
        "moe_grouped_ffn_backward": (st, [P, i64, i32, i32, P, P, P, P, P, i32, i64, P, P, P, P,
                                          ctypes.POINTER(FfnWeights), P, P, P, P, P, P, P, sz, P]),
        "moe_dispatch_workspace_bytes": (sz, [i64, i32, i32]),
        "moe_dispatch_permute": (st, [P, P, st, i64, i32, P, i32, i32, P, P, P, P, P, P, P, sz, P]),
        "moe_pack_ffn_weights_bytes": (sz, [ctypes.POINTER(FfnWeights)]),
        "moe_pack_ffn_weights": (st, [ctypes.POINTER(FfnWeights), P, sz, ctypes.POINTER(FfnWeights), P]),
        "moe_grouped_ffn_workspace_bytes": (sz, [ctypes.POINTER(FfnWeights), i64]),
        "moe_grouped_ffn": (st, [P, P, P, i32, i64, ctypes.POINTER(FfnWeights), P, P, sz, P]),
        "moe_grouped_ffn_gate_up": (st, [P, P, P, i32, i64, ctypes.POINTER(FfnWeights), P, sz, P]),
        "moe_grouped_ffn_down": (st, [P, i32, i64, ctypes.POINTER(FfnWeights), P, P, sz, P]),
        "moe_combine": (st, [P, P, P, P, i64, i32, i32, i32, i32, P, st, P]),
        "moe_payload_bytes": (ctypes.c_uint64, [i64, i32, i32, i32]),
        "moe_grouped_ffn_gate_up_gather": (st, [P, P, P, i64, P, i32, i64, ctypes.POINTER(FfnWeights), P, sz, P]),
        "moe_grouped_ffn_down_scatter": (st, [P, i32, i64, ctypes.POINTER(FfnWeights), P, P, P, i64, i32, P, P, sz,
                                              P]),
        "moe_grouped_ffn_fused": (st, [P, P, P, P, P, i64, i32, P, i32, i64, ctypes.POINTER(FfnWeights), P, P, sz,
                                       P]),
        "moe_combine_slots": (st, [P, P, P, i64, i32, i32, i32, i32, P, st, P]),
        "moe_dispatch_permute_capacity": (st, [P, P, st, i64, i32, P, i32, i32, i32, P, P, P, P, P, P, P, sz, P]),
        "moe_dispatch_permute_noalloc": (st, [P, P, st, i64, i32, P, i32, i32, P, P, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def _check(status: int, what: str):
    if status == MOE_OK:
        return
    msg = f"{what}: {lib.moe_status_string(status).decode()}: {lib.moe_last_error().decode()}"
    if status == MOE_ERR_INVALID_ARG:
        raise ValueError(msg)
    if status == MOE_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _alloc_on(stream):
    """Context for a wrapper's own allocations (outputs, workspaces): the stream its kernels are enqueued on, so
    torch's caching allocator ties the memory to that stream and reuses it only for later work on it.  With a
    raw stream handle the caller passes every buffer instead."""
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, torch.cuda.Stream):
        return torch.cuda.stream(stream)

    class _NoAlloc:
        def __enter__(self):
            raise ValueError("a raw stream handle needs caller-provided outputs and workspaces (or a torch.cuda.Stream)")

        def __exit__(self, *exc):
            return False

    return _NoAlloc()


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return MOE_DTYPE_F32
    if t == torch.bfloat16:
        return MOE_DTYPE_BF16
    if t in (torch.uint8, torch.float8_e4m3fn):
        return MOE_DTYPE_FP8_E4M3
    raise ValueError(f"unsupported dtype {t}")


def moe_payload_bytes(tokens: int, k: int, H: int, bytes_per_elem: int) -> int:
    return lib.moe_payload_bytes(tokens, k, H, bytes_per_elem)


def moe_route_topk(logits, k, topk_idx=None, topk_w=None, stream=None):
    T, E = logits.shape
    dev = logits.device
    if topk_idx is None or topk_w is None:
        with _alloc_on(stream):
            if topk_idx is None:
                topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
            if topk_w is None:
                topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(lib.moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_w), _stream(stream)), "moe_route_topk")
    return topk_idx, topk_w


def moe_router_topk(x, w_router, k, x_scales=None, logits=None, topk_idx=None, topk_w=None, want_logits=True,
                    stream=None):
    """Router logits x W_r (fp32) and the softmax top-k in one call; returns (logits or None, topk_idx, topk_w)."""
    T, H = x.shape
    E = w_router.shape[1]
    dev = x.device
    if (logits is None and want_logits) or topk_idx is None or topk_w is None:
        with _alloc_on(stream):
            if logits is None and want_logits:
                logits = torch.empty((T, E), dtype=torch.float32, device=dev)
            if topk_idx is None:
                topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
            if topk_w is None:
                topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(lib.moe_router_topk(_ptr(x), _ptr(x_scales), dtype_code(x.dtype), T, H, _ptr(w_router), E, k,
                               _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _stream(stream)), "moe_router_topk")
    return logits, topk_idx, topk_w


@dataclasses.dataclass
class Dispatch:
    counts: torch.Tensor
    offsets: torch.Tensor
    row_of_pair: torch.Tensor
    token_of_row: torch.Tensor
    x_perm: torch.Tensor
    x_perm_scales: torch.Tensor | None


def moe_dispatch_workspace_bytes(T, k, E) -> int:
    return lib.moe_dispatch_workspace_bytes(T, k, E)


def moe_dispatch_permute(x, topk_idx, E, x_scales=None, out: Dispatch | None = None, workspace=None, stream=None,
                         gather=True, capacity=None):
    """gather=False: counts, offsets and the permutation only (x_perm stays None), for the fused form.
    capacity: each expert keeps its first `capacity` pairs (row_of_pair -1 for the others); x_perm then has
    min(T*k, E*capacity) rows."""
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    dt = dtype_code(x.dtype)
    rows = T * k if capacity is None else min(T * k, E * capacity)
    need = moe_dispatch_workspace_bytes(T, k, E)
    if out is None or workspace is None:
        with _alloc_on(stream):
            if out is None:
                out = Dispatch(
                    counts=torch.empty(E, dtype=torch.int32, device=dev),
                    offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                    row_of_pair=torch.empty(T * k, dtype=torch.int32, device=dev),
                    token_of_row=torch.empty(T * k, dtype=torch.int32, device=dev),
                    x_perm=torch.empty((rows, H), dtype=x.dtype, device=dev) if gather else None,
                    x_perm_scales=(torch.empty((rows, H // 128), dtype=torch.float32, device=dev)
                                   if x_scales is not None and gather else None),
                )
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if capacity is None:
        _check(lib.moe_dispatch_permute(
            _ptr(x), _ptr(x_scales), dt, T, H, _ptr(topk_idx), k, E, _ptr(out.counts), _ptr(out.offsets),
            _ptr(out.row_of_pair), _ptr(out.token_of_row), _ptr(out.x_perm), _ptr(out.x_perm_scales),
            _ptr(workspace), workspace.numel(), _stream(stream)), "moe_dispatch_permute")
    else:
        _check(lib.moe_dispatch_permute_capacity(
            _ptr(x), _ptr(x_scales), dt, T, H, _ptr(topk_idx), k, E, capacity, _ptr(out.counts), _ptr(out.offsets),
            _ptr(out.row_of_pair), _ptr(out.token_of_row), _ptr(out.x_perm), _ptr(out.x_perm_scales),
            _ptr(workspace), workspace.numel(), _stream(stream)), "moe_dispatch_permute_capacity")
    return out


def moe_dispatch_permute_noalloc(x, topk_idx, E, out: Dispatch, x_scales=None, stream=None):
    """moe_dispatch_permute with the library's fixed scratch instead of a workspace (nothing is allocated by the
    call or here: the outputs are the caller's preallocated ``out``; x_perm None = the permutation only)."""
    T, H = x.shape
    k = topk_idx.shape[1]
    _check(lib.moe_dispatch_permute_noalloc(
        _ptr(x), _ptr(x_scales), dtype_code(x.dtype), T, H, _ptr(topk_idx), k, E, _ptr(out.counts),
        _ptr(out.offsets), _ptr(out.row_of_pair), _ptr(out.token_of_row), _ptr(out.x_perm), _ptr(out.x_perm_scales),
        _stream(stream)), "moe_dispatch_permute_noalloc")
    return out


@dataclasses.dataclass
class PackedWeights:
    desc: FfnWeights
    storage: torch.Tensor  # owns the packed matrices
    scales: tuple  # keeps the fp8 scale tensors alive
    dtype: int
    E_local: int
    H: int
    F: int


def moe_pack_ffn_weights(w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None, stream=None) -> PackedWeights:
    """Natural-layout weights (w_gate, w_up [E_local, H, F]; w_down [E_local, F, H]) -> packed layout."""
    E_local, H, F = w_gate.shape
    dt = dtype_code(w_gate.dtype)
    src = FfnWeights(dt, MOE_LAYOUT_NATURAL, E_local, H, F, w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr(),
                     s_gate.data_ptr() if s_gate is not None else None, s_up.data_ptr() if s_up is not None else None,
                     s_down.data_ptr() if s_down is not None else None)
    nbytes = lib.moe_pack_ffn_weights_bytes(ctypes.byref(src))
    with _alloc_on(stream):
        storage = torch.empty(nbytes, dtype=torch.uint8, device=w_gate.device)
    packed = FfnWeights()
    _check(lib.moe_pack_ffn_weights(ctypes.byref(src), _ptr(storage), nbytes, ctypes.byref(packed), _stream(stream)),
           "moe_pack_ffn_weights")
    return PackedWeights(packed, storage, (s_gate, s_up, s_down), dt, E_local, H, F)


def moe_grouped_ffn_workspace_bytes(weights: "PackedWeights", R_max: int) -> int:
    return lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(weights.desc), R_max)


def moe_grouped_ffn(x_perm, offsets, weights: PackedWeights, x_perm_scales=None, e_lo=0, y_perm=None,
                    workspace=None, stream=None):
    R_max = x_perm.shape[0]
    dev = x_perm.device
    need = moe_grouped_ffn_workspace_bytes(weights, R_max)
    if y_perm is None or workspace is None:
        with _alloc_on(stream):
            if y_perm is None:
                y_perm = torch.empty((R_max, weights.H), dtype=torch.float32, device=dev)
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib.moe_grouped_ffn(_ptr(x_perm), _ptr(x_perm_scales), _ptr(offsets), e_lo, R_max,
                               ctypes.byref(weights.desc), _ptr(y_perm), _ptr(workspace), workspace.numel(),
                               _stream(stream)), "moe_grouped_ffn")
    return y_perm


def moe_grouped_ffn_gate_up(x_perm, offsets, weights: PackedWeights, workspace, x_perm_scales=None, e_lo=0,
                            stream=None):
    """First half of moe_grouped_ffn: h (in the workspace) = silu(x_perm Wg) * (x_perm Wu)."""
    _check(lib.moe_grouped_ffn_gate_up(_ptr(x_perm), _ptr(x_perm_scales), _ptr(offsets), e_lo, x_perm.shape[0],
                                       ctypes.byref(weights.desc), _ptr(workspace), workspace.numel(),
                                       _stream(stream)), "moe_grouped_ffn_gate_up")


def moe_grouped_ffn_down(offsets, weights: PackedWeights, workspace, y_perm, e_lo=0, stream=None):
    """Second half of moe_grouped_ffn: y_perm = h Wd, h read from the workspace."""
    _check(lib.moe_grouped_ffn_down(_ptr(offsets), e_lo, y_perm.shape[0], ctypes.byref(weights.desc), _ptr(y_perm),
                                    _ptr(workspace), workspace.numel(), _stream(stream)), "moe_grouped_ffn_down")
    return y_perm


def moe_grouped_ffn_train(x_perm, offsets, weights: PackedWeights, e_lo=0, h=None, gu=None, y_perm=None,
                          workspace=None, stream=None):
    """moe_grouped_ffn keeping what the backward needs: returns (h [R, F], gu [R, 2F] fp32, y_perm [R, H] fp32)."""
    R_max = x_perm.shape[0]
    dev = x_perm.device
    if h is None or gu is None or y_perm is None or workspace is None:
        with _alloc_on(stream):
            if h is None:
                h = torch.empty((R_max, weights.F), dtype=x_perm.dtype, device=dev)
            if gu is None:
                gu = torch.empty((R_max, 2 * weights.F), dtype=torch.float32, device=dev)
            if y_perm is None:
                y_perm = torch.empty((R_max, weights.H), dtype=torch.float32, device=dev)
            if workspace is None:
                workspace = torch.empty(moe_grouped_ffn_workspace_bytes(weights, R_max), dtype=torch.uint8,
                                        device=dev)
    _check(lib.moe_grouped_ffn_train(_ptr(x_perm), _ptr(offsets), e_lo, R_max, ctypes.byref(weights.desc), _ptr(h),
                                     _ptr(gu), _ptr(y_perm), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_grouped_ffn_train")
    return h, gu, y_perm


def natural_weights(w_gate, w_up, w_down) -> FfnWeights:
    """Descriptor of natural-layout weights (w_gate, w_up [E_local, H, F]; w_down [E_local, F, H]); the tensors
    must stay alive while it is used."""
    E_local, H, F = w_gate.shape
    return FfnWeights(dtype_code(w_gate.dtype), MOE_LAYOUT_NATURAL, E_local, H, F, w_gate.data_ptr(),
                      w_up.data_ptr(), w_down.data_ptr(), None, None, None)


def moe_grouped_ffn_backward(dout, topk_idx, topk_w, row_of_pair, token_of_row, offsets, x_perm, h, gu, y_perm,
                             w_gate, w_up, w_down, E, e_lo=0, want_logits=True, out=None, workspace=None,
                             stream=None):
    """Gradients of the layer for dout = dL/dout [T, H]: returns dict(dx, dw_gate, dw_up, dw_down, d_topk_w,
    d_logits) (weights in natural layouts; d_logits None unless wanted)."""
    T, k = topk_idx.shape
    H = dout.shape[1]
    E_local, _, F = w_gate.shape
    R_max = x_perm.shape[0]
    dev = dout.device
    desc = natural_weights(w_gate, w_up, w_down)
    need = lib.moe_grouped_ffn_backward_workspace_bytes(ctypes.byref(desc), R_max)
    if out is None or workspace is None:
        with _alloc_on(stream):
            if out is None:
                out = dict(dx=torch.empty((T, H), dtype=dout.dtype, device=dev),
                           dw_gate=torch.empty((E_local, H, F), dtype=torch.float32, device=dev),
                           dw_up=torch.empty((E_local, H, F), dtype=torch.float32, device=dev),
                           dw_down=torch.empty((E_local, F, H), dtype=torch.float32, device=dev),
                           d_topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
                           d_logits=torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None)
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib.moe_grouped_ffn_backward(
        _ptr(dout), T, k, E, _ptr(topk_idx), _ptr(topk_w), _ptr(row_of_pair), _ptr(token_of_row), _ptr(offsets),
        e_lo, R_max, _ptr(x_perm), _ptr(h), _ptr(gu), _ptr(y_perm), ctypes.byref(desc), _ptr(out["dx"]),
        _ptr(out["dw_gate"]), _ptr(out["dw_up"]), _ptr(out["dw_down"]), _ptr(out["d_topk_w"]), _ptr(out["d_logits"]),
        _ptr(workspace), workspace.numel(), _stream(stream)), "moe_grouped_ffn_backward")
    return out


def moe_combine(y_perm, row_of_pair, topk_idx, topk_w, e_lo=0, E_local=None, out_dtype=torch.bfloat16, out=None,
                stream=None):
    T, k = topk_idx.shape
    H = y_perm.shape[1]
    if E_local is None:
        raise ValueError("moe_combine: E_local is required")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((T, H), dtype=out_dtype, device=y_perm.device)
    _check(lib.moe_combine(_ptr(y_perm), _ptr(row_of_pair), _ptr(topk_idx), _ptr(topk_w), T, k, H, e_lo, E_local,
                           _ptr(out), dtype_code(out.dtype), _stream(stream)), "moe_combine")
    return out


def moe_grouped_ffn_gate_up_gather(x, token_of_row, offsets, weights: PackedWeights, workspace, x_scales=None,
                                   e_lo=0, stream=None):
    """Gate/up product reading rows x[token_of_row[r]] directly (no x_perm); h goes to the workspace."""
    _check(lib.moe_grouped_ffn_gate_up_gather(_ptr(x), _ptr(x_scales), _ptr(token_of_row), x.shape[0], _ptr(offsets),
                                              e_lo, token_of_row.shape[0], ctypes.byref(weights.desc),
                                              _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_grouped_ffn_gate_up_gather")


def moe_grouped_ffn_down_scatter(offsets, weights: PackedWeights, workspace, token_of_row, row_of_pair, topk_w,
                                 y_slot, e_lo=0, stream=None):
    """Down product writing topk_w[p] * (h[r] Wd) into pair-major slots y_slot[p] (p: row_of_pair[p] == r)."""
    T, k = topk_w.shape
    _check(lib.moe_grouped_ffn_down_scatter(_ptr(offsets), e_lo, token_of_row.shape[0], ctypes.byref(weights.desc),
                                            _ptr(token_of_row), _ptr(row_of_pair), _ptr(topk_w), T, k,
                                            _ptr(y_slot), _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_grouped_ffn_down_scatter")
    return y_slot


def moe_grouped_ffn_fused(x, token_of_row, row_of_pair, topk_w, offsets, weights: PackedWeights, x_scales=None,
                          e_lo=0, y_slot=None, workspace=None, stream=None):
    T, k = topk_w.shape
    R_max = token_of_row.shape[0]
    dev = x.device
    if y_slot is None or workspace is None:
        with _alloc_on(stream):
            if y_slot is None:
                y_slot = torch.empty((T * k, weights.H), dtype=torch.float32, device=dev)
            if workspace is None:
                workspace = torch.empty(moe_grouped_ffn_workspace_bytes(weights, R_max), dtype=torch.uint8,
                                        device=dev)
    _check(lib.moe_grouped_ffn_fused(_ptr(x), _ptr(x_scales), _ptr(token_of_row), _ptr(row_of_pair), _ptr(topk_w), T,
                                     k, _ptr(offsets), e_lo, R_max, ctypes.byref(weights.desc), _ptr(y_slot),
                                     _ptr(workspace), workspace.numel(), _stream(stream)), "moe_grouped_ffn_fused")
    return y_slot


def moe_combine_slots(y_slot, topk_idx, e_lo=0, E_local=None, out_dtype=torch.bfloat16, out=None, stream=None,
                      row_of_pair=None):
    T, k = topk_idx.shape
    H = y_slot.shape[1]
    if E_local is None:
        raise ValueError("moe_combine_slots: E_local is required")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((T, H), dtype=out_dtype, device=y_slot.device)
    _check(lib.moe_combine_slots(_ptr(y_slot), _ptr(row_of_pair), _ptr(topk_idx), T, k, H, e_lo, E_local, _ptr(out),
                                 dtype_code(out.dtype), _stream(stream)), "moe_combine_slots")
    return out


class MoELayer:
    """The four calls with buffers allocated once for a fixed (T, H, E, k, F) and dtype.

    ``weights`` are natural-layout tensors already on the device; they are packed at construction.
    ``form``:
      "permuted" (default) the dispatch writes x_perm, the grouped FFN reads it, the combine un-permutes y_perm;
      "fused"    (or ``fused=True``) the dispatch builds only the permutation, the gate/up product gathers x rows
                 itself and the down product writes weighted pair-major slots that the combine sums;
      "gather"   the gate/up product gathers x rows itself (no x_perm), then the permuted down product and
                 combine: the same bits as "permuted" without the permuted copy of x.
    ``train``: also keeps the natural-layout weights and the buffers of forward_train() / backward()."""

    FORMS = ("permuted", "fused", "gather")

    def __init__(self, T, H, E, k, F, dtype: torch.dtype, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None,
                 e_lo=0, out_dtype=None, device="cuda", fused=False, train=False, form=None):
        form = form or ("fused" if fused else "permuted")
        if form not in self.FORMS:
            raise ValueError(f"MoELayer: form {form!r} is not one of {self.FORMS}")
        if train and form != "permuted":
            raise ValueError("MoELayer: the training form uses the permuted layout (form='permuted')")
        self.form = form
        self.fused = form == "fused"
        gather_in = form != "permuted"
        self.T, self.H, self.E, self.k, self.F = T, H, E, k, F
        self.e_lo = e_lo
        self.E_local = w_gate.shape[0]
        self.dtype = dtype
        self.fp8 = dtype_code(dtype) == MOE_DTYPE_FP8_E4M3
        self.out_dtype = out_dtype or (torch.float32 if dtype == torch.float32 else torch.bfloat16)
        self.weights = moe_pack_ffn_weights(w_gate, w_up, w_down, s_gate, s_up, s_down)
        R = T * k
        d = device
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=d)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=d)
        self.disp = Dispatch(
            counts=torch.empty(E, dtype=torch.int32, device=d),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=d),
            row_of_pair=torch.empty(R, dtype=torch.int32, device=d),
            token_of_row=torch.empty(R, dtype=torch.int32, device=d),
            x_perm=None if gather_in else torch.empty((R, H), dtype=dtype, device=d),
            x_perm_scales=torch.empty((R, H // 128), dtype=torch.float32, device=d) if self.fp8 and not gather_in
            else None,
        )
        self.ws_disp = torch.empty(moe_dispatch_workspace_bytes(T, k, E), dtype=torch.uint8, device=d)
        self.ws_ffn = torch.empty(moe_grouped_ffn_workspace_bytes(self.weights, R), dtype=torch.uint8, device=d)
        self.y_perm = torch.empty((R, H), dtype=torch.float32, device=d)
        self.out = torch.empty((T, H), dtype=self.out_dtype, device=d)
        self.train = train
        if train:
            self.w_nat = (w_gate, w_up, w_down)
            El = self.E_local
            self.h = torch.empty((R, F), dtype=dtype, device=d)
            self.gu = torch.empty((R, 2 * F), dtype=torch.float32, device=d)
            self.grads = dict(dx=torch.empty((T, H), dtype=dtype, device=d),
                              dw_gate=torch.empty((El, H, F), dtype=torch.float32, device=d),
                              dw_up=torch.empty((El, H, F), dtype=torch.float32, device=d),
                              dw_down=torch.empty((El, F, H), dtype=torch.float32, device=d),
                              d_topk_w=torch.empty((T, k), dtype=torch.float32, device=d),
                              d_logits=torch.empty((T, E), dtype=torch.float32, device=d))
            desc = natural_weights(*self.w_nat)
            self.ws_bwd = torch.empty(lib.moe_grouped_ffn_backward_workspace_bytes(ctypes.byref(desc), R),
                                      dtype=torch.uint8, device=d)

    def forward_train(self, stream=None):
        """The grouped FFN keeping h and the pre-activations for backward() (after route and dispatch)."""
        return moe_grouped_ffn_train(self.disp.x_perm, self.disp.offsets, self.weights, self.e_lo, self.h, self.gu,
                                     self.y_perm, self.ws_ffn, stream)

    def backward(self, dout, stream=None):
        """Gradients for dout = dL/dout [T, H] of the last forward_train(): dx, expert weight, routing-weight and
        logit gradients (dict of preallocated tensors)."""
        return moe_grouped_ffn_backward(dout, self.topk_idx, self.topk_w, self.disp.row_of_pair,
                                        self.disp.token_of_row, self.disp.offsets, self.disp.x_perm, self.h, self.gu,
                                        self.y_perm, *self.w_nat, E=self.E, e_lo=self.e_lo, out=self.grads,
                                        workspace=self.ws_bwd, stream=stream)

    def route(self, logits, stream=None):
        return moe_route_topk(logits, self.k, self.topk_idx, self.topk_w, stream)

    def route_x(self, x, w_router, x_scales=None, stream=None):
        """Routing from the hidden rows: router logits x W_r and the top-k (one kernel for E <= 64; above, the
        logits go through a buffer kept by the layer)."""
        lg = None
        if self.E > 64:
            if getattr(self, "router_logits", None) is None:
                self.router_logits = torch.empty((self.T, self.E), dtype=torch.float32, device=x.device)
            lg = self.router_logits
        _, idx, w = moe_router_topk(x, w_router, self.k, x_scales, lg, self.topk_idx, self.topk_w,
                                    want_logits=lg is not None, stream=stream)
        return idx, w

    def dispatch(self, x, x_scales=None, stream=None):
        self.x, self.x_scales = x, x_scales  # the fused gate/up product reads them
        return moe_dispatch_permute(x, self.topk_idx, self.E, x_scales, self.disp, self.ws_disp, stream,
                                    gather=self.form == "permuted")

    def gate_up(self, stream=None):
        if self.form != "permuted":
            return moe_grouped_ffn_gate_up_gather(self.x, self.disp.token_of_row, self.disp.offsets, self.weights,
                                                  self.ws_ffn, self.x_scales, self.e_lo, stream)
        return moe_grouped_ffn_gate_up(self.disp.x_perm, self.disp.offsets, self.weights, self.ws_ffn,
                                       self.disp.x_perm_scales, self.e_lo, stream)

    def down(self, stream=None):
        if self.fused:
            return moe_grouped_ffn_down_scatter(self.disp.offsets, self.weights, self.ws_ffn, self.disp.token_of_row,
                                                self.disp.row_of_pair, self.topk_w, self.y_perm, self.e_lo, stream)
        return moe_grouped_ffn_down(self.disp.offsets, self.weights, self.ws_ffn, self.y_perm, self.e_lo, stream)

    def ffn(self, stream=None):
        if self.fused:
            return moe_grouped_ffn_fused(self.x, self.disp.token_of_row, self.disp.row_of_pair, self.topk_w,
                                         self.disp.offsets, self.weights, self.x_scales, self.e_lo, self.y_perm,
                                         self.ws_ffn, stream)
        if self.form == "gather":
            self.gate_up(stream)
            return self.down(stream)
        return moe_grouped_ffn(self.disp.x_perm, self.disp.offsets, self.weights, self.disp.x_perm_scales, self.e_lo,
                               self.y_perm, self.ws_ffn, stream)

    def combine(self, stream=None):
        if self.fused:
            return moe_combine_slots(self.y_perm, self.topk_idx, self.e_lo, self.E_local, out=self.out, stream=stream)
        return moe_combine(self.y_perm, self.disp.row_of_pair, self.topk_idx, self.topk_w, self.e_lo, self.E_local,
                           out=self.out, stream=stream)

    def forward(self, logits, x, x_scales=None, stream=None):
        self.route(logits, stream)
        self.dispatch(x, x_scales, stream)
        self.ffn(stream)
        return self.combine(stream)
