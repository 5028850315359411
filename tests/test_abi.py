"""The C-ABI library loads, exports every function include/moe_ep.h declares, and rejects bad arguments on the
host before touching the GPU (CPU only: no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ep.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    import grouped_expert_ffn_router_amd as m

    names = declared_functions()
    assert len(names) >= 12
    assert sorted(names) == sorted(m.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert m.lib.moe_abi_version() == 1


def test_payload_closed_form_through_the_abi():
    import grouped_expert_ffn_router_amd as m

    assert m.moe_payload_bytes(1, 8, 7168, 1) == 114688
    assert m.moe_payload_bytes(8000, 8, 7168, 1) * 50 == 45_875_200_000
    assert m.moe_payload_bytes(1, 8, 2 * 7168, 1) == 2 * 114688
    assert m.moe_payload_bytes(-1, 8, 7168, 1) == 0


def _st(code):
    import grouped_expert_ffn_router_amd as m

    return m.lib.moe_status_string(code).decode()


def test_validation_rejects_before_launch():
    import grouped_expert_ffn_router_amd as m

    L = m.lib
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first
    odd = ctypes.c_void_p(0x10002)
    # route: k > E, E = 0, k > 32, negative T, T*k overflow, NULL and misaligned pointers
    assert _st(L.moe_route_topk(fake, 10, 4, 5, fake, fake, None)) == "MOE_ERR_INVALID_ARG"
    assert "k = 5" in L.moe_last_error().decode()
    assert L.moe_route_topk(fake, 10, 0, 1, fake, fake, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(fake, 10, 64, 33, fake, fake, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(fake, -1, 8, 2, fake, fake, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(fake, 1 << 30, 8, 2, fake, fake, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(None, 10, 8, 2, fake, fake, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(fake, 10, 8, 2, odd, fake, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(fake, 10, 2000, 2, fake, fake, None) == m.MOE_ERR_INVALID_ARG
    # T = 0 is a successful no-op
    assert L.moe_route_topk(None, 0, 8, 2, None, None, None) == m.MOE_OK
    # dispatch: H not a multiple of 128, bad dtype, missing fp8 scales, workspace too small
    ws = m.moe_dispatch_workspace_bytes(100, 2, 8)
    big = ctypes.c_void_p(0x100000)
    args = lambda **kw: [kw.get("x", fake), kw.get("xs", None), kw.get("dt", m.MOE_DTYPE_BF16), kw.get("T", 100),
                         kw.get("H", 256), fake, kw.get("k", 2), kw.get("E", 8), fake, fake, fake, fake, fake,
                         kw.get("xps", None), kw.get("ws", big), kw.get("wsb", ws), None]
    assert L.moe_dispatch_permute(*args(H=100)) == m.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch_permute(*args(dt=7)) == m.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch_permute(*args(dt=m.MOE_DTYPE_FP8_E4M3)) == m.MOE_ERR_INVALID_ARG
    assert "x_scales" in L.moe_last_error().decode()
    assert L.moe_dispatch_permute(*args(wsb=ws - 1)) == m.MOE_ERR_WORKSPACE
    assert L.moe_dispatch_permute(*args(ws=None)) == m.MOE_ERR_WORKSPACE
    assert L.moe_dispatch_permute(*args(x=odd)) == m.MOE_ERR_INVALID_ARG
    # grouped FFN: natural layout is unsupported (pack first); bad shapes; fp8 without scales
    w = m.FfnWeights(m.MOE_DTYPE_BF16, m.MOE_LAYOUT_NATURAL, 8, 256, 384, 0x10000, 0x10000, 0x10000, None, None, None)
    wsf = m.lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(w), 200)
    call = lambda w, wsb=wsf: L.moe_grouped_ffn(fake, None, fake, 0, 200, ctypes.byref(w), fake, big, wsb, None)
    assert call(w) == m.MOE_ERR_UNSUPPORTED
    w.layout = m.MOE_LAYOUT_PACKED
    assert call(w, wsf - 1) == m.MOE_ERR_WORKSPACE
    w.F = 100
    assert call(w) == m.MOE_ERR_INVALID_ARG
    w.F = 384
    w.dtype = m.MOE_DTYPE_FP8_E4M3
    assert call(w) == m.MOE_ERR_INVALID_ARG
    assert "s_gate" in L.moe_last_error().decode()
    w.layout = 5
    assert call(w) == m.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_ffn(fake, None, fake, 0, 200, None, fake, big, wsf, None) == m.MOE_ERR_INVALID_ARG
    # combine: fp8 output is unsupported, empty window, k > 32
    cargs = lambda **kw: [fake, fake, fake, fake, kw.get("T", 10), kw.get("k", 2), 256, kw.get("e_lo", 0),
                          kw.get("El", 8), fake, kw.get("dt", m.MOE_DTYPE_BF16), None]
    assert L.moe_combine(*cargs(dt=m.MOE_DTYPE_FP8_E4M3)) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(*cargs(El=0)) == m.MOE_ERR_INVALID_ARG
    assert L.moe_combine(*cargs(k=33)) == m.MOE_ERR_INVALID_ARG
    assert L.moe_combine(*cargs(T=0)) == m.MOE_OK
    # pack: destination too small
    w = m.FfnWeights(m.MOE_DTYPE_BF16, m.MOE_LAYOUT_NATURAL, 8, 256, 384, 0x10000, 0x10000, 0x10000, None, None, None)
    need = L.moe_pack_ffn_weights_bytes(ctypes.byref(w))
    assert need == 3 * 8 * 256 * 384 * 2
    out = m.FfnWeights()
    assert L.moe_pack_ffn_weights(ctypes.byref(w), big, need - 1, ctypes.byref(out), None) == m.MOE_ERR_INVALID_ARG


def test_fused_entry_points_validate_before_launch():
    import grouped_expert_ffn_router_amd as m

    L = m.lib
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first
    big = ctypes.c_void_p(0x100000)
    w = m.FfnWeights(m.MOE_DTYPE_BF16, m.MOE_LAYOUT_PACKED, 8, 256, 384, 0x10000, 0x10000, 0x10000, None, None, None)
    wsf = L.moe_grouped_ffn_workspace_bytes(ctypes.byref(w), 200)
    # scatter: R_max beyond T*k; gate/up gather: the activations' byte span past 32-bit offsets, no token table
    assert L.moe_grouped_ffn_down_scatter(fake, 0, 200, ctypes.byref(w), fake, fake, fake, 10, 2, fake, big, wsf,
                                          None) == m.MOE_ERR_INVALID_ARG
    assert "R_max" in L.moe_last_error().decode()
    assert L.moe_grouped_ffn_gate_up_gather(fake, None, fake, 1 << 23, fake, 0, 200, ctypes.byref(w), big, wsf,
                                            None) == m.MOE_ERR_INVALID_ARG
    assert "2^32" in L.moe_last_error().decode()
    assert L.moe_grouped_ffn_gate_up_gather(fake, None, None, 200, fake, 0, 200, ctypes.byref(w), big, wsf,
                                            None) == m.MOE_ERR_INVALID_ARG
    assert "token_of_row" in L.moe_last_error().decode()
    # fp8 without x_scales
    w8 = m.FfnWeights(m.MOE_DTYPE_FP8_E4M3, m.MOE_LAYOUT_PACKED, 8, 256, 384, 0x10000, 0x10000, 0x10000, 0x10000,
                      0x10000, 0x10000)
    ws8 = L.moe_grouped_ffn_workspace_bytes(ctypes.byref(w8), 200)
    assert L.moe_grouped_ffn_gate_up_gather(fake, None, fake, 200, fake, 0, 200, ctypes.byref(w8), big, ws8,
                                            None) == m.MOE_ERR_INVALID_ARG
    assert "x_scales" in L.moe_last_error().decode()
    # down scatter: k out of range, missing slots, natural layout
    assert L.moe_grouped_ffn_down_scatter(fake, 0, 200, ctypes.byref(w), fake, fake, fake, 100, 33, fake, big, wsf,
                                          None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_ffn_down_scatter(fake, 0, 200, ctypes.byref(w), fake, fake, fake, 100, 2, None, big, wsf,
                                          None) == m.MOE_ERR_INVALID_ARG
    assert "y_slot" in L.moe_last_error().decode()
    w.layout = m.MOE_LAYOUT_NATURAL
    assert L.moe_grouped_ffn_fused(fake, None, fake, fake, fake, 100, 2, fake, 0, 200, ctypes.byref(w), fake, big,
                                   wsf, None) == m.MOE_ERR_UNSUPPORTED
    w.layout = m.MOE_LAYOUT_PACKED
    assert L.moe_grouped_ffn_fused(fake, None, fake, fake, fake, 100, 2, fake, 0, 200, ctypes.byref(w), fake, big,
                                   wsf - 1, None) == m.MOE_ERR_WORKSPACE
    # R_max = 0 is a successful no-op
    assert L.moe_grouped_ffn_fused(None, None, None, None, None, 0, 2, fake, 0, 0, ctypes.byref(w), None, big,
                                   wsf, None) == m.MOE_OK
    # slot combine: fp8 output, k > 32, empty window; T = 0 is a no-op
    assert L.moe_combine_slots(fake, None, fake, 10, 2, 256, 0, 8, fake, m.MOE_DTYPE_FP8_E4M3,
                               None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_combine_slots(fake, None, fake, 10, 33, 256, 0, 8, fake, m.MOE_DTYPE_BF16,
                               None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_combine_slots(fake, None, fake, 10, 2, 256, 0, 0, fake, m.MOE_DTYPE_BF16,
                               None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_combine_slots(fake, ctypes.c_void_p(0x10002), fake, 10, 2, 256, 0, 8, fake, m.MOE_DTYPE_BF16,
                               None) == m.MOE_ERR_INVALID_ARG  # misaligned row_of_pair
    assert L.moe_combine_slots(None, None, None, 0, 2, 256, 0, 8, None, m.MOE_DTYPE_BF16, None) == m.MOE_OK
    # fixed capacity: capacity < 1, then the shared dispatch checks (k > E)
    wsd = m.moe_dispatch_workspace_bytes(100, 2, 8)
    assert L.moe_dispatch_permute_capacity(fake, None, m.MOE_DTYPE_BF16, 100, 256, fake, 2, 8, 0, fake, fake, fake,
                                           fake, fake, None, big, wsd, None) == m.MOE_ERR_INVALID_ARG
    assert "capacity" in L.moe_last_error().decode()
    assert L.moe_dispatch_permute_capacity(fake, None, m.MOE_DTYPE_BF16, 100, 256, fake, 9, 8, 4, fake, fake, fake,
                                           fake, fake, None, big, wsd, None) == m.MOE_ERR_INVALID_ARG
    # dispatch without x_perm still needs the permutation outputs
    ws = m.moe_dispatch_workspace_bytes(100, 2, 8)
    assert L.moe_dispatch_permute(None, None, m.MOE_DTYPE_BF16, 100, 256, fake, 2, 8, fake, fake, None, fake, None,
                                  None, big, ws, None) == m.MOE_ERR_INVALID_ARG
    assert "row_of_pair" in L.moe_last_error().decode()
    # the workspace calls reject a NULL workspace; the no-allocation variant validates every argument before its
    # fixed scratch is looked up, and refuses requests beyond that scratch (1 MiB) without touching a device
    assert L.moe_dispatch_permute(fake, None, m.MOE_DTYPE_BF16, 100, 256, fake, 2, 8, fake, fake, fake, fake, fake,
                                  None, None, 0, None) == m.MOE_ERR_WORKSPACE
    assert L.moe_dispatch_permute_noalloc(fake, None, m.MOE_DTYPE_BF16, 100, 256, fake, 9, 8, fake, fake, fake,
                                          fake, fake, None, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch_permute_noalloc(fake, None, m.MOE_DTYPE_BF16, 100, 200, fake, 2, 8, fake, fake, fake,
                                          fake, fake, None, None) == m.MOE_ERR_INVALID_ARG  # H % 128
    assert L.moe_dispatch_permute_noalloc(fake, None, m.MOE_DTYPE_BF16, 1 << 18, 256, fake, 8, 256, fake, fake, fake,
                                          fake, fake, None, None) == m.MOE_ERR_WORKSPACE
    assert "more than the fixed 1048576" in L.moe_last_error().decode()
    assert m.moe_dispatch_workspace_bytes(1 << 18, 8, 256) > 1 << 20 >= m.moe_dispatch_workspace_bytes(65536, 8, 256)


def test_workspace_sizes():
    import grouped_expert_ffn_router_amd as m

    # dispatch: one int32 per (expert, 128-token count tile), rounded up, plus the expert offsets
    assert m.moe_dispatch_workspace_bytes(8192, 8, 32) >= 32 * 64 * 4 + 33 * 4
    assert m.moe_dispatch_workspace_bytes(8193, 8, 32) >= 32 * 65 * 4 + 33 * 4
    # FFN: h in the layer dtype (+ fp8 scales) (+ fp32 partial sums when the down product is split over K)
    fp8 = m.FfnWeights(m.MOE_DTYPE_FP8_E4M3, m.MOE_LAYOUT_PACKED, 32, 7168, 2048, 1, 1, 1, 1, 1, 1)
    assert m.lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(fp8), 65536) >= 65536 * 2048 + 65536 * 16 * 4
    bf = m.FfnWeights(m.MOE_DTYPE_BF16, m.MOE_LAYOUT_PACKED, 8, 4096, 14336, 1, 1, 1, None, None, None)
    need = m.lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(bf), 4096)
    # the Mixtral shape's down product (~272 output tiles for 256 CUs) is not split: h only, no partial sums
    assert 4096 * 14336 * 2 <= need < 4096 * 14336 * 2 + 4096 * 4096 * 4
    # few output tiles (14, at most half the CUs) with an even stage count: split in two, one fp32 partial
    few = m.FfnWeights(m.MOE_DTYPE_BF16, m.MOE_LAYOUT_PACKED, 8, 256, 1024, 1, 1, 1, None, None, None)
    assert m.lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(few), 1200) >= 1200 * 1024 * 2 + 1200 * 256 * 4
    assert m.lib.moe_grouped_ffn_workspace_bytes(None, 10) == 0


def test_python_binding_errors_map_to_exceptions():
    import torch

    import grouped_expert_ffn_router_amd as m

    with pytest.raises(ValueError, match="k = 9"):
        m.moe_route_topk(torch.empty((4, 8)), 9, topk_idx=torch.empty((4, 9), dtype=torch.int32),
                         topk_w=torch.empty((4, 9)), stream=0)


def test_router_entry_point_validates_before_launch():
    import grouped_expert_ffn_router_amd as m

    L = m.lib
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first
    odd = ctypes.c_void_p(0x10002)
    call = lambda **kw: L.moe_router_topk(kw.get("x", fake), kw.get("xs", None), kw.get("dt", m.MOE_DTYPE_BF16),
                                          kw.get("T", 100), kw.get("H", 256), kw.get("W", fake), kw.get("E", 8),
                                          kw.get("k", 2), kw.get("lg", fake), kw.get("idx", fake), kw.get("w", fake),
                                          None)
    # above 64 experts the selection reads the logits back, so the buffer is required; E past 1024 is invalid
    assert call(E=65, lg=None) == m.MOE_ERR_INVALID_ARG
    assert "logits" in L.moe_last_error().decode()
    assert call(E=2000) == m.MOE_ERR_INVALID_ARG
    assert call(k=9) == m.MOE_ERR_INVALID_ARG
    assert call(k=0) == m.MOE_ERR_INVALID_ARG
    assert call(T=-1) == m.MOE_ERR_INVALID_ARG
    assert call(H=100) == m.MOE_ERR_INVALID_ARG
    assert call(H=0) == m.MOE_ERR_INVALID_ARG
    # fp8: H a multiple of 128 and scales present
    assert call(dt=m.MOE_DTYPE_FP8_E4M3, H=136, xs=fake) == m.MOE_ERR_INVALID_ARG
    assert call(dt=m.MOE_DTYPE_FP8_E4M3, H=256) == m.MOE_ERR_INVALID_ARG
    assert "x_scales" in L.moe_last_error().decode()
    assert call(dt=7) == m.MOE_ERR_INVALID_ARG
    assert call(x=odd) == m.MOE_ERR_INVALID_ARG
    assert call(x=None) == m.MOE_ERR_INVALID_ARG
    assert call(W=None) == m.MOE_ERR_INVALID_ARG
    assert call(lg=odd) == m.MOE_ERR_INVALID_ARG
    assert call(idx=None) == m.MOE_ERR_INVALID_ARG
    assert call(w=odd) == m.MOE_ERR_INVALID_ARG
    # nothing to do: OK without touching a pointer
    assert call(T=0, x=None, W=None, lg=None, idx=None, w=None) == m.MOE_OK


def test_training_entry_points_validate_before_launch():
    import grouped_expert_ffn_router_amd as m

    L = m.lib
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first
    big = ctypes.c_void_p(0x100000)
    nat = m.FfnWeights(m.MOE_DTYPE_BF16, m.MOE_LAYOUT_NATURAL, 8, 256, 384, 0x10000, 0x10000, 0x10000, None, None, None)
    pk = m.FfnWeights(m.MOE_DTYPE_BF16, m.MOE_LAYOUT_PACKED, 8, 256, 384, 0x10000, 0x10000, 0x10000, None, None, None)
    f8 = m.FfnWeights(m.MOE_DTYPE_FP8_E4M3, m.MOE_LAYOUT_NATURAL, 8, 256, 384, 0x10000, 0x10000, 0x10000, 0x10000,
                      0x10000, 0x10000)
    wsn = L.moe_grouped_ffn_backward_workspace_bytes(ctypes.byref(nat), 200)
    assert wsn > 200 * 256 * 2
    assert L.moe_grouped_ffn_backward_workspace_bytes(ctypes.byref(f8), 200) == 0

    def bwd(w=nat, T=100, k=2, E=8, e_lo=0, R=200, ws=big, wsb=wsn, dl=fake, dout=fake):
        return L.moe_grouped_ffn_backward(dout, T, k, E, fake, fake, fake, fake, fake, e_lo, R, fake, fake, fake, fake,
                                          ctypes.byref(w), fake, fake, fake, fake, fake, dl, ws, wsb, None)

    assert bwd(w=pk) == m.MOE_ERR_UNSUPPORTED
    assert "NATURAL" in L.moe_last_error().decode()
    assert bwd(w=f8) == m.MOE_ERR_UNSUPPORTED
    assert bwd(k=33) == m.MOE_ERR_INVALID_ARG
    assert bwd(E=7) == m.MOE_ERR_INVALID_ARG  # window [0, 8) outside [0, 7)
    assert bwd(e_lo=1) == m.MOE_ERR_INVALID_ARG
    assert bwd(R=201) == m.MOE_ERR_INVALID_ARG  # more rows than pairs
    assert bwd(T=-1) == m.MOE_ERR_INVALID_ARG
    assert bwd(dl=ctypes.c_void_p(0x10002)) == m.MOE_ERR_INVALID_ARG
    assert bwd(dout=None) == m.MOE_ERR_INVALID_ARG
    assert bwd(wsb=wsn - 1) == m.MOE_ERR_WORKSPACE
    assert bwd(ws=ctypes.c_void_p(0x100010)) == m.MOE_ERR_WORKSPACE
    # the training forward: packed weights, no fp8, its two extra outputs present
    wsf = L.moe_grouped_ffn_workspace_bytes(ctypes.byref(pk), 200)
    tr = lambda w=pk, h=fake, gu=fake: L.moe_grouped_ffn_train(fake, fake, 0, 200, ctypes.byref(w), h, gu, fake, big,
                                                               wsf, None)
    assert tr(w=nat) == m.MOE_ERR_UNSUPPORTED
    assert tr(h=None) == m.MOE_ERR_INVALID_ARG
    assert tr(gu=ctypes.c_void_p(0x10008)) == m.MOE_ERR_INVALID_ARG


def test_header_compiles_as_c_and_cpp_and_links(tmp_path):
    """include/moe_ep.h is plain C: it compiles as C99 and C++11 with -pedantic, and a C program that includes it
    links against the library (every declaration has a definition with C linkage)."""
    import shutil

    import grouped_expert_ffn_router_amd as m

    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "use_header.c"
    calls = "\n".join(f"  (void)&{n};" for n in declared_functions())
    src.write_text('#include "moe_ep.h"\nint main(void) {\n' + calls + "\n  return moe_abi_version() == "
                   "MOE_EP_ABI_VERSION ? 0 : 1;\n}\n")
    inc = os.path.join(ROOT, "include")
    for cc, std, lang in (("gcc", "-std=c99", "c"), ("g++", "-std=c++11", "c++")):
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-I", inc, "-x",
                            lang, str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
    exe = tmp_path / "use_header"
    libdir = os.path.dirname(m.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-L", libdir, "-l:libmoe_ep.so",
                        f"-Wl,-rpath,{libdir}", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
