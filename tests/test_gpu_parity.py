"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded synthetic inputs.

Bars: routing indices, counts, offsets, the permutation and x_perm bit-exact; routing weights within 2 fp32
ulps of the oracle's fp64 weights; layer output max|gpu - oracle| / RMS(oracle) <= 1e-4 (fp32), 2e-2 (bf16),
6e-2 (fp8).  Full outputs at sizes that span several tiles with ragged tails; sampled tokens (covering every
non-empty expert) at the five workload sizes, in the launch configuration the benchmark times.
"""
import zlib

import numpy as np
import pytest
import torch

import checks
import moe_inputs
import oracle

pytestmark = pytest.mark.gpu

BAR = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


def lib():
    import grouped_expert_ffn_router_amd as m

    return m


def _dev(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


class Dev:
    """Device copies of one workload's inputs."""

    def __init__(self, inp):
        wl = inp.wl
        self.inp = inp
        self.x = _dev(inp.x, wl.dtype)
        self.x_scales = None if inp.x_scales is None else torch.from_numpy(inp.x_scales).cuda()
        self.logits = torch.from_numpy(inp.logits).cuda()
        self.w = [_dev(a, wl.dtype) for a in (inp.w_gate, inp.w_up, inp.w_down)]
        self.s = [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
                  for a in (inp.s_gate, inp.s_up, inp.s_down)]


def run_layer(d: Dev, packed=None, out_f32=False, fused=False):
    """The four C-ABI calls (fused: dispatch without x_perm, the fused grouped FFN and the slot combine);
    returns every intermediate as host arrays."""
    m = lib()
    wl = d.inp.wl
    idx, w = m.moe_route_topk(d.logits, wl.k)
    disp = m.moe_dispatch_permute(d.x, idx, wl.E, x_scales=d.x_scales, gather=not fused)
    if packed is None:
        packed = m.moe_pack_ffn_weights(*d.w, *d.s)
    out_dtype = torch.float32 if (wl.dtype == "f32" or out_f32) else torch.bfloat16
    if fused:
        assert disp.x_perm is None
        y = m.moe_grouped_ffn_fused(d.x, disp.token_of_row, disp.row_of_pair, w, disp.offsets, packed,
                                    x_scales=d.x_scales, e_lo=wl.e_lo)
        out = m.moe_combine_slots(y, idx, e_lo=wl.e_lo, E_local=wl.n_local, out_dtype=out_dtype)
    else:
        y = m.moe_grouped_ffn(disp.x_perm, disp.offsets, packed, x_perm_scales=disp.x_perm_scales, e_lo=wl.e_lo)
        out = m.moe_combine(y, disp.row_of_pair, idx, w, e_lo=wl.e_lo, E_local=wl.n_local, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return dict(topk_idx=idx.cpu().numpy(), topk_w=w.cpu().numpy(), counts=disp.counts.cpu().numpy(),
                offsets=disp.offsets.cpu().numpy(), row_of_pair=disp.row_of_pair.cpu().numpy(),
                token_of_row=disp.token_of_row.cpu().numpy(), x_perm=disp.x_perm,
                x_perm_scales=disp.x_perm_scales, y_perm=y, out=out.float().cpu().numpy().astype(np.float64),
                packed=packed)


def check_route(g, ref_idx, ref_w):
    np.testing.assert_array_equal(g["topk_idx"], ref_idx)
    ref32 = ref_w.astype(np.float32)
    ulp = np.spacing(np.abs(ref32))
    assert np.all(np.abs(g["topk_w"].astype(np.float64) - ref32.astype(np.float64)) <= 2 * ulp)


def check_dispatch(g, d: Dev, ref):
    counts, offsets, rop, tor = ref
    np.testing.assert_array_equal(g["counts"], counts)
    np.testing.assert_array_equal(g["offsets"], offsets)
    np.testing.assert_array_equal(g["row_of_pair"], rop)
    np.testing.assert_array_equal(g["token_of_row"], tor)
    if g["x_perm"] is None:  # fused form: no permuted copy
        return
    idx_t = torch.from_numpy(tor.astype(np.int64)).cuda()
    assert torch.equal(g["x_perm"].view(torch.uint8), d.x[idx_t].view(torch.uint8))
    if d.x_scales is not None:
        assert torch.equal(g["x_perm_scales"], d.x_scales[idx_t])


def layer_err(gpu_rows, ref_rows):
    rms = np.sqrt(np.mean(ref_rows**2))
    return np.max(np.abs(gpu_rows - ref_rows)) / rms


def sample_tokens(idx, wl, n_extra, seed=0):
    """One token for every non-empty local expert, plus n_extra seeded random tokens."""
    rng = np.random.default_rng(seed)
    picks = set()
    for e in range(wl.e_lo, wl.e_lo + wl.n_local):
        t = np.nonzero((idx == e).any(axis=1))[0]
        if len(t):
            picks.add(int(rng.choice(t)))
    picks |= set(int(t) for t in rng.choice(wl.T, size=min(n_extra, wl.T), replace=False))
    return np.array(sorted(picks), dtype=np.int64)


def out_floor(ref, dtype):
    """max |round(ref) - ref| / RMS(ref): the part of the error owed to the output format itself."""
    r = ref.astype(np.float32)
    if dtype != "f32":
        r = torch.from_numpy(r).to(torch.bfloat16).float().numpy()
    return layer_err(r.astype(np.float64), ref)


def full_check(wl, tokens=None, out_f32=False, fused=False):
    inp = moe_inputs.make_inputs(wl)
    d = Dev(inp)
    g = run_layer(d, out_f32=out_f32, fused=fused)
    idx, w = oracle.route_topk(inp.logits, wl.k)
    check_route(g, idx, w)
    check_dispatch(g, d, oracle.dispatch(idx, wl.E))
    if tokens is None:
        tokens = np.arange(wl.T)
    ref = oracle.moe_tokens(inp, idx, w, tokens=tokens)
    err = layer_err(g["out"][tokens], ref)
    floor = out_floor(ref, "f32" if out_f32 else wl.dtype)
    print(f"{wl.name}{' fused' if fused else ''}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} F={wl.F} {wl.dtype}: err {err:.3e} "
          f"(output-format floor {floor:.3e}) bar {BAR[wl.dtype]}")
    if wl.dtype == "fp8" and wl.F < FP8_PLAIN_BAR_F:
        check_fp8_with_midpoint_slack(inp, idx, w, tokens, g["out"][tokens], ref)
    else:
        assert err <= BAR[wl.dtype], (err, floor)
    return g, inp, d, ref, tokens


# fp8 layers: an h element whose exact value lies within the GPU's error bound of an e4m3 rounding midpoint may
# be stored as either neighbour (both are correct roundings); one such element moves the outputs of its token by
# one e4m3 step of h times its W_down row, about 0.08 RMS sqrt(384 / F) at most.  From F = 2048 up the max|err| /
# RMS bar holds with that included; below, the outputs are checked element by element against the bar plus the
# steps of the elements the oracle finds within their bound of a midpoint (a tolerance from the oracle alone).
FP8_PLAIN_BAR_F = 2048


def _wd_abs(inp, e):
    v = moe_inputs.e4m3_codes_to_f32(inp.w_down[e]).astype(np.float64)
    return np.abs(v * np.repeat(np.repeat(inp.s_down[e].astype(np.float64), 128, axis=0), 128, axis=1))


def check_fp8_with_midpoint_slack(inp, idx, w, tokens, got, ref):
    wl = inp.wl
    slack = np.zeros_like(ref)
    pairs = [(i, t * wl.k + j, int(idx[t, j]) - wl.e_lo) for i, t in enumerate(tokens) for j in range(wl.k)
             if 0 <= int(idx[t, j]) - wl.e_lo < wl.n_local]
    hr = oracle.pair_h(inp, idx, np.array([p for _, p, _ in pairs], dtype=np.int64))
    mask, delta = checks.midpoint_window("fp8", wl.H, hr)
    wd = {}
    for n, (i, p, e) in enumerate(pairs):
        if mask[n].any():
            if e not in wd:
                wd[e] = _wd_abs(inp, e)
            slack[i] += abs(w[p // wl.k, p % wl.k]) * (delta[n] @ wd[e])
    rms = np.sqrt(np.mean(ref**2))
    ratio = np.abs(got - ref) / (BAR["fp8"] * rms + slack)
    print(f"  fp8 F={wl.F}: {int(mask.sum())} of {mask.size} h elements within their bound of a midpoint; "
          f"max |err| / (bar RMS + their steps) = {ratio.max():.3f}")
    assert ratio.max() <= 1.0


# ------------------------------------------------------------------------------------------------------------
# full-output parity at small sizes (several tiles, ragged tails) through every tile configuration
# ------------------------------------------------------------------------------------------------------------
SMALL = [
    # name, T, H, E, k, F, dtype, logits   -> mean rows per expert picks the row-block size 32 / 64 / 128 / 256
    ("s_f32_bm64", 256, 128, 8, 2, 256, "f32", "router"),
    ("s_f32_bm32", 40, 256, 8, 3, 384, "f32", "gauss"),
    ("s_bf16_bm32", 100, 384, 32, 8, 256, "bf16", "gauss"),
    ("s_bf16_bm64", 300, 256, 8, 2, 384, "bf16", "gauss"),
    ("s_bf16_bm128", 700, 256, 8, 2, 256, "bf16", "router"),
    ("s_bf16_bm256", 1300, 256, 8, 2, 384, "bf16", "gauss"),
    ("s_bf16_h384", 1300, 384, 8, 2, 256, "bf16", "gauss"),
    ("s_bf16_zipf", 900, 256, 64, 4, 256, "bf16", "zipf"),
    ("s_bf16_ksplit", 600, 256, 8, 2, 1024, "bf16", "gauss"),  # few output tiles: the down product is split over K
    ("s_bf16_wide_few", 40, 2048, 16, 4, 256, "bf16", "gauss"),  # few tokens, wide rows: the combine splits rows
    ("s_bf16_k12", 120, 256, 24, 12, 256, "bf16", "gauss"),  # k > 8: the combine's one-slot-at-a-time form
    # a hot expert with more rows than the down product has weight rows (its weight tiles go fastest) while the
    # down product is split over K (few output tiles)
    ("s_bf16_hot_ksplit", 1200, 256, 2, 1, 2048, "bf16", "zipf"),
    ("s_fp8_hot_ksplit", 1200, 256, 2, 1, 2048, "fp8", "zipf"),
    # fp8 at F = 256 and 384 (checked with the midpoint slack below F = 2048) and at the fp8 workload's F = 2048
    ("s_fp8_bm32_f256", 60, 256, 32, 8, 256, "fp8", "gauss"),
    ("s_fp8_bm64_f256", 200, 384, 8, 3, 256, "fp8", "gauss"),
    ("s_fp8_bm128_f384", 600, 256, 8, 2, 384, "fp8", "gauss"),
    ("s_fp8_bm256_f384", 1100, 512, 8, 2, 384, "fp8", "gauss"),
    ("s_fp8_bm32", 60, 256, 32, 8, 2048, "fp8", "gauss"),
    ("s_fp8_bm64", 200, 384, 8, 3, 2048, "fp8", "gauss"),
    ("s_fp8_bm128", 600, 512, 8, 2, 2048, "fp8", "gauss"),
    ("s_fp8_bm256", 1100, 512, 8, 2, 2048, "fp8", "gauss"),  # 256-row tiles; few output tiles: down split over K
    ("s_fp8_bm256_h384", 1100, 384, 8, 2, 2048, "fp8", "gauss"),  # 128-column down tiles
    # more than 64 local experts: the tile lookup walks the experts 64 at a time
    ("s_bf16_e96", 500, 256, 96, 4, 256, "bf16", "gauss"),
    ("s_fp8_e130", 600, 256, 130, 4, 256, "fp8", "zipf"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_full_output(case):
    name, T, H, E, k, F, dt, lg = case
    full_check(moe_inputs.Workload(name, T=T, H=H, E=E, k=k, F=F, dtype=dt, logits=lg, seed=zlib.crc32(name.encode()) % 1000))


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_full_output_fused(case):
    """The fused form (gather inside the gate/up product, weighted pair-major slots, slot combine)."""
    name, T, H, E, k, F, dt, lg = case
    full_check(moe_inputs.Workload(name, T=T, H=H, E=E, k=k, F=F, dtype=dt, logits=lg,
                                   seed=zlib.crc32(name.encode()) % 1000), fused=True)


# ------------------------------------------------------------------------------------------------------------
# the stored SwiGLU intermediate h against the oracle's, element by element (tests/checks.py: bit-exact except
# within the GPU arithmetic's error bound of a rounding midpoint, where it must be one of the two neighbours)
# ------------------------------------------------------------------------------------------------------------
HCASES = [
    ("h_fp8_f256", 600, 512, 8, 2, 256, "fp8", "gauss"),
    ("h_fp8_f384", 1100, 384, 8, 2, 384, "fp8", "gauss"),
    ("h_fp8_f2048", 200, 384, 8, 3, 2048, "fp8", "gauss"),
    ("h_fp8_bm32", 60, 256, 32, 8, 256, "fp8", "gauss"),
    ("h_fp8_zipf", 900, 256, 64, 4, 384, "fp8", "zipf"),
    ("h_bf16_f384", 1300, 256, 8, 2, 384, "bf16", "gauss"),
    ("h_bf16_bm32", 100, 384, 32, 8, 256, "bf16", "gauss"),
    ("h_f32", 256, 128, 8, 2, 256, "f32", "router"),
]


def gate_up_h(d: Dev, gather=False):
    """Route, dispatch and the gate/up half of the grouped FFN; returns (oracle-checked dispatch tables, the
    stored h [R, F] as element bits, the fp8 scales [R, F/128] or None) read from the FFN workspace, whose layout
    include/moe_ep.h documents (h at byte 0, fp8 scales at the next 256-byte boundary)."""
    m = lib()
    wl = d.inp.wl
    idx, w = m.moe_route_topk(d.logits, wl.k)
    disp = m.moe_dispatch_permute(d.x, idx, wl.E, x_scales=d.x_scales, gather=not gather)
    packed = m.moe_pack_ffn_weights(*d.w, *d.s)
    R = wl.T * wl.k
    ws = torch.zeros(m.moe_grouped_ffn_workspace_bytes(packed, R), dtype=torch.uint8, device="cuda")
    if gather:
        m.moe_grouped_ffn_gate_up_gather(d.x, disp.token_of_row, disp.offsets, packed, ws, d.x_scales, wl.e_lo)
    else:
        m.moe_grouped_ffn_gate_up(disp.x_perm, disp.offsets, packed, ws, disp.x_perm_scales, wl.e_lo)
    torch.cuda.synchronize()
    b = moe_inputs.ELEM_BYTES[wl.dtype]
    hb = ws[: R * wl.F * b].cpu().numpy()
    bits = {1: hb, 2: hb.view(np.uint16), 4: hb.view(np.uint32)}[b].reshape(R, wl.F).astype(np.uint32)
    sc = None
    if wl.dtype == "fp8":
        o = (R * wl.F + 255) // 256 * 256
        sc = ws[o: o + R * (wl.F // 128) * 4].cpu().numpy().view(np.float32).reshape(R, wl.F // 128)
    return idx.cpu().numpy(), disp.row_of_pair.cpu().numpy(), bits, sc


@pytest.mark.parametrize("gather", [False, True], ids=["permuted", "gather"])
@pytest.mark.parametrize("case", HCASES, ids=[c[0] for c in HCASES])
def test_stored_h_against_the_oracle(case, gather):
    name, T, H, E, k, F, dt, lg = case
    wl = moe_inputs.Workload(name, T=T, H=H, E=E, k=k, F=F, dtype=dt, logits=lg, seed=zlib.crc32(name.encode()) % 991)
    inp = moe_inputs.make_inputs(wl)
    idx, rop, bits, sc = gate_up_h(Dev(inp), gather=gather)
    ridx, _ = oracle.route_topk(inp.logits, k)
    np.testing.assert_array_equal(idx, ridx)
    np.testing.assert_array_equal(rop, oracle.dispatch(ridx, E)[2])
    pairs = np.arange(T * k, dtype=np.int64)
    ref = oracle.pair_h(inp, ridx, pairs)
    st = checks.check_h(dt, H, ref, bits[rop], None if sc is None else sc[rop])
    print(f"{name}: {st['elements']} h elements, {st['window']} within their bound of a midpoint, "
          f"{st['differing']} differ (largest distance / bound {st['worst']:.3g}, kappa needed "
          f"{st['kappa_needed']:.3g})")


def test_stored_h_at_the_fp8_workload_tile_edges():
    """The DeepSeek-V3-shaped fp8 layer at full size: h of the first and last row of every 256-row block of every
    expert (the gate/up product's tile edges) against the oracle."""
    wl = moe_inputs.get("dsv3_fp8")
    inp = moe_inputs.make_inputs(wl)
    idx, rop, bits, sc = gate_up_h(Dev(inp))
    ridx, _ = oracle.route_topk(inp.logits, wl.k)
    np.testing.assert_array_equal(idx, ridx)
    counts, offsets, rop_o, tor = oracle.dispatch(ridx, wl.E)
    np.testing.assert_array_equal(rop, rop_o)
    pair_of_row = np.empty(wl.T * wl.k, np.int64)
    pair_of_row[rop_o] = np.arange(wl.T * wl.k)
    bm = tile_rows(wl.T * wl.k, wl.n_local, wl.dtype)
    rows = sorted({int(offsets[e]) + r for e in range(wl.E) for m0 in range(0, int(counts[e]), bm)
                   for r in (m0, min(m0 + bm, int(counts[e])) - 1)})
    ref = oracle.pair_h(inp, ridx, pair_of_row[rows])
    st = checks.check_h("fp8", wl.H, ref, bits[rows], sc[rows])
    print(f"dsv3_fp8 h at {len(rows)} tile-edge rows: {st['window']} of {st['elements']} elements within their "
          f"bound of a midpoint, {st['differing']} differ (largest distance / bound {st['worst']:.3g}, kappa needed "
          f"{st['kappa_needed']:.3g})")


# ------------------------------------------------------------------------------------------------------------
# the five workloads at full size: every routing / dispatch output, and the layer output on sampled tokens
# ------------------------------------------------------------------------------------------------------------
def tile_rows(R_max, E_local, dtype):
    """The row-block size the grouped FFN takes from the mean rows per expert (bf16: 320 from 256 rows on, fp8:
    256; then 128, 64, 32); used only to choose which rows to sample."""
    avg = R_max // max(E_local, 1)
    if avg >= 256 and dtype in ("bf16", "fp8"):
        return 320 if dtype == "bf16" else 256
    return 128 if avg >= 96 else 64 if avg >= 48 else 32


def edge_tokens(idx, wl, n_extra, seed=0):
    """The tokens of the first and last row of every row block of every local expert (the tile edges of the
    grouped products, from the oracle's permutation), plus n_extra seeded random tokens."""
    counts, offsets, rop, tor = oracle.dispatch(idx, wl.E)
    bm = tile_rows(wl.T * wl.k, wl.n_local, wl.dtype)
    picks = set()
    for e in range(wl.e_lo, wl.e_lo + wl.n_local):
        b, n = int(offsets[e]), int(counts[e])
        for m0 in range(0, n, bm):
            picks.add(int(tor[b + m0]))
            picks.add(int(tor[b + min(m0 + bm, n) - 1]))
    rng = np.random.default_rng(seed)
    picks |= set(int(t) for t in rng.choice(wl.T, size=min(n_extra, wl.T), replace=False))
    return np.array(sorted(picks), dtype=np.int64)


@pytest.mark.parametrize("name,n_extra", [("tiny_fp32", None), ("mixtral_bf16", 24), ("decode_bf16", None),
                                          ("dsv3_fp8", 16), ("skewed_bf16", 16)])
@pytest.mark.parametrize("fused", [False, True], ids=["permuted", "fused"])
def test_workload_parity(name, n_extra, fused):
    """The five workloads at full size in the benchmark's launch configuration: every routing and dispatch output,
    and the layer output of every token (tiny, decode) or of the tokens at every row block's first and last row
    of every expert (the grouped products' tile edges) plus a seeded sample."""
    wl = moe_inputs.get(name)
    if n_extra is None:
        full_check(wl, fused=fused)
        return
    inp = moe_inputs.make_inputs(wl, with_weights=False)
    idx, _ = oracle.route_topk(inp.logits, wl.k)
    toks = edge_tokens(idx, wl, n_extra)
    print(f"{name}: {len(toks)} tokens at tile edges and sampled", flush=True)
    full_check(wl, tokens=toks, fused=fused)


# ------------------------------------------------------------------------------------------------------------
# edge cases
# ------------------------------------------------------------------------------------------------------------
def test_route_ties_neg_inf_and_wide_expert_counts():
    m = lib()
    rng = np.random.default_rng(1)
    for E, k in [(8, 2), (1, 1), (3, 3), (64, 32), (100, 7), (256, 8), (1000, 32), (1024, 1)]:
        L = rng.standard_normal((203, E)).astype(np.float32)
        L[0, :] = 0.25  # all equal
        L[1, : min(E, 5)] = 3.0  # ties inside and across the k boundary
        if E > 3:
            L[2, 1::2] = -np.inf
            L[3, -1] = L[3].max()  # a tie between the first and last expert for first place
        L[4] = np.round(L[4] * 2) / 2  # many ties
        idx, w = m.moe_route_topk(torch.from_numpy(L).cuda(), k)
        ridx, rw = oracle.route_topk(L, k)
        check_route(dict(topk_idx=idx.cpu().numpy(), topk_w=w.cpu().numpy()), ridx, rw)


def test_zero_tokens():
    m = lib()
    dev = torch.device("cuda")
    idx, w = m.moe_route_topk(torch.empty((0, 8), device=dev), 2)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    disp = m.moe_dispatch_permute(x, idx, 8)
    torch.cuda.synchronize()
    assert disp.counts.cpu().tolist() == [0] * 8 and disp.offsets.cpu().tolist() == [0] * 9
    wg = torch.zeros((8, 256, 128), dtype=torch.bfloat16, device=dev)
    wd = torch.zeros((8, 128, 256), dtype=torch.bfloat16, device=dev)
    packed = m.moe_pack_ffn_weights(wg, wg, wd)
    y = m.moe_grouped_ffn(disp.x_perm, disp.offsets, packed)
    out = m.moe_combine(y, disp.row_of_pair, idx, w, E_local=8)
    torch.cuda.synchronize()
    assert out.shape == (0, 256)


@pytest.mark.parametrize("fused", [False, True], ids=["permuted", "fused"])
@pytest.mark.parametrize("case", ["T1", "k1", "kE", "E1", "one_hot_expert", "empty_experts"])
def test_degenerate_layers(case, fused):
    base = dict(T=300, H=256, E=8, k=2, F=256, dtype="bf16", logits="gauss", seed=77)
    if case == "T1":
        base.update(T=1)
    elif case == "k1":
        base.update(k=1)
    elif case == "kE":
        base.update(E=4, k=4)
    elif case == "E1":
        base.update(E=1, k=1)
    wl = moe_inputs.Workload(case, **base)
    if case in ("one_hot_expert", "empty_experts"):
        inp = moe_inputs.make_inputs(wl)
        L = inp.logits.copy()
        if case == "one_hot_expert":
            L[:, 5] += 100.0  # every token picks expert 5 first
        else:
            L[:, [1, 2, 6]] -= 100.0  # experts 1, 2, 6 stay empty
        inp.logits = L
        d = Dev(inp)
        g = run_layer(d, fused=fused)
        idx, w = oracle.route_topk(L, wl.k)
        check_route(g, idx, w)
        check_dispatch(g, d, oracle.dispatch(idx, wl.E))
        ref = oracle.moe_tokens(inp, idx, w)
        assert layer_err(g["out"], ref) <= BAR["bf16"]
        if case == "empty_experts":
            assert (g["counts"][[1, 2, 6]] == 0).all()
        return
    full_check(wl, fused=fused)


@pytest.mark.parametrize("fused", [False, True], ids=["permuted", "fused"])
def test_window_of_local_experts(fused):
    """Route over 32 experts, hold experts [8, 16): picks outside the window contribute nothing.

    A window's partial sums are heavy-tailed (many tokens have one small local pick or none), so the bf16
    output's own rounding can exceed the 2e-2 bar by itself; the kernels are checked with an fp32 output, and
    the bf16 output against the oracle's bf16 rounding floor."""
    wl = moe_inputs.Workload("window", T=200, H=256, E=32, k=4, F=256, dtype="bf16", logits="gauss", seed=5,
                             e_lo=8, E_local=8)
    g, inp, d, ref, tokens = full_check(wl, out_f32=True, fused=fused)
    assert (g["out"][~np.isin(oracle.route_topk(inp.logits, 4)[0], np.arange(8, 16)).any(axis=1)] == 0).all()
    gb = run_layer(d, packed=g["packed"], fused=fused)
    err = layer_err(gb["out"], ref)
    assert err <= out_floor(ref, "bf16") + 5e-3, err


def test_identity_experts_combine_gives_x():
    """With y_perm = x_perm (in fp32), the combine returns sum_j w_j x_t = x_t up to fp32 rounding."""
    m = lib()
    wl = moe_inputs.Workload("ident", T=500, H=384, E=16, k=4, F=128, dtype="bf16", logits="gauss", seed=3)
    inp = moe_inputs.make_inputs(wl, with_weights=False)
    d_x = _dev(inp.x, "bf16")
    idx, w = m.moe_route_topk(torch.from_numpy(inp.logits).cuda(), wl.k)
    disp = m.moe_dispatch_permute(d_x, idx, wl.E)
    out = m.moe_combine(disp.x_perm.float(), disp.row_of_pair, idx, w, E_local=wl.E, out_dtype=torch.float32)
    x = moe_inputs.stored_x_values(inp)
    ridx, rw = oracle.route_topk(inp.logits, wl.k)
    ref = x * rw.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=4e-7, atol=1e-30)
    np.testing.assert_allclose(out.cpu().numpy(), x, rtol=1e-6, atol=1e-30)


def run_capacity(d: Dev, C, fused, out_f32=False):
    m = lib()
    wl = d.inp.wl
    idx, w = m.moe_route_topk(d.logits, wl.k)
    disp = m.moe_dispatch_permute(d.x, idx, wl.E, x_scales=d.x_scales, gather=not fused, capacity=C)
    packed = m.moe_pack_ffn_weights(*d.w, *d.s)
    od = torch.float32 if (wl.dtype == "f32" or out_f32) else torch.bfloat16
    if fused:
        y = m.moe_grouped_ffn_fused(d.x, disp.token_of_row, disp.row_of_pair, w, disp.offsets, packed,
                                    x_scales=d.x_scales)
        out = m.moe_combine_slots(y, idx, E_local=wl.E, out_dtype=od, row_of_pair=disp.row_of_pair)
    else:
        assert disp.x_perm.shape[0] == min(wl.T * wl.k, wl.E * C)
        y = m.moe_grouped_ffn(disp.x_perm, disp.offsets, packed, x_perm_scales=disp.x_perm_scales)
        out = m.moe_combine(y, disp.row_of_pair, idx, w, E_local=wl.E, out_dtype=od)
    torch.cuda.synchronize()
    return disp, out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("fused", [False, True], ids=["permuted", "fused"])
@pytest.mark.parametrize("case", [("cap_bf16", 300, 256, 8, 2, 256, "bf16", "zipf", 40),
                                  ("cap_fp8", 200, 256, 16, 4, 2048, "fp8", "zipf", 30),
                                  ("cap_k1", 200, 256, 8, 1, 256, "bf16", "gauss", 10)], ids=lambda c: c[0])
def test_capacity_dispatch_and_layer(case, fused):
    """Fixed capacity: each expert keeps its first C pairs (bit-exact vs the oracle); dropped pairs add nothing.

    Outputs with dropped picks are partial sums (heavy-tailed, some rows zero), so, as in the window test, the
    kernels are checked with an fp32 output and the bf16 output against the oracle's bf16 rounding floor."""
    name, T, H, E, k, F, dt, lg, C = case
    wl = moe_inputs.Workload(name, T=T, H=H, E=E, k=k, F=F, dtype=dt, logits=lg, seed=zlib.crc32(name.encode()) % 1000)
    inp = moe_inputs.make_inputs(wl)
    d = Dev(inp)
    disp, out = run_capacity(d, C, fused, out_f32=True)
    ridx, rw = oracle.route_topk(inp.logits, k)
    counts, offsets, rop, tor, keep = oracle.dispatch_capacity(ridx, E, C)
    assert 0 < keep.sum() < keep.size  # some pairs are dropped
    np.testing.assert_array_equal(disp.counts.cpu().numpy(), counts)
    np.testing.assert_array_equal(disp.offsets.cpu().numpy(), offsets)
    np.testing.assert_array_equal(disp.row_of_pair.cpu().numpy(), rop)
    np.testing.assert_array_equal(disp.token_of_row.cpu().numpy()[: offsets[E]], tor)
    if not fused:
        idx_t = torch.from_numpy(tor.astype(np.int64)).cuda()
        assert torch.equal(disp.x_perm[: offsets[E]].view(torch.uint8), d.x[idx_t].view(torch.uint8))
    ref = oracle.moe_tokens(inp, ridx, rw, keep=keep)
    err = layer_err(out, ref)
    _, out16 = run_capacity(d, C, fused)
    err16, floor = layer_err(out16, ref), out_floor(ref, dt)
    print(f"{name}{' fused' if fused else ''}: capacity {C}, kept {keep.sum()}/{keep.size}: err {err:.3e} "
          f"(fp32 out), {err16:.3e} (bf16 out; its floor {floor:.3e})")
    assert err <= BAR[dt]
    if dt != "f32":
        assert err16 <= max(BAR[dt], floor + 5e-3), (err16, floor)


@pytest.mark.parametrize("fused", [False, True], ids=["permuted", "fused"])
def test_capacity_on_the_skewed_workload(fused):
    """Capacity factor 1.25 on the skewed workload: the hot experts drop most of their pairs."""
    wl = moe_inputs.get("skewed_bf16")
    inp = moe_inputs.make_inputs(wl)
    d = Dev(inp)
    C = int(np.ceil(1.25 * wl.T * wl.k / wl.E))
    disp, out = run_capacity(d, C, fused, out_f32=True)
    ridx, rw = oracle.route_topk(inp.logits, wl.k)
    counts, offsets, rop, tor, keep = oracle.dispatch_capacity(ridx, wl.E, C)
    np.testing.assert_array_equal(disp.row_of_pair.cpu().numpy(), rop)
    tokens = sample_tokens(ridx, wl, 16)
    ref = oracle.moe_tokens(inp, ridx, rw, tokens=tokens, keep=keep)
    err = layer_err(out[tokens], ref)
    print(f"skewed capacity {C}: kept {keep.sum()}/{keep.size}: err {err:.3e}")
    assert err <= BAR["bf16"]


def test_wrappers_on_a_side_stream_allocate_there():
    """The functional wrappers run on a side stream, allocating their outputs and workspaces there, while the
    current stream allocates, fills and frees memory in between: the results equal a run on the current stream bit
    for bit (memory a wrapper allocated is not handed to other work while its kernels may still run)."""
    m = lib()
    wl = moe_inputs.Workload("side", T=3000, H=512, E=16, k=4, F=1024, dtype="bf16", logits="gauss", seed=12)
    d = Dev(moe_inputs.make_inputs(wl))
    packed = m.moe_pack_ffn_weights(*d.w, *d.s)
    torch.cuda.synchronize()

    def layer(stream):
        idx, w = m.moe_route_topk(d.logits, wl.k, stream=stream)
        disp = m.moe_dispatch_permute(d.x, idx, wl.E, stream=stream)
        y = m.moe_grouped_ffn(disp.x_perm, disp.offsets, packed, stream=stream)
        return m.moe_combine(y, disp.row_of_pair, idx, w, E_local=wl.E, stream=stream)

    ref = layer(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for i in range(3):
        outs.append(layer(side))
        for _ in range(4):  # churn the current stream's allocations while the side stream works
            junk = torch.empty(wl.T * wl.k * wl.H * 2, dtype=torch.float32, device="cuda").fill_(float(i))
            del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)


def test_fused_split_calls_match_fused_call():
    """moe_grouped_ffn_gate_up_gather + moe_grouped_ffn_down_scatter give the bytes moe_grouped_ffn_fused gives
    (the benchmark times the two halves separately); covers a split down product (few output tiles)."""
    m = lib()
    wl = moe_inputs.Workload("split", T=600, H=256, E=8, k=2, F=1024, dtype="bf16", logits="gauss", seed=21)
    d = Dev(moe_inputs.make_inputs(wl))
    a = run_layer(d, fused=True)
    idx, w = m.moe_route_topk(d.logits, wl.k)
    disp = m.moe_dispatch_permute(d.x, idx, wl.E, gather=False)
    ws = torch.empty(m.moe_grouped_ffn_workspace_bytes(a["packed"], wl.T * wl.k), dtype=torch.uint8, device="cuda")
    y = torch.empty((wl.T * wl.k, wl.H), dtype=torch.float32, device="cuda")
    m.moe_grouped_ffn_gate_up_gather(d.x, disp.token_of_row, disp.offsets, a["packed"], ws)
    m.moe_grouped_ffn_down_scatter(disp.offsets, a["packed"], ws, disp.token_of_row, disp.row_of_pair, w, y)
    out = m.moe_combine_slots(y, idx, E_local=wl.E, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y, a["y_perm"])
    np.testing.assert_array_equal(out.float().cpu().numpy().astype(np.float64), a["out"])


@pytest.mark.parametrize("fused", [False, True], ids=["permuted", "fused"])
def test_deterministic_and_launch_independent(fused):
    """Two runs give identical bytes for every output (no atomics in any reduction)."""
    wl = moe_inputs.Workload("det", T=700, H=256, E=16, k=4, F=256, dtype="fp8", logits="zipf", seed=9)
    inp = moe_inputs.make_inputs(wl)
    d = Dev(inp)
    a = run_layer(d, fused=fused)
    b = run_layer(d, packed=a["packed"], fused=fused)
    for key in ["topk_idx", "topk_w", "counts", "offsets", "row_of_pair", "token_of_row", "out"]:
        np.testing.assert_array_equal(a[key], b[key])
    assert torch.equal(a["y_perm"], b["y_perm"])


@pytest.mark.parametrize("E,k,T,C", [(256, 8, 1000, None), (1024, 8, 700, None), (1024, 32, 200, None),
                                     (1024, 4, 3000, 9), (256, 8, 1000, 25),
                                     # above 16384 pairs: the histogram / scan / rank launches, up to 1024 experts
                                     (256, 8, 2500, 25), (1024, 8, 3000, None), (1024, 4, 5000, 9),
                                     # k = 32 (a rank tile is 8 chunks of 64 pairs; up to 3584 earlier pairs
                                     # counted per workgroup) and k = 1, with ragged last count and rank tiles
                                     (64, 32, 700, None), (8, 1, 20001, None), (48, 32, 613, 50)])
def test_dispatch_and_combine_with_many_experts(E, k, T, C):
    """Up to the domain's 1024 experts (the scans' one-thread-per-expert paths), with and without a capacity, on
    both counting forms (one workgroup up to 16384 pairs, three launches above): bit-exact tables and permuted
    rows, and the combine of seeded expert outputs against the oracle's."""
    m = lib()
    H = 256
    rng = np.random.default_rng(E + k + T)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16).cuda()
    idx, w = m.moe_route_topk(torch.from_numpy(logits).cuda(), k)
    disp = m.moe_dispatch_permute(x, idx, E, capacity=C)
    torch.cuda.synchronize()
    ig = idx.cpu().numpy()
    if C is None:
        ref = oracle.dispatch(ig, E)
    else:
        counts, offsets, rop, tor, keep = oracle.dispatch_capacity(ig, E, C)
        ref = (counts, offsets, rop, tor)
    g = dict(counts=disp.counts.cpu().numpy(), offsets=disp.offsets.cpu().numpy(),
             row_of_pair=disp.row_of_pair.cpu().numpy(),
             token_of_row=disp.token_of_row.cpu().numpy()[: int(ref[1][E])], x_perm=None)
    check_dispatch(g, None, ref)
    n = int(ref[1][E])
    tor = torch.from_numpy(ref[3].astype(np.int64)).cuda()
    assert torch.equal(disp.x_perm[:n].view(torch.int16), x[tor].view(torch.int16))
    # combine of seeded expert outputs (fp32 out) against the oracle's slot-ordered weighted sum
    y = torch.from_numpy(rng.standard_normal((disp.x_perm.shape[0], H)).astype(np.float32)).cuda()
    out = m.moe_combine(y, disp.row_of_pair, idx, w, E_local=E, out_dtype=torch.float32)
    torch.cuda.synchronize()
    wv = w.cpu().numpy().astype(np.float64)
    rop = ref[2]
    if C is not None:
        wv = wv * keep.reshape(T, k)  # dropped pairs add nothing
        rop = np.where(rop < 0, 0, rop)
    refo = oracle.combine(y.cpu().numpy(), rop, ig, wv, 0, E)
    err = np.max(np.abs(out.cpu().numpy() - refo)) / np.sqrt(np.mean(refo**2))
    assert err < 1e-5, err


def test_integer_outputs_and_rows_do_not_depend_on_the_launch_grid():
    """The same pairs through launches of different shape give the same bits.

    Dispatch: 20000 pairs take the multi-workgroup count/scan/rank form, the first 3000 tokens' 12000 pairs the
    one-workgroup form; ordering is stable by pair, so a prefix token's rank inside its expert and its permuted
    row agree between the two.  Route and combine: a short tail of tokens (a different grid and, in the combine,
    the row-sliced form) reproduces the full launch's bits for those tokens, since each token's picks and its
    slot-ordered fp32 sum do not depend on the other tokens."""
    m = lib()
    T, T1, H, E, k = 5000, 3000, 256, 16, 4
    rng = np.random.default_rng(4242)
    logits = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16).cuda()
    idx, w = m.moe_route_topk(logits, k)
    big = m.moe_dispatch_permute(x, idx, E)
    small = m.moe_dispatch_permute(x[:T1], idx[:T1], E)
    torch.cuda.synchronize()
    ig = idx.cpu().numpy()
    for disp, n in ((big, T), (small, T1)):  # both forms against the oracle
        counts, offsets, rop, tor = oracle.dispatch(ig[:n], E)
        np.testing.assert_array_equal(disp.offsets.cpu().numpy(), offsets)
        np.testing.assert_array_equal(disp.row_of_pair.cpu().numpy(), rop)
    e_of = ig[:T1].reshape(-1)
    rank_big = big.row_of_pair.cpu().numpy()[: T1 * k] - big.offsets.cpu().numpy()[e_of]
    rank_small = small.row_of_pair.cpu().numpy() - small.offsets.cpu().numpy()[e_of]
    np.testing.assert_array_equal(rank_big, rank_small)
    rows_big = big.row_of_pair[: T1 * k].long()
    rows_small = small.row_of_pair.long()
    assert torch.equal(big.x_perm[rows_big].view(torch.uint8), small.x_perm[rows_small].view(torch.uint8))
    # route and combine on a 40-token tail
    s = T - 40
    idx_t, w_t = m.moe_route_topk(logits[s:], k)
    y = torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32)).cuda()
    out = m.moe_combine(y, big.row_of_pair, idx, w, E_local=E, out_dtype=torch.float32)
    out_t = m.moe_combine(y, big.row_of_pair[s * k:], idx[s:], w[s:], E_local=E, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(idx_t, idx[s:]) and torch.equal(w_t.view(torch.int32), w[s:].view(torch.int32))
    assert torch.equal(out_t.view(torch.int32), out[s:].view(torch.int32))


@pytest.mark.parametrize("fused", [False, True], ids=["permuted", "fused"])
@pytest.mark.parametrize("dtype,H,F", [("bf16", 65536, 128), ("bf16", 128, 65536), ("f32", 65536, 128)],
                         ids=["bf16_H65536", "bf16_F65536", "f32_H65536"])
def test_largest_hidden_and_ffn_sizes(dtype, H, F, fused):
    """The largest H and F the ABI accepts (65536): 128 KiB-256 KiB rows, 512-1024 pipeline stages per tile,
    the widest per-lane byte offsets; full output against the oracle."""
    wl = moe_inputs.Workload(f"max_{dtype}_{H}_{F}", T=40, H=H, E=2, k=1, F=F, dtype=dtype, logits="gauss",
                             seed=H // 128 + F // 128)
    full_check(wl, fused=fused)


@pytest.mark.parametrize("case", [c for c in SMALL if c[0] in ("s_f32_bm64", "s_bf16_bm32", "s_bf16_bm128",
                                                              "s_bf16_ksplit", "s_bf16_k12", "s_fp8_bm64",
                                                              "s_fp8_bm256")], ids=lambda c: c[0])
def test_gather_form_gives_the_permuted_bits(case):
    """MoELayer(form="gather"): the gate/up product reads x rows through token_of_row (no x_perm), then the
    permuted down product and combine.  Every row of h is the same row of the same product, so y_perm and the
    output equal the permuted form's bit for bit."""
    m = lib()
    name, T, H, E, k, F, dt, lg = case
    wl = moe_inputs.Workload(name, T=T, H=H, E=E, k=k, F=F, dtype=dt, logits=lg, seed=zlib.crc32(name.encode()) % 997)
    inp = moe_inputs.make_inputs(wl)
    d = Dev(inp)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[dt]
    outs = {}
    for form in ("permuted", "gather"):
        layer = m.MoELayer(T, H, E, k, F, tdt, *d.w, *d.s, form=form)
        layer.forward(d.logits, d.x, d.x_scales)
        torch.cuda.synchronize()
        assert (layer.disp.x_perm is None) == (form == "gather")
        outs[form] = (layer.y_perm.clone(), layer.out.clone())
    assert torch.equal(outs["gather"][0], outs["permuted"][0])  # every expert is local: all T*k rows written
    assert torch.equal(outs["gather"][1], outs["permuted"][1])


@pytest.mark.parametrize("dt,F", [("bf16", 256), ("fp8", 2048)])
def test_gather_form_with_a_capacity_gives_the_permuted_bits(dt, F):
    """Fixed capacity through the gather form's entry points (dispatch without x_perm, gate/up gathering x rows,
    permuted down product, combine skipping dropped pairs) against the permuted form with the same capacity."""
    m = lib()
    wl = moe_inputs.Workload(f"cap_gather_{dt}", T=300, H=256, E=8, k=2, F=F, dtype=dt, logits="zipf", seed=61)
    d = Dev(moe_inputs.make_inputs(wl))
    C = 40
    packed = m.moe_pack_ffn_weights(*d.w, *d.s)
    idx, w = m.moe_route_topk(d.logits, wl.k)
    res = {}
    for form in ("permuted", "gather"):
        disp = m.moe_dispatch_permute(d.x, idx, wl.E, x_scales=d.x_scales, gather=form == "permuted", capacity=C)
        # both halves of the FFN take the same R_max: x_perm's rows (E*C here) or token_of_row's (T*k)
        R = disp.x_perm.shape[0] if form == "permuted" else wl.T * wl.k
        ws = torch.empty(m.moe_grouped_ffn_workspace_bytes(packed, R), dtype=torch.uint8, device="cuda")
        y = torch.zeros((R, wl.H), dtype=torch.float32, device="cuda")
        if form == "permuted":
            m.moe_grouped_ffn_gate_up(disp.x_perm, disp.offsets, packed, ws, disp.x_perm_scales)
        else:
            assert disp.x_perm is None
            m.moe_grouped_ffn_gate_up_gather(d.x, disp.token_of_row, disp.offsets, packed, ws, d.x_scales)
        m.moe_grouped_ffn_down(disp.offsets, packed, ws, y)
        out = m.moe_combine(y, disp.row_of_pair, idx, w, E_local=wl.E, out_dtype=torch.float32)
        torch.cuda.synchronize()
        res[form] = (disp.row_of_pair.clone(), y, out)
    assert torch.equal(res["gather"][0], res["permuted"][0])
    assert (res["gather"][0] < 0).any()  # some pairs are dropped
    Rp = res["permuted"][1].shape[0]
    assert Rp == wl.E * C < wl.T * wl.k
    assert torch.equal(res["gather"][1][:Rp], res["permuted"][1]) and not res["gather"][1][Rp:].any()
    assert torch.equal(res["gather"][2], res["permuted"][2])


CANARY = 0x7FC0DEAD  # a quiet-NaN bit pattern no kernel produces


def _canary(shape, dtype=torch.float32):
    n = int(np.prod(shape)) * torch.finfo(dtype).bits // 32 if dtype.is_floating_point else int(np.prod(shape))
    return torch.full((n,), CANARY, dtype=torch.int32, device="cuda").view(dtype).view(*shape)


@pytest.mark.parametrize("dtype,F,T", [("bf16", 256, 200), ("fp8", 2048, 300), ("f32", 256, 150),
                                       ("bf16", 512, 3000)])
def test_outputs_outside_the_window_keep_their_bits(dtype, F, T):
    """The grouped FFN on a window of local experts writes exactly the window's rows of y_perm (the small cases
    take the split reduction, whose partial sums are added over the window's rows only), and the fused form
    exactly the slots of the window's pairs: every other element keeps a NaN canary bit for bit, and the
    written elements equal those of a run into zeroed buffers."""
    m = lib()
    H, E, k, e_lo, E_local = 256, 32, 4, 8, 8
    wl = moe_inputs.Workload(f"canary_{dtype}", T=T, H=H, E=E, k=k, F=F, dtype=dtype, logits="gauss", seed=17,
                             e_lo=e_lo, E_local=E_local)
    print(f"canary: {dtype} T={T} F={F}", flush=True)
    d = Dev(moe_inputs.make_inputs(wl))
    idx, w = m.moe_route_topk(d.logits, k)
    disp = m.moe_dispatch_permute(d.x, idx, E, x_scales=d.x_scales)
    packed = m.moe_pack_ffn_weights(*d.w, *d.s)
    R = T * k
    y = _canary((R, H))
    y0 = torch.zeros((R, H), dtype=torch.float32, device="cuda")
    for out in (y, y0):
        m.moe_grouped_ffn(disp.x_perm, disp.offsets, packed, x_perm_scales=disp.x_perm_scales, e_lo=e_lo, y_perm=out)
    ys = _canary((R, H))
    ys0 = torch.zeros((R, H), dtype=torch.float32, device="cuda")
    for out in (ys, ys0):
        m.moe_grouped_ffn_fused(d.x, disp.token_of_row, disp.row_of_pair, w, disp.offsets, packed,
                                x_scales=d.x_scales, e_lo=e_lo, y_slot=out)
    torch.cuda.synchronize()
    off = disp.offsets.cpu().numpy()
    r0, r1 = int(off[e_lo]), int(off[e_lo + E_local])
    assert 0 < r0 < r1 < R
    yb, y0b = y.view(torch.int32).cpu(), y0.view(torch.int32).cpu()
    assert (yb[:r0] == CANARY).all() and (yb[r1:] == CANARY).all()
    assert torch.equal(yb[r0:r1], y0b[r0:r1]) and torch.isfinite(y0[r0:r1]).all()
    local = ((idx >= e_lo) & (idx < e_lo + E_local)).reshape(-1).cpu()
    sb, s0b = ys.view(torch.int32).cpu(), ys0.view(torch.int32).cpu()
    assert (sb[~local] == CANARY).all()
    assert torch.equal(sb[local], s0b[local]) and torch.isfinite(ys0[local.cuda()]).all()


def test_dispatch_rows_past_the_kept_rows_keep_their_bits():
    """With a capacity, x_perm (and its fp8 scale rows) and token_of_row have rows for E * C pairs, of which
    offsets[E] are kept: the dispatch writes exactly those, on both counting forms (one workgroup, and the
    count / scan / rank+gather launches above 16384 pairs)."""
    m = lib()
    for T, E, k, C in ((300, 16, 4, 70), (5000, 16, 4, 1400)):
        H = 256
        print(f"dispatch canary: T={T} E={E} k={k} C={C}", flush=True)
        wl = moe_inputs.Workload(f"dcanary_{T}", T=T, H=H, E=E, k=k, F=256, dtype="fp8", logits="zipf", seed=T)
        d = Dev(moe_inputs.make_inputs(wl))
        idx, _ = m.moe_route_topk(d.logits, k)
        rows = min(T * k, E * C)
        out = m.Dispatch(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
                         offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                         row_of_pair=torch.empty(T * k, dtype=torch.int32, device="cuda"),
                         token_of_row=_canary((T * k,), torch.int32),
                         x_perm=_canary((rows, H // 4), torch.float32).view(torch.uint8).view(rows, H),
                         x_perm_scales=_canary((rows, H // 128)))
        m.moe_dispatch_permute(d.x, idx, E, x_scales=d.x_scales, out=out, capacity=C)
        torch.cuda.synchronize()
        n = int(out.offsets[E])
        assert 0 < n < rows
        assert (out.x_perm[n:].contiguous().view(torch.int32) == CANARY).all()
        assert (out.x_perm_scales[n:].view(torch.int32) == CANARY).all()
        assert (out.token_of_row[n:] == CANARY).all()
        tor = out.token_of_row[:n].long()
        assert torch.equal(out.x_perm[:n], d.x[tor]) and torch.equal(out.x_perm_scales[:n], d.x_scales[tor])
