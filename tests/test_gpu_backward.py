"""GPU parity of the training path (moe_grouped_ffn_train + moe_grouped_ffn_backward) against the oracle.

Every gradient is compared element by element with the oracle's fp64 backward on the GPU's own routing.

dx and the weight gradients: each element is a sum of terms whose one rounded operand ([dg | du], or w * h for
dWd) is stored in the layer dtype (unit roundoff u = 2^-8 for bf16, 2^-24 for fp32), accumulated in fp32 over
at most K terms (a nested fp32 sum feeds dg: K counts both), so
    |gpu - oracle| <= (2 u + K 2^-24) * A + u_out |oracle|,
A = sum of |terms| from the oracle, u_out the rounding of the output itself (dx in the layer dtype; fp32
weight gradients).  The factor 2 covers the rounded operand and second-order effects.
Beside that worst-case bound (which grows with the sum of |terms|, so on long reductions it would also admit a
dropped term), the rounding noise: sqrt(sum err^2 / sum var) <= 1 over all compared elements, var being the
expected variance of one rounded operand per term (tests/checks.py noise_ratio, from the oracle's sums of squared
terms).
d_topk_w and d_logits: max |gpu - oracle| / RMS(oracle) within the forward's bar for the dtype (their error
comes from the forward's y).  The full Mixtral shape is checked on sampled tokens (every expert's first and last
row among them) and on weight-gradient elements of every expert.
"""
import zlib

import numpy as np
import pytest
import torch

import checks
import moe_inputs
import oracle

pytestmark = pytest.mark.gpu

BAR = {"f32": 1e-4, "bf16": 2e-2}


def lib():
    import grouped_expert_ffn_router_amd as m

    return m


def _dev(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _dout(wl, seed):
    """Seeded loss gradient in the layer dtype, and its exact fp64 values."""
    d32 = np.random.default_rng(seed).standard_normal((wl.T, wl.H), dtype=np.float32)
    if wl.dtype == "bf16":
        bits = moe_inputs._store(d32, "bf16")[0]
        return _dev(bits, "bf16"), moe_inputs.bf16_bits_to_f32(bits).astype(np.float64)
    return _dev(d32, "f32"), d32.astype(np.float64)


def run_training(inp, capacity=None, want_logits=True, seed=7, to_host=True):
    """Route, dispatch, the training forward and the backward through the C ABI; host copies of the gradients
    (to_host=False keeps them on the device)."""
    m = lib()
    wl = inp.wl
    x = _dev(inp.x, wl.dtype)
    w = [_dev(a, wl.dtype) for a in (inp.w_gate, inp.w_up, inp.w_down)]
    idx, tw = m.moe_route_topk(torch.from_numpy(inp.logits).cuda(), wl.k)
    disp = m.moe_dispatch_permute(x, idx, wl.E, capacity=capacity)
    packed = m.moe_pack_ffn_weights(*w)
    h, gu, y = m.moe_grouped_ffn_train(disp.x_perm, disp.offsets, packed, e_lo=wl.e_lo)
    dout, dout64 = _dout(wl, seed)
    g = m.moe_grouped_ffn_backward(dout, idx, tw, disp.row_of_pair, disp.token_of_row, disp.offsets, disp.x_perm, h,
                                   gu, y, *w, E=wl.E, e_lo=wl.e_lo, want_logits=want_logits)
    torch.cuda.synchronize()
    host = {k2: (None if v is None else (v.float().cpu().numpy().astype(np.float64) if to_host else v))
            for k2, v in g.items()}
    host.update(topk_idx=idx.cpu().numpy(), topk_w=tw.cpu().numpy().astype(np.float64), dout64=dout64,
                row_of_pair=disp.row_of_pair.cpu().numpy(), offsets=disp.offsets.cpu().numpy(),
                h=h, gu=gu, y=y, disp=disp, x_perm=disp.x_perm)
    return host


def _err(got, ref):
    rms = float(np.sqrt(np.mean(ref**2)))
    return float(np.max(np.abs(got - ref))) / rms if rms > 0 else float(np.max(np.abs(got)))


U = {"f32": 2.0**-24, "bf16": 2.0**-8}


def bound_ratio(got, ref, absum, K, dtype, out_rounded):
    """max over elements of |got - ref| / ((2 u + K 2^-24) A + u_out |ref|)."""
    u = U[dtype]
    b = (2 * u + K * 2.0**-24) * absum + (u if out_rounded else 2.0**-24) * np.abs(ref)
    err = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(b > 0, err / b, np.where(err > 0, np.inf, 0.0))
    return float(np.max(r)) if r.size else 0.0


def full_check(inp, g, keep=None, label=""):
    wl = inp.wl
    bar = BAR[wl.dtype]
    dx, dtw, dl, dxa, dxs = oracle.backward_rows(inp, g["topk_idx"], g["topk_w"], g["dout64"], keep=keep,
                                                 with_abs=True, with_sq=True)
    dwg, dwu, dwd, ag, au, ad, sg, su, sd = oracle.backward_weights(inp, g["topk_idx"], g["topk_w"], g["dout64"],
                                                                    keep=keep, with_abs=True, with_sq=True)
    Kx = wl.H + 2 * wl.F
    Kw = wl.T * wl.k + wl.H
    ratios = {"dx": bound_ratio(g["dx"], dx, dxa, Kx, wl.dtype, wl.dtype == "bf16"),
              "dw_gate": bound_ratio(g["dw_gate"], dwg, ag, Kw, wl.dtype, False),
              "dw_up": bound_ratio(g["dw_up"], dwu, au, Kw, wl.dtype, False),
              "dw_down": bound_ratio(g["dw_down"], dwd, ad, Kw, wl.dtype, False)}
    noise = {"dx": checks.noise_ratio(g["dx"], dx, dxs, Kx, wl.dtype, wl.dtype == "bf16"),
             "dw_gate": checks.noise_ratio(g["dw_gate"], dwg, sg, Kw, wl.dtype, False),
             "dw_up": checks.noise_ratio(g["dw_up"], dwu, su, Kw, wl.dtype, False),
             "dw_down": checks.noise_ratio(g["dw_down"], dwd, sd, Kw, wl.dtype, False)}
    rel = {"d_topk_w": _err(g["d_topk_w"], dtw)}
    if g["d_logits"] is not None:
        rel["d_logits"] = _err(g["d_logits"], dl)
        # exact zeros off the picks
        off = np.ones_like(dl, dtype=bool)
        np.put_along_axis(off, g["topk_idx"].astype(np.int64), False, axis=1)
        assert np.all(g["d_logits"][off] == 0.0)
    print(f"{label}: err/bound " + ", ".join(f"{k2} {v:.2f}" for k2, v in ratios.items()) + "; noise ratio " +
          ", ".join(f"{k2} {v:.2f}" for k2, v in noise.items()) + "; max/RMS " +
          ", ".join(f"{k2} {v:.2e}" for k2, v in rel.items()) +
          f"; (max/RMS dx {_err(g['dx'], dx):.2e}, dw_gate {_err(g['dw_gate'], dwg):.2e})")
    for k2, v in ratios.items():
        assert v <= 1.0, f"{label}: {k2} outside its rounding bound (err/bound {v:.3g})"
    for k2, v in noise.items():
        assert v <= 1.0, f"{label}: {k2} error above its rounding noise (ratio {v:.3g})"
    for k2, v in rel.items():
        assert v <= bar, f"{label}: {k2} error {v:.3g} above the {wl.dtype} bar {bar}"
    # experts without rows get exactly zero weight gradients
    counts = np.diff(g["offsets"])[wl.e_lo: wl.e_lo + wl.n_local]
    for e in np.nonzero(counts == 0)[0]:
        assert not np.any(g["dw_gate"][e]) and not np.any(g["dw_up"][e]) and not np.any(g["dw_down"][e])
    return ratios


SMALL = [
    # name, T, H, E, k, F, dtype, logits kind, window (e_lo, E_local)
    ("bwd_f32", 96, 256, 4, 2, 256, "f32", "gauss", None),
    ("bwd_bf16", 160, 256, 8, 2, 384, "bf16", "gauss", None),
    ("bwd_bf16_k1", 130, 384, 6, 1, 256, "bf16", "gauss", None),
    ("bwd_bf16_k4_skew", 200, 256, 16, 4, 256, "bf16", "zipf", None),  # hot experts, some empty ones
    ("bwd_f32_window", 120, 256, 8, 2, 256, "f32", "gauss", (2, 3)),
    ("bwd_bf16_window", 150, 256, 8, 3, 384, "bf16", "zipf", (5, 3)),
    # experts averaging >= 256 rows and shapes dividing 256: the 8-wavefront tiles (320-row blocks for the data
    # products, 256 x 256 for the weight products), uniform and skewed
    ("bwd_bf16_big", 600, 512, 2, 1, 512, "bf16", "gauss", None),
    ("bwd_bf16_big_skew", 700, 512, 4, 2, 768, "bf16", "zipf", None),
    ("bwd_bf16_k12", 100, 256, 16, 12, 256, "bf16", "gauss", None),  # k > 8
    # experts with more rows than the products have weight rows: those take their column tiles fastest (H, F of
    # 512 so the 256-wide column tiles are several)
    ("bwd_bf16_hot", 1500, 512, 4, 1, 512, "bf16", "zipf", None),
    ("bwd_f32_hot", 800, 256, 2, 1, 256, "f32", "gauss", None),
    # more than 64 local experts: the data products' tile lookup walks the experts 64 at a time
    ("bwd_bf16_e80", 400, 256, 80, 2, 256, "bf16", "gauss", None),
]


def _inputs(case):
    name, T, H, E, k, F, dt, lg, win = case
    wl = moe_inputs.Workload(name, T=T, H=H, E=E, k=k, F=F, dtype=dt, logits=lg,
                             seed=zlib.crc32(name.encode()) % 1000)
    if win is not None:
        wl = wl.replace(e_lo=win[0], E_local=win[1])
    return moe_inputs.make_inputs(wl)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_backward_small_full(case):
    inp = _inputs(case)
    print(f"case {case[0]}", flush=True)
    g = run_training(inp)
    full_check(inp, g, label=case[0])


def test_backward_training_forward_matches_the_forward():
    """The training forward gives the same y_perm bits as moe_grouped_ffn, h as its own product, and gu whose
    SwiGLU reproduces h."""
    m = lib()
    inp = _inputs(SMALL[1])
    wl = inp.wl
    x = _dev(inp.x, wl.dtype)
    w = [_dev(a, wl.dtype) for a in (inp.w_gate, inp.w_up, inp.w_down)]
    idx, _ = m.moe_route_topk(torch.from_numpy(inp.logits).cuda(), wl.k)
    disp = m.moe_dispatch_permute(x, idx, wl.E)
    packed = m.moe_pack_ffn_weights(*w)
    h, gu, y = m.moe_grouped_ffn_train(disp.x_perm, disp.offsets, packed)
    y2 = m.moe_grouped_ffn(disp.x_perm, disp.offsets, packed)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    gf = gu.float()
    F = wl.F
    a = torch.nn.functional.silu(gf[:, :F]) * gf[:, F:]
    # h is the bf16 rounding of silu(g) * u from the same fp32 accumulators gu holds
    assert float((a - h.float()).abs().max()) <= 2.0**-8 * float(h.float().abs().max())
    # gu against the oracle's g, u on a few rows
    xs = moe_inputs.stored_x_values(inp)
    wg = moe_inputs.bf16_bits_to_f32(inp.w_gate).astype(np.float64)
    tor = disp.token_of_row.cpu().numpy()
    offs = disp.offsets.cpu().numpy()
    for r in [0, 7, int(offs[3]), int(offs[-1]) - 1]:
        e = int(np.searchsorted(offs, r, side="right") - 1)
        gref = xs[tor[r]] @ wg[e]
        err = np.abs(gf[r, :F].cpu().numpy() - gref).max() / np.sqrt(np.mean(gref**2))
        assert err < 2e-2


def test_backward_with_capacity_drops():
    case = ("bwd_cap", 180, 256, 8, 2, 256, "bf16", "zipf", None)
    inp = _inputs(case)
    wl = inp.wl
    C = 30
    g = run_training(inp, capacity=C)
    _, _, _, _, keep = oracle.dispatch_capacity(g["topk_idx"], wl.E, C)
    assert 0 < keep.sum() < keep.size
    full_check(inp, g, keep=keep, label="capacity")
    assert np.all(g["d_topk_w"].reshape(-1)[keep == 0] == 0.0)


def test_backward_without_logits_and_deterministic():
    inp = _inputs(SMALL[1])
    g1 = run_training(inp, want_logits=False)
    g2 = run_training(inp, want_logits=True)
    assert g1["d_logits"] is None
    for k2 in ("dx", "dw_gate", "dw_up", "dw_down", "d_topk_w"):
        np.testing.assert_array_equal(g1[k2], g2[k2])


def test_backward_mixtral_shape_sampled():
    """Full Mixtral shape (T = 2048, H = 4096, F = 14336, E = 8, k = 2, bf16): sampled tokens (dx, d_topk_w,
    d_logits) and sampled weight-gradient elements against the oracle, one by one."""
    inp = moe_inputs.make_inputs(moe_inputs.get("mixtral_bf16"))
    wl = inp.wl
    g = run_training(inp, to_host=False)
    rng = np.random.default_rng(17)
    # every expert's first and last row (its slab's edges in every grouped product), plus seeded tokens
    offs = g["offsets"]
    tor = g["disp"].token_of_row.cpu().numpy()
    edges = {int(tor[offs[e]]) for e in range(wl.E)} | {int(tor[offs[e + 1] - 1]) for e in range(wl.E)}
    toks = np.array(sorted(edges | set(int(t) for t in rng.choice(wl.T, 6, replace=False))))
    dx, dtw, dl, dxa, dxs = oracle.backward_rows(inp, g["topk_idx"], g["topk_w"], g["dout64"], tokens=toks,
                                                 with_abs=True, with_sq=True)
    host = lambda t: t.float().cpu().numpy().astype(np.float64)
    r = bound_ratio(host(g["dx"])[toks], dx, dxa, wl.H + 2 * wl.F, "bf16", True)
    z = checks.noise_ratio(host(g["dx"])[toks], dx, dxs, wl.H + 2 * wl.F, "bf16", True)
    print(f"mixtral dx of {len(toks)} tokens: err/bound {r:.2f}, noise ratio {z:.2f}")
    assert r <= 1.0 and z <= 1.0
    for name, got, ref in [("d_topk_w", host(g["d_topk_w"])[toks], dtw), ("d_logits", host(g["d_logits"])[toks], dl)]:
        e = _err(got, ref)
        print(f"mixtral sampled {name}: max/RMS {e:.2e}")
        assert e <= BAR["bf16"]
    n = 96  # 12 per expert, each of the three gradients
    which = np.tile(np.arange(3), n // 3)
    ex = np.repeat(np.arange(wl.E), n // wl.E)
    ii = np.where(which == 2, rng.integers(0, wl.F, n), rng.integers(0, wl.H, n))
    jj = np.where(which == 2, rng.integers(0, wl.H, n), rng.integers(0, wl.F, n))
    ref, ab, sq = oracle.backward_weight_elems(inp, g["topk_idx"], g["topk_w"], g["dout64"], which, ex, ii, jj,
                                               with_abs=True, with_sq=True)
    mats = (g["dw_gate"], g["dw_up"], g["dw_down"])
    got = np.array([float(mats[a][e, i, j]) for a, e, i, j in zip(which, ex, ii, jj)])
    K = wl.T * wl.k + wl.H
    r = bound_ratio(got, ref, ab, K, "bf16", False)
    z = checks.noise_ratio(got, ref, sq, K, "bf16", False)
    print(f"mixtral weight-gradient elements ({n}, every expert): err/bound {r:.2f}, noise ratio {z:.2f}")
    assert r <= 1.0 and z <= 1.0
