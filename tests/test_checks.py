"""CPU self-tests of the comparison rules the GPU parity tests use (tests/checks.py): each rule accepts the
oracle's own values and rejects plausible mistakes planted in the oracle's inputs (a reduction block dropped, a
row taken from the wrong pair, a code moved away from a midpoint, a wrong scale)."""
import dataclasses

import numpy as np
import pytest

import checks
import moe_inputs
import oracle


def _ref(dtype, F=256, H=256, T=40, seed=11):
    wl = moe_inputs.Workload("chk", T=T, H=H, E=4, k=2, F=F, dtype=dtype, logits="gauss", seed=seed)
    inp = moe_inputs.make_inputs(wl)
    idx, _ = oracle.route_topk(inp.logits, wl.k)
    pairs = np.arange(wl.T * wl.k)
    return wl, inp, idx, pairs, oracle.pair_h(inp, idx, pairs)


@pytest.mark.parametrize("dtype", ["fp8", "bf16", "f32"])
def test_check_h_accepts_the_oracle_and_rejects_planted_mistakes(dtype):
    wl, inp, idx, pairs, ref = _ref(dtype)
    st = checks.check_h(dtype, wl.H, ref, ref["h_bits"], ref["h_scales"])
    assert st["differing"] == 0 and st["elements"] == len(pairs) * wl.F
    # one reduction block of x (128 columns) dropped for every pair: a skipped pipeline stage
    x = inp.x.copy()
    x[:, 128:256] = 0
    bad = oracle.pair_h(dataclasses.replace(inp, x=x), idx, pairs)
    with pytest.raises(AssertionError):
        checks.check_h(dtype, wl.H, ref, bad["h_bits"], bad["h_scales"])
    # the rows of the wrong pairs (one row off): a dropped or shifted row
    with pytest.raises(AssertionError):
        checks.check_h(dtype, wl.H, ref, np.roll(ref["h_bits"], 1, axis=0),
                       None if ref["h_scales"] is None else np.roll(ref["h_scales"], 1, axis=0))
    if dtype == "f32":
        return
    # one element moved to its neighbour where the exact value is far from any midpoint
    da = checks.a_bound(ref, dtype, wl.H)
    scale = np.repeat(ref["h_scales"], 128, axis=1).astype(np.float64) if dtype == "fp8" else 1.0
    v = ref["a"] / scale
    vals = checks.e4m3_values(ref["h_bits"]) if dtype == "fp8" else checks.bf16_values(ref["h_bits"])
    rel = np.abs(v - vals) / np.maximum(np.abs(vals), 1e-30)
    mag = ref["h_bits"] & (0x7F if dtype == "fp8" else 0x7FFF)
    far = da / scale < 1e-3 * np.abs(v)  # the error bound is a small part of the code spacing
    cand = np.nonzero((rel < 1e-3) & far & (mag > 8) & (mag < (0x70 if dtype == "fp8" else 0x7F00)))
    i, j = cand[0][0], cand[1][0]
    moved = ref["h_bits"].copy()
    moved[i, j] += 1
    with pytest.raises(AssertionError):
        checks.check_h(dtype, wl.H, ref, moved, ref["h_scales"])
    if dtype == "fp8":
        # a group's scale taken from its neighbour group
        sc = ref["h_scales"].copy()
        sc[3, 1] = sc[3, 0]
        with pytest.raises(AssertionError):
            checks.check_h(dtype, wl.H, ref, ref["h_bits"], sc)


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_check_h_takes_either_neighbour_only_at_a_midpoint(dtype):
    """Constructed values a hair from a midpoint: both neighbours pass; a value the same distance from the
    midpoint but outside the error bound must keep its own code."""
    F = 128
    mids = np.array([1.5 + 0.125 / 2, 3.0 + 0.25 / 2, -(20.0 + 2.0 / 2), 0.75 + 0.0625 / 2])  # e4m3 midpoints
    if dtype == "bf16":
        mids = np.array([1.0 + 2.0**-8, 3.0 + 2.0**-7, -(20.0 + 2.0**-4), 0.75 + 2.0**-9])  # bf16 midpoints
    n = len(mids)
    g = np.full((n, F), 3.0)
    u = np.ones((n, F))
    a = np.zeros((n, F))
    sig = 1.0 / (1.0 + np.exp(-3.0))
    # a = silu(g) u with u chosen per element; element 0 of each row sits 1e-6 relative above a midpoint, element 1 at
    # 1e-3 relative above it; the rest small
    a[:, 2:] = 0.1
    a[:, 0] = mids * (1 + 1e-6)
    a[:, 1] = mids * (1 + 1e-3)
    u = a / (3.0 * sig)
    ref = dict(g=g, u=u, gabs=np.abs(g) * 2, uabs=np.abs(u) * 2, a=a)
    if dtype == "fp8":
        # scale 1 for every group: put 448 in the last column so max|a| / 448 = 1
        a[:, -1] = 448.0
        u[:, -1] = 448.0 / (3.0 * sig)
        ref["uabs"] = np.abs(u) * 2
        import torch
        ref["h_scales"] = np.ones((n, 1), np.float32)
        codes = torch.from_numpy(a.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    else:
        import torch
        codes = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
        codes = codes.astype(np.uint16)
    ref["h_bits"] = codes.astype(np.uint32)
    base = checks.check_h(dtype, 256, ref, ref["h_bits"], ref.get("h_scales"))
    assert base["window"] >= n  # the near-midpoint elements
    down = ref["h_bits"].copy()
    down[:, 0] -= 1  # the other neighbour for element 0 (1e-6 from the midpoint): accepted
    checks.check_h(dtype, 256, ref, down, ref.get("h_scales"))
    down1 = ref["h_bits"].copy()
    down1[:, 1] -= 1  # 1e-3 relative from the midpoint: outside the bound, rejected
    with pytest.raises(AssertionError):
        checks.check_h(dtype, 256, ref, down1, ref.get("h_scales"))


def _bwd_inputs(T, H, F, E, k, seed):
    wl = moe_inputs.Workload("chk_bwd", T=T, H=H, E=E, k=k, F=F, dtype="bf16", logits="gauss", seed=seed)
    inp = moe_inputs.make_inputs(wl)
    idx, w = oracle.route_topk(inp.logits, k)
    dout = np.random.default_rng(seed + 1).standard_normal((T, H))
    return wl, inp, idx, w, dout


def _bound_ratio(got, ref, absum, K):
    u = 2.0**-8
    b = (2 * u + K * 2.0**-24) * absum + 2.0**-24 * np.abs(ref)
    return float(np.max(np.abs(got - ref) / b))


def test_noise_ratio_flags_a_dropped_row_that_the_worst_case_bound_admits():
    """Weight gradients over a long reduction (about 600 rows per expert): the oracle's values with simulated
    rounding noise pass both checks; the same with one row of an expert dropped (a pair removed through the
    capacity mask) stays within the elementwise worst-case bound on most elements (so a sample of a few dozen
    elements would likely pass it) but fails the noise check."""
    wl, inp, idx, w, dout = _bwd_inputs(T=1200, H=128, F=128, E=2, k=1, seed=31)
    res = oracle.backward_weights(inp, idx, w, dout, with_abs=True, with_sq=True)
    dwg, ag, sg = res[0], res[3], res[6]
    K = wl.T * wl.k + wl.H
    rng = np.random.default_rng(5)
    noisy = dwg + rng.standard_normal(dwg.shape) * 0.6 * np.sqrt((2.0**-16 / 3) * sg)
    assert _bound_ratio(noisy, dwg, ag, K) <= 1.0
    assert checks.noise_ratio(noisy, dwg, sg, K, "bf16", False) <= 1.0
    keep = np.ones(wl.T * wl.k, np.uint8)
    keep[int(np.nonzero(idx.reshape(-1) == 1)[0][0])] = 0  # expert 1's first row
    dropped = oracle.backward_weights(inp, idx, w, dout, keep=keep)[0]
    b = (2 * 2.0**-8 + K * 2.0**-24) * ag[1] + 2.0**-24 * np.abs(dwg[1])
    assert np.mean(np.abs(dropped[1] - dwg[1]) > b) < 0.05  # the worst-case bound admits it almost everywhere
    assert checks.noise_ratio(dropped[1], dwg[1], sg[1], K, "bf16", False) > 3.0


def test_noise_ratio_and_bound_flag_a_dropped_stage_of_dx():
    """dx: 64 reduction columns (one pipeline stage of the dX product) dropped for one expert fails both checks."""
    wl, inp, idx, w, dout = _bwd_inputs(T=64, H=256, F=512, E=4, k=2, seed=37)
    dx, _, _, dxa, dxs = oracle.backward_rows(inp, idx, w, dout, with_abs=True, with_sq=True)
    K = wl.H + 2 * wl.F
    wg, wu = inp.w_gate.copy(), inp.w_up.copy()
    wg[2, :, 64:128] = 0  # bf16 bit pattern 0 = 0.0
    wu[2, :, 64:128] = 0
    bad = oracle.backward_rows(dataclasses.replace(inp, w_gate=wg, w_up=wu), idx, w, dout)[0]
    u = 2.0**-8
    b = (2 * u + K * 2.0**-24) * dxa + u * np.abs(dx)
    assert float(np.max(np.abs(bad - dx) / b)) > 1.0
    assert checks.noise_ratio(bad, dx, dxs, K, "bf16", True) > 3.0
