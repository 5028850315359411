"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against a library routine, a closed form printed on the pages, an invariant, or a
special case that reduces to a textbook computation.  The rounding helpers below work on float64 bit patterns
(integer round-half-even on the dropped mantissa bits), a different method from the oracle's binade/nearbyint
codec, and are themselves checked against torch's dtype casts.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import moe_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------------------------------------
# independent exact rounding helpers (float64 bit manipulation)
# ------------------------------------------------------------------------------------------------------------
def _rne_f64(a, mant_bits, min_normal_exp):
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    tiny = np.abs(a) < 2.0**min_normal_exp
    q = 2.0 ** (min_normal_exp - mant_bits)
    out[tiny] = np.rint(a[tiny] / q) * q  # subnormal range of the target: fixed quantum, half-even
    u = a[~tiny].view(np.uint64)
    drop = np.uint64(52 - mant_bits)
    one = np.uint64(1)
    rem = u & ((one << drop) - one)
    half = one << (drop - one)
    keep = u >> drop
    up = (rem > half) | ((rem == half) & ((keep & one) == one))
    out[~tiny] = ((keep + up.astype(np.uint64)) << drop).view(np.float64)
    return out


def bf16_round(a):
    return _rne_f64(a, 7, -126)


def e4m3_round(a):
    r = _rne_f64(a, 3, -6)
    return np.clip(r, -448.0, 448.0)


def test_rounding_helpers_match_torch_casts():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_round(v.astype(np.float64)), ref)
    w = rng.uniform(-440, 440, 20000).astype(np.float32)
    w = np.concatenate([w, rng.uniform(-0.02, 0.02, 5000).astype(np.float32)])
    ref8 = torch.from_numpy(w).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(e4m3_round(w.astype(np.float64)), ref8)


# ------------------------------------------------------------------------------------------------------------
# number formats
# ------------------------------------------------------------------------------------------------------------
def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_decode(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.nanmax(got) == 448.0 and oracle.e4m3_decode(0x01) == 2.0**-9


def test_e4m3_encode_roundtrip_midpoints_and_saturation():
    vals = sorted({oracle.e4m3_decode(c) for c in range(0, 127)})
    for c in range(0, 127):
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c
        assert oracle.e4m3_encode(-oracle.e4m3_decode(c)) == (c | 0x80)
    # every midpoint between neighbours rounds to the neighbour with an even mantissa (torch's RNE cast agrees)
    mids = np.array([(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])])
    ref = torch.from_numpy(mids.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(m) for m in mids], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)
    assert all(int(g) % 2 == 0 for g in got)
    for v in [448.0, 449.0, 463.9, 464.0, 1e6]:
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    rng = np.random.default_rng(3)
    r = rng.uniform(-447, 447, 3000)
    np.testing.assert_array_equal([oracle.e4m3_decode(oracle.e4m3_encode(x)) for x in r], e4m3_round(r))


def test_bf16_codec_vs_torch_and_ties():
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(5000) * np.exp(rng.uniform(-80, 80, 5000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_encode(float(x)) for x in v], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)
    # exact ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert oracle.bf16_encode(1.0 + 2.0**-8) == 0x3F80
    assert oracle.bf16_encode(1.0 + 3 * 2.0**-8) == 0x3F82
    # fp64 input just above a tie rounds up (no double rounding through fp32)
    assert oracle.bf16_encode(1.0 + 2.0**-8 + 2.0**-40) == 0x3F81
    for b in [0x0001, 0x3F80, 0xC2F7, 0x7F7F, 0x0080]:
        assert oracle.bf16_encode(oracle.bf16_decode(b)) == b
    r = rng.standard_normal(3000) * 100
    np.testing.assert_array_equal([oracle.bf16_decode(oracle.bf16_encode(x)) for x in r], bf16_round(r))


# ------------------------------------------------------------------------------------------------------------
# the pages' closed form for the dispatch + combine payload
# ------------------------------------------------------------------------------------------------------------
def test_payload_closed_form_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "traffic_closed_form.json")))
    per_tok = oracle.payload_bytes(1, g["k"], g["H"], g["bytes_per_elem"])
    assert per_tok == g["per_token_per_layer_bytes"] == 114688
    assert per_tok / 1024 == g["per_token_per_layer_KiB"]
    assert g["moe_layers"] * per_tok / 1024 == g["per_token_all_layers_KiB"]
    assert abs(g["moe_layers"] * per_tok / 2**20 - g["per_token_all_layers_MiB_about"]) < 0.05
    total = oracle.payload_bytes(g["prefill_tokens"], g["k"], g["H"], g["bytes_per_elem"]) * g["moe_layers"]
    assert 44.5e9 <= total < 47e9
    # traffic is proportional to H (doubling H doubles it)
    assert oracle.payload_bytes(1, 8, 2 * 7168, 1) == 2 * per_tok
    assert oracle.payload_bytes(0, 8, 7168, 1) == 0


# ------------------------------------------------------------------------------------------------------------
# step 1: routing
# ------------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("E,k", [(8, 2), (32, 8), (64, 4), (1, 1), (5, 5), (256, 8), (1000, 32)])
def test_route_matches_stable_argsort_and_softmax(E, k):
    rng = np.random.default_rng(E * 100 + k)
    L = rng.standard_normal((300, E)).astype(np.float32)
    # plant exact ties across the k boundary and inside the top-k
    L[0, :] = 0.5
    L[1, : min(E, 3)] = 2.0
    if E > 2:
        L[2, E - 1] = L[2, 0]
    idx, w = oracle.route_topk(L, k)
    ref_idx = np.argsort(-L, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(idx, ref_idx)
    sm = scipy.special.softmax(L.astype(np.float64), axis=1)
    ref_w = np.take_along_axis(sm, ref_idx, axis=1)
    ref_w /= ref_w.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, ref_w, rtol=1e-13, atol=0)


def test_route_closed_forms():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((64, 16)).astype(np.float32)
    idx, w = oracle.route_topk(L, 1)
    assert (w == 1.0).all() and (idx[:, 0] == np.argmax(L, axis=1)).all()
    idx, w = oracle.route_topk(np.zeros((4, 16), np.float32), 8)
    assert (idx == np.arange(8)).all() and (w == 1 / 8).all()
    idx, w = oracle.route_topk(L, 2)
    l0 = np.take_along_axis(L, idx[:, :1], 1).astype(np.float64)[:, 0]
    l1 = np.take_along_axis(L, idx[:, 1:2], 1).astype(np.float64)[:, 0]
    np.testing.assert_allclose(w[:, 0], 1 / (1 + np.exp(l1 - l0)), rtol=1e-15)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-15)


def test_route_neg_inf_sorts_last_with_zero_weight():
    L = np.array([[-np.inf, 1.0, -np.inf, 0.0, -np.inf]], np.float32)
    idx, w = oracle.route_topk(L, 4)
    assert idx.tolist() == [[1, 3, 0, 2]]
    assert w[0, 2] == 0.0 and w[0, 3] == 0.0
    assert w[0, 0] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)


# ------------------------------------------------------------------------------------------------------------
# steps 2-3: counts, offsets, permutation
# ------------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k", [(300, 8, 2), (64, 32, 8), (1000, 64, 4), (1, 4, 4), (0, 8, 2), (50, 1, 1)])
def test_dispatch_matches_bincount_and_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E + k)
    L = rng.standard_normal((T, E)).astype(np.float32) + np.linspace(3, 0, E, dtype=np.float32)
    idx, _ = oracle.route_topk(L, k)
    counts, offsets, rop, tor = oracle.dispatch(idx, E)
    flat = idx.reshape(-1)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert counts.sum() == T * k and offsets[E] == T * k
    order = np.argsort(flat, kind="stable")  # row r holds pair order[r]
    np.testing.assert_array_equal(rop[order], np.arange(T * k))
    np.testing.assert_array_equal(np.sort(rop), np.arange(T * k))  # a bijection
    np.testing.assert_array_equal(tor[rop], np.arange(T * k) // k)
    # rows of one expert are contiguous and in ascending token order
    for e in range(E):
        toks = tor[offsets[e]:offsets[e + 1]]
        assert (np.diff(toks) > 0).all()
        assert (flat[order[offsets[e]:offsets[e + 1]]] == e).all()
    # undoing the sort restores the token order: x_perm[row_of_pair[p]] is token p // k's row
    x = rng.standard_normal((T, 3))
    x_perm = x[tor]
    np.testing.assert_array_equal(x_perm[rop].reshape(T, k, 3), np.repeat(x[:, None, :], k, axis=1))


# ------------------------------------------------------------------------------------------------------------
# step 4: the expert FFN and the weighted sum
# ------------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k,C", [(50, 8, 2, 5), (300, 16, 4, 40), (1, 4, 4, 1), (200, 8, 1, 1000),
                                      (400, 64, 4, 7), (120, 3, 3, 2)])
def test_capacity_dispatch_keeps_first_pairs_in_order(T, E, k, C):
    """Fixed capacity: expert e keeps its first C pairs in ascending pair order, packed; the rest are dropped."""
    rng = np.random.default_rng(T * 31 + C)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, rop, tor, keep = oracle.dispatch_capacity(idx, E, C)
    full = np.bincount(idx.ravel(), minlength=E)
    np.testing.assert_array_equal(counts, np.minimum(full, C))
    assert offsets[0] == 0
    np.testing.assert_array_equal(np.diff(offsets), counts)
    flat = idx.ravel()
    for e in range(E):
        ps = np.nonzero(flat == e)[0]  # ascending pair order
        kept, dropped = ps[:C], ps[C:]
        assert (keep[kept] == 1).all() and (keep[dropped] == 0).all()
        np.testing.assert_array_equal(rop[kept], offsets[e] + np.arange(len(kept)))
        assert (rop[dropped] == -1).all()
        np.testing.assert_array_equal(tor[rop[kept]], kept // k)
    if C >= full.max():  # nothing dropped: the uncapped dispatch exactly
        for a, b in zip((counts, offsets, rop, tor), oracle.dispatch(idx, E)):
            np.testing.assert_array_equal(a, b)
    if C == 1:  # each expert keeps its lowest pair index
        for e in range(E):
            ps = np.nonzero(flat == e)[0]
            if len(ps):
                assert keep[ps[0]] == 1 and keep[ps[1:]].sum() == 0


def test_dropped_pairs_equal_zero_weights():
    """A dropped pair contributes nothing: the same as routing weight 0 for that pair (the layer is linear in
    the weights); keeping every pair is the uncapped layer."""
    inp = _small("bf16", T=40, E=4, k=2)
    idx, w = oracle.route_topk(inp.logits, 2)
    _, _, _, _, keep = oracle.dispatch_capacity(idx, 4, 12)
    assert 0 < keep.sum() < keep.size
    dropped = oracle.moe_tokens(inp, idx, w, keep=keep)
    zeroed = oracle.moe_tokens(inp, idx, w * keep.reshape(w.shape))
    np.testing.assert_array_equal(dropped, zeroed)
    np.testing.assert_array_equal(oracle.moe_tokens(inp, idx, w, keep=np.ones_like(keep)),
                                  oracle.moe_tokens(inp, idx, w))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_router_logits_vs_library_matmul_and_identity(dtype):
    """Router logits x W_r: an independent fp64 library matmul on the decoded stored x; W_r = [I | 0] returns the
    first E columns of x exactly; linear in W_r."""
    inp = _small(dtype, T=33, H=256, E=8, logits="router")
    x = moe_inputs.stored_x_values(inp)
    lg, ab = oracle.router_logits(inp)
    np.testing.assert_allclose(lg, x @ inp.w_router.astype(np.float64), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ab, np.abs(x)[:, :, None].__mul__(np.abs(inp.w_router.astype(np.float64))[None]).sum(1),
                               rtol=1e-12)
    eye = np.zeros((256, 8), np.float32)
    eye[np.arange(8), np.arange(8)] = 1.0
    lg_i, _ = oracle.router_logits(inp, eye)
    np.testing.assert_array_equal(lg_i, x[:, :8])
    lg2, _ = oracle.router_logits(inp, inp.w_router * 2)
    np.testing.assert_array_equal(lg2, 2 * lg)
    if dtype != "fp8":  # the generator's fp32 logits are these values rounded once
        np.testing.assert_array_equal(lg.astype(np.float32), inp.logits)


def _small(dtype, T=24, H=256, E=4, k=2, F=256, seed=0, logits="gauss"):
    wl = moe_inputs.Workload("pin", T=T, H=H, E=E, k=k, F=F, dtype=dtype, logits=logits, seed=seed)
    return moe_inputs.make_inputs(wl)


def _weights_f64(inp):
    """Exact fp64 values of the stored weights (scales applied), natural layouts."""
    wl = inp.wl
    def dec(a, s):
        if wl.dtype == "f32":
            return a.astype(np.float64)
        if wl.dtype == "bf16":
            return moe_inputs.bf16_bits_to_f32(a).astype(np.float64)
        v = moe_inputs.e4m3_codes_to_f32(a).astype(np.float64)
        return v * np.repeat(np.repeat(s.astype(np.float64), 128, axis=1), 128, axis=2)
    return dec(inp.w_gate, inp.s_gate), dec(inp.w_up, inp.s_up), dec(inp.w_down, inp.s_down)


def _store_h(a, dtype):
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_round(a)
    R, F = a.shape
    g = a.reshape(R, F // 128, 128)
    amax = np.abs(g).max(axis=2)
    s = np.where(amax == 0, 1.0, (amax / 448.0).astype(np.float32)).astype(np.float64)
    return (e4m3_round(g / s[:, :, None]) * s[:, :, None]).reshape(R, F)


def _vectorised_layer(inp):
    """Independent formulation: library argsort for routing, library matmuls per expert over all of its rows,
    scatter of the expert outputs back by pair index."""
    wl = inp.wl
    L = inp.logits.astype(np.float64)
    idx = np.argsort(-inp.logits, axis=1, kind="stable")[:, : wl.k]
    sel = np.take_along_axis(L, idx, 1)
    w = scipy.special.softmax(sel, axis=1)
    x = moe_inputs.stored_x_values(inp)
    Wg, Wu, Wd = _weights_f64(inp)
    Y = np.zeros((wl.T, wl.k, wl.H))
    for e in range(wl.n_local):
        tt, jj = np.nonzero(idx == e + wl.e_lo)
        if len(tt) == 0:
            continue
        X = torch.from_numpy(x[tt])
        G = X @ torch.from_numpy(Wg[e])
        U = X @ torch.from_numpy(Wu[e])
        A = (torch.nn.functional.silu(G) * U).numpy()
        h = torch.from_numpy(_store_h(A, wl.dtype))
        Y[tt, jj] = (h @ torch.from_numpy(Wd[e])).numpy()
    return (w[:, :, None] * Y).sum(axis=1)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_layer_brute_force_vs_vectorised(dtype):
    inp = _small(dtype, seed={"f32": 1, "bf16": 2, "fp8": 3}[dtype])
    res = oracle.layer(inp)
    ref = _vectorised_layer(inp)
    rms = np.sqrt(np.mean(ref**2))
    assert rms > 0.05
    # identical math up to fp64 summation order; an h element that lands within fp64 noise of a rounding
    # boundary could flip, so the bound is loose enough for that and tight enough to catch any real mistake
    assert np.max(np.abs(res["out"] - ref)) / rms < (1e-12 if dtype == "f32" else 1e-9)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_pair_h_vs_library_matmuls_and_the_storage_rule(dtype):
    """oracle.pair_h (the SwiGLU intermediate of each pair before and after its storage) against library fp64
    matmuls of the decoded inputs, the independent bit-level rounding helpers, and the layer oracle: the stored h
    of every pair, times W_down and summed with the routing weights, is the layer output."""
    inp = _small(dtype, T=30, H=256, E=4, k=2, F=384, seed={"f32": 21, "bf16": 22, "fp8": 23}[dtype])
    wl = inp.wl
    idx, w = oracle.route_topk(inp.logits, wl.k)
    pairs = np.arange(wl.T * wl.k)
    r = oracle.pair_h(inp, idx, pairs)
    x = torch.from_numpy(moe_inputs.stored_x_values(inp))
    Wg, Wu, Wd = (torch.from_numpy(a) for a in _weights_f64(inp))
    t, e = pairs // wl.k, torch.from_numpy(idx.reshape(-1).astype(np.int64))
    xt = x[t]
    G = torch.einsum("ph,phf->pf", xt, Wg[e])
    U = torch.einsum("ph,phf->pf", xt, Wu[e])
    GA = torch.einsum("ph,phf->pf", xt.abs(), Wg[e].abs())
    UA = torch.einsum("ph,phf->pf", xt.abs(), Wu[e].abs())
    tol = 1e-12 * float(GA.max())
    for name, ref in (("g", G), ("u", U), ("gabs", GA), ("uabs", UA)):
        np.testing.assert_allclose(r[name], ref.numpy(), rtol=0, atol=tol, err_msg=name)
    A = (torch.nn.functional.silu(G) * U).numpy()
    np.testing.assert_allclose(r["a"], A, rtol=0, atol=tol)
    # the stored elements: the rounding of the oracle's own a, by the independent helpers
    a = r["a"]
    if dtype == "f32":
        np.testing.assert_array_equal(r["h_bits"].astype(np.uint32).view(np.float32), a.astype(np.float32))
        h = a.astype(np.float32).astype(np.float64)
    elif dtype == "bf16":
        h = bf16_round(a)
        got = torch.from_numpy(r["h_bits"].astype(np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(got, h)
    else:
        g = a.reshape(len(a), -1, 128)
        amax = np.abs(g).max(axis=2)
        s = np.where(amax == 0, 1.0, (amax / 448.0).astype(np.float32)).astype(np.float32)
        np.testing.assert_array_equal(r["h_scales"], s)
        q = e4m3_round(g / s.astype(np.float64)[:, :, None]).reshape(a.shape)
        got = torch.from_numpy(r["h_bits"].astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
        np.testing.assert_array_equal(got, q)
        h = q * np.repeat(s.astype(np.float64), 128, axis=1)
    # the stored h agrees with the vectorised formulation's storage rule, and drives the layer output
    np.testing.assert_allclose(h, _store_h(A, dtype), rtol=0, atol=1e-9 * np.abs(h).max())
    Y = torch.einsum("pf,pfh->ph", torch.from_numpy(h), Wd[e]).numpy()
    out = (Y.reshape(wl.T, wl.k, wl.H) * w[:, :, None]).sum(axis=1)
    ref_out = oracle.layer(inp)["out"]
    assert np.max(np.abs(out - ref_out)) <= 1e-12 * np.abs(ref_out).max()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_dense_special_case_E1_k1(dtype):
    """E = 1, k = 1: every token goes to the one expert with weight 1, so the layer is a dense SwiGLU block."""
    inp = _small(dtype, T=9, E=1, k=1, seed=4)
    res = oracle.layer(inp)
    assert (res["topk_idx"] == 0).all() and (res["topk_w"] == 1.0).all()
    x = torch.from_numpy(moe_inputs.stored_x_values(inp))
    Wg, Wu, Wd = (torch.from_numpy(a[0]) for a in _weights_f64(inp))
    a = torch.nn.functional.silu(x @ Wg) * (x @ Wu)
    ref = (torch.from_numpy(_store_h(a.numpy(), dtype)) @ Wd).numpy()
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_linearity_label_permutation_and_zero_input():
    inp = _small("f32", seed=9, E=6, k=3)
    base = oracle.layer(inp)["out"]
    # doubling W_down doubles the output exactly
    inp2 = moe_inputs.Inputs(**{**inp.__dict__, "w_down": inp.w_down * np.float32(2)})
    np.testing.assert_array_equal(oracle.layer(inp2)["out"], 2 * base)
    # relabelling the experts together with their logits and weights leaves the output unchanged
    perm = np.array([3, 0, 5, 1, 4, 2])
    inv = np.argsort(perm)
    inp3 = moe_inputs.Inputs(**{**inp.__dict__, "logits": np.ascontiguousarray(inp.logits[:, perm]),
                                "w_gate": inp.w_gate[perm], "w_up": inp.w_up[perm], "w_down": inp.w_down[perm]})
    assert (oracle.route_topk(inp3.logits, 3)[0] == inv[oracle.route_topk(inp.logits, 3)[0]]).all()
    np.testing.assert_array_equal(oracle.layer(inp3)["out"], base)
    # zero input gives zero output
    inp4 = moe_inputs.Inputs(**{**inp.__dict__, "x": np.zeros_like(inp.x)})
    assert (oracle.layer(inp4)["out"] == 0).all()


def test_window_drops_non_local_experts():
    inp = _small("bf16", E=8, k=4, seed=12)
    idx, w = oracle.route_topk(inp.logits, 4)
    full = oracle.moe_tokens(inp, idx, w, e_lo=0, E_local=8)
    wl = inp.wl
    sub = moe_inputs.Inputs(**{**inp.__dict__, "wl": wl.replace(e_lo=2, E_local=3), "w_gate": inp.w_gate[2:5],
                               "w_up": inp.w_up[2:5], "w_down": inp.w_down[2:5]})
    part = oracle.moe_tokens(sub, idx, w)
    rest = moe_inputs.Inputs(**{**inp.__dict__, "wl": wl.replace(e_lo=0, E_local=2), "w_gate": inp.w_gate[:2],
                                "w_up": inp.w_up[:2], "w_down": inp.w_down[:2]})
    rest2 = moe_inputs.Inputs(**{**inp.__dict__, "wl": wl.replace(e_lo=5, E_local=3), "w_gate": inp.w_gate[5:],
                                 "w_up": inp.w_up[5:], "w_down": inp.w_down[5:]})
    # the windows partition the experts, so their outputs add up to the full layer
    tot = part + oracle.moe_tokens(rest, idx, w) + oracle.moe_tokens(rest2, idx, w)
    np.testing.assert_allclose(tot, full, rtol=0, atol=1e-13 * np.abs(full).max())
    none = np.ones(wl.T, bool)
    none[np.isin(idx, [2, 3, 4]).any(axis=1)] = False
    assert (part[none] == 0).all()


def test_identity_experts_combine_gives_x():
    """With every expert output equal to its input row, the combine gives sum_j w_j x_t = x_t."""
    inp = _small("bf16", T=40, E=8, k=3, seed=21)
    idx, w = oracle.route_topk(inp.logits, 3)
    counts, offsets, rop, tor = oracle.dispatch(idx, 8)
    x = moe_inputs.stored_x_values(inp)
    y = x[tor]  # the permuted rows, passed through unchanged
    out = oracle.combine(y, rop, idx, w, 0, 8)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-15)
    np.testing.assert_allclose(out, x, rtol=1e-15, atol=1e-15)
    # one-hot weights (k = 1) return the expert output row itself
    idx1, w1 = oracle.route_topk(inp.logits, 1)
    _, _, rop1, tor1 = oracle.dispatch(idx1, 8)
    np.testing.assert_array_equal(oracle.combine(x[tor1], rop1, idx1, w1, 0, 8), x)


def test_generator_is_deterministic():
    wl = moe_inputs.Workload("det", T=16, H=128, E=4, k=2, F=128, dtype="fp8", logits="gauss", seed=5)
    a, b = moe_inputs.make_inputs(wl), moe_inputs.make_inputs(wl)
    for f in ["x", "x_scales", "logits", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"]:
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    c = moe_inputs.make_inputs(wl, seed=6)
    assert not np.array_equal(a.x, c.x)


def test_skewed_bias_gives_about_a_quarter_to_the_top_expert():
    wl = moe_inputs.get("skewed_bf16").replace(T=4096)
    inp = moe_inputs.make_inputs(wl, with_weights=False)
    idx, _ = oracle.route_topk(inp.logits, wl.k)
    share = np.bincount(idx.ravel(), minlength=wl.E) / idx.size
    assert 0.22 < share[0] < 0.28
    assert (share == 0).sum() > 20  # many empty experts


# ------------------------------------------------------------------------------------------------------------
# Backward pass (training): pinned by torch fp64 autograd of an independently written forward, by central
# finite differences of the forward oracle (itself pinned above), and by the softmax-Jacobian invariant.
# ------------------------------------------------------------------------------------------------------------
def _torch_grads(inp, dout, keep=None):
    """fp64 autograd of a vectorised forward (library argsort routing, per-expert matmuls, h stored in the
    layer dtype with a straight-through rounding).  -> dx, dWg, dWu, dWd, d_topk_w, d_logits."""
    wl = inp.wl
    idx = np.argsort(-inp.logits, axis=1, kind="stable")[:, : wl.k]
    L = torch.tensor(inp.logits.astype(np.float64), requires_grad=True)
    w = torch.softmax(torch.gather(L, 1, torch.from_numpy(idx)), dim=1)
    x = torch.tensor(moe_inputs.stored_x_values(inp), requires_grad=True)
    Wg, Wu, Wd = (torch.tensor(a, requires_grad=True) for a in _weights_f64(inp))
    D = torch.from_numpy(dout)

    def out_of(wts):
        out = torch.zeros((wl.T, wl.H), dtype=torch.float64)
        for e in range(wl.n_local):
            m = idx == e + wl.e_lo
            if keep is not None:
                m &= keep.reshape(wl.T, wl.k).astype(bool)
            tt, jj = np.nonzero(m)
            if len(tt) == 0:
                continue
            tt_t = torch.from_numpy(tt)
            X = x[tt_t]
            A = torch.nn.functional.silu(X @ Wg[e]) * (X @ Wu[e])
            Hs = A + (torch.from_numpy(_store_h(A.detach().numpy(), wl.dtype)) - A).detach()
            out = out.index_add(0, tt_t, wts[tt_t, torch.from_numpy(jj)][:, None] * (Hs @ Wd[e]))
        return out

    (out_of(w) * D).sum().backward()
    w_leaf = w.detach().clone().requires_grad_(True)
    (dw,) = torch.autograd.grad((out_of(w_leaf) * D).sum(), w_leaf)  # leaves the other .grad fields alone
    return (x.grad.numpy(), Wg.grad.numpy(), Wu.grad.numpy(), Wd.grad.numpy(), dw.numpy(), L.grad.numpy())


def _bwd_case(dtype, seed, **kw):
    inp = _small(dtype, seed=seed, **kw)
    rng = np.random.default_rng(seed + 100)
    dout = rng.standard_normal((inp.wl.T, inp.wl.H))
    idx, w = oracle.route_topk(inp.logits, inp.wl.k)
    return inp, dout, idx, w


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b**2)), 1e-300))


@pytest.mark.parametrize("dtype,kw", [("f32", {}), ("bf16", {}), ("f32", dict(E=6, k=3, F=384)),
                                      ("bf16", dict(T=40, E=8, k=2, E_local=3, e_lo=2))])
def test_backward_matches_torch_autograd(dtype, kw):
    wl_kw = {k2: v for k2, v in kw.items() if k2 not in ("E_local", "e_lo")}
    inp, dout, idx, w = _bwd_case(dtype, 11, **wl_kw)
    if "E_local" in kw:  # a window of local experts: the weights hold only those
        wl = inp.wl.replace(e_lo=kw["e_lo"], E_local=kw["E_local"])
        sl = slice(kw["e_lo"], kw["e_lo"] + kw["E_local"])
        inp = moe_inputs.Inputs(wl, inp.x, inp.x_scales, inp.logits, inp.w_gate[sl], inp.w_up[sl], inp.w_down[sl],
                                None, None, None)
    dx_t, dwg_t, dwu_t, dwd_t, dtw_t, dl_t = _torch_grads(inp, dout)
    dx, dtw, dl = oracle.backward_rows(inp, idx, w, dout)
    dwg, dwu, dwd = oracle.backward_weights(inp, idx, w, dout)
    for got, ref in [(dx, dx_t), (dwg, dwg_t), (dwu, dwu_t), (dwd, dwd_t), (dtw, dtw_t), (dl, dl_t)]:
        assert np.sqrt(np.mean(ref**2)) > 1e-3
        assert _rel(got, ref) < 1e-10


def test_backward_with_capacity_drops_matches_autograd():
    inp, dout, idx, w = _bwd_case("f32", 12, T=32, E=4, k=2)
    _, _, _, _, keep = oracle.dispatch_capacity(idx, 4, 9)
    assert 0 < keep.sum() < keep.size
    dx_t, dwg_t, dwu_t, dwd_t, dtw_t, dl_t = _torch_grads(inp, dout, keep=keep)
    dx, dtw, dl = oracle.backward_rows(inp, idx, w, dout, keep=keep)
    dwg, dwu, dwd = oracle.backward_weights(inp, idx, w, dout, keep=keep)
    for got, ref in [(dx, dx_t), (dwg, dwg_t), (dwu, dwu_t), (dwd, dwd_t), (dtw, dtw_t), (dl, dl_t)]:
        assert _rel(got, ref) < 1e-10
    assert np.all(dtw.reshape(-1)[keep == 0] == 0.0)


def test_backward_finite_differences_of_the_forward_oracle():
    """Central differences of L = <dout, out> through the forward oracle, fp32 layer."""
    inp, dout, idx, w = _bwd_case("f32", 13, T=12, H=128, F=128, E=4, k=2)
    wl = inp.wl
    dx, dtw, dl = oracle.backward_rows(inp, idx, w, dout)
    dwg, dwu, dwd = oracle.backward_weights(inp, idx, w, dout)

    def loss(inp2, w2=w):
        return float(np.sum(dout * oracle.moe_tokens(inp2, idx, w2)))

    def fd_array(name, arr, pos, delta=2.0**-7):
        a = arr.copy()
        lo = a.copy()
        a[pos] = np.float32(arr[pos] + delta)
        lo[pos] = np.float32(arr[pos] - delta)
        step = float(a[pos]) - float(lo[pos])
        return (loss(dataclasses_replace(inp, **{name: a})) - loss(dataclasses_replace(inp, **{name: lo}))) / step

    rng = np.random.default_rng(5)
    for _ in range(6):
        t, c = int(rng.integers(wl.T)), int(rng.integers(wl.H))
        assert abs(fd_array("x", inp.x, (t, c)) - dx[t, c]) < 1e-4 * np.sqrt(np.mean(dx**2))
    used = sorted(set(idx.reshape(-1).tolist()))
    for name, g in [("w_gate", dwg), ("w_up", dwu), ("w_down", dwd)]:
        for _ in range(4):
            e = used[int(rng.integers(len(used)))]
            i, j = int(rng.integers(g.shape[1])), int(rng.integers(g.shape[2]))
            fd = fd_array(name, getattr(inp, name), (e, i, j))
            assert abs(fd - g[e, i, j]) < 1e-4 * np.sqrt(np.mean(g**2)), name
    # routing weights: the loss is linear in each weight
    for t, j in [(0, 0), (3, 1), (wl.T - 1, 1)]:
        wp, wm = w.copy(), w.copy()
        wp[t, j] += 0.5
        wm[t, j] -= 0.5
        assert abs(loss(inp, wp) - loss(inp, wm) - dtw[t, j]) < 1e-9 * max(1.0, abs(dtw[t, j]))
    # logits: re-route (picks unchanged for a small step) and run the forward with the new weights
    for t, e in [(1, int(idx[1, 0])), (2, int(idx[2, 1])), (4, int(np.setdiff1d(np.arange(4), idx[4])[0]))]:
        vals = []
        for sgn in (1, -1):
            L2 = inp.logits.copy()
            L2[t, e] = np.float32(L2[t, e] + sgn * 2.0**-10)
            i2, w2 = oracle.route_topk(L2, wl.k)
            assert (i2 == idx).all()
            vals.append((loss(inp, w2), float(L2[t, e])))
        fd = (vals[0][0] - vals[1][0]) / (vals[0][1] - vals[1][1])
        assert abs(fd - dl[t, e]) < 1e-5 * max(1.0, np.abs(dl).max())


def dataclasses_replace(inp, **kw):
    import dataclasses

    return dataclasses.replace(inp, **kw)


def test_backward_invariants_and_sampled_elements():
    inp, dout, idx, w = _bwd_case("bf16", 14, T=30, E=5, k=3)
    wl = inp.wl
    dx, dtw, dl = oracle.backward_rows(inp, idx, w, dout)
    # the softmax Jacobian: every token's logit gradient sums to zero, and non-picked experts get none
    assert np.all(np.abs(dl.sum(axis=1)) < 1e-12 * (1 + np.abs(dl).max()))
    for t in range(wl.T):
        assert np.all(dl[t, np.setdiff1d(np.arange(wl.E), idx[t])] == 0.0)
    # the sampled element routine agrees with the full weight gradients
    dwg, dwu, dwd = oracle.backward_weights(inp, idx, w, dout)
    rng = np.random.default_rng(3)
    n = 40
    which = rng.integers(0, 3, n)
    ex = rng.integers(0, wl.E, n)
    ii = np.where(which == 2, rng.integers(0, wl.F, n), rng.integers(0, wl.H, n))
    jj = np.where(which == 2, rng.integers(0, wl.H, n), rng.integers(0, wl.F, n))
    got = oracle.backward_weight_elems(inp, idx, w, dout, which, ex, ii, jj)
    ref = np.array([(dwg, dwu, dwd)[a][e, i, j] for a, e, i, j in zip(which, ex, ii, jj)])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    # the listed-token routine agrees with the all-token one, and dout = 0 gives zero gradients
    dx2, dtw2, dl2 = oracle.backward_rows(inp, idx, w, dout, tokens=[5, 0, 29])
    np.testing.assert_array_equal(dx2, dx[[5, 0, 29]])
    np.testing.assert_array_equal(dtw2, dtw[[5, 0, 29]])
    z = oracle.backward_rows(inp, idx, w, np.zeros_like(dout))
    assert all(np.all(a == 0) for a in z)
    # the gradient is linear in dout
    dxh, _, _ = oracle.backward_rows(inp, idx, w, 0.5 * dout)
    np.testing.assert_allclose(dxh, 0.5 * dx, rtol=1e-12, atol=1e-15)


def test_backward_absolute_term_sums():
    """The |term| sums bound the gradients, equal them for an all-positive case, and agree between routines."""
    inp, dout, idx, w = _bwd_case("f32", 15, T=20, E=4, k=2)
    dx, dtw, dl, dxa = oracle.backward_rows(inp, idx, w, dout, with_abs=True)
    dwg, dwu, dwd, ag, au, ad = oracle.backward_weights(inp, idx, w, dout, with_abs=True)
    for v, a in [(dx, dxa), (dwg, ag), (dwu, au), (dwd, ad)]:
        assert np.all(np.abs(v) <= a * (1 + 1e-12)) and np.all(a >= 0)
        assert np.mean(np.abs(v) < 0.999 * a) > 0.5  # terms of both signs in most sums
    # the sampled routine's sums equal the full routine's
    which = np.array([0, 1, 2, 2, 0])
    ex = np.array([0, 1, 2, 3, 3])
    ii = np.array([3, 5, 7, 200, 100])
    jj = np.array([9, 11, 13, 17, 250])
    got, ga = oracle.backward_weight_elems(inp, idx, w, dout, which, ex, ii, jj, with_abs=True)
    ref = np.array([(ag, au, ad)[a][e, i, j] for a, e, i, j in zip(which, ex, ii, jj)])
    np.testing.assert_allclose(ga, ref, rtol=1e-12)
    # sign flip of dout leaves the sums unchanged
    _, _, _, dxa2 = oracle.backward_rows(inp, idx, w, -dout, with_abs=True)
    np.testing.assert_allclose(dxa2, dxa, rtol=1e-12)


def test_backward_squared_term_sums():
    """The sums of squared terms (rounding-noise estimates) lie between (sum |t|)^2 / K and (sum |t|)^2 (Cauchy-
    Schwarz, K terms per sum), scale with dout squared, and agree between the full and the sampled routines."""
    inp, dout, idx, w = _bwd_case("bf16", 16, T=20, E=4, k=2)
    wl = inp.wl
    _, _, _, dxa, dxs = oracle.backward_rows(inp, idx, w, dout, with_abs=True, with_sq=True)
    res = oracle.backward_weights(inp, idx, w, dout, with_abs=True, with_sq=True)
    ab, sq = res[3:6], res[6:9]
    rows_per_expert = np.bincount(idx.reshape(-1), minlength=wl.E)[:, None, None]
    for a, q, K in [(dxa, dxs, 2 * wl.F * wl.k)] + [(a, q, np.maximum(rows_per_expert, 1)) for a, q in zip(ab, sq)]:
        assert np.all(q <= a * a * (1 + 1e-12)) and np.all(q * K >= a * a * (1 - 1e-12))
    _, _, _, dxs2 = oracle.backward_rows(inp, idx, w, 2.0 * dout, with_sq=True)
    np.testing.assert_allclose(dxs2, 4.0 * dxs, rtol=1e-12)
    which, ex = np.array([0, 1, 2]), np.array([0, 1, 3])
    ii, jj = np.array([3, 5, 7]), np.array([9, 11, 13])
    _, gsq = oracle.backward_weight_elems(inp, idx, w, dout, which, ex, ii, jj, with_sq=True)
    np.testing.assert_allclose(gsq, [sq[a][e, i, j] for a, e, i, j in zip(which, ex, ii, jj)], rtol=1e-12)
