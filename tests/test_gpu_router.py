"""GPU parity of moe_router_topk (router logits x W_r fused with the softmax top-k) against the oracle.

Logits: every element within the fp32 dot-product bound (H + 3) 2^-24 sum_h |x_h W_r[h, e]| of the oracle's
fp64 value.  Routing: bit-exact against the oracle's route on the GPU's own logits (ties to the lower id), and
bit-identical to moe_route_topk on those logits.  Against routing on the host logits, picks may differ only at
near-ties, where two logits are closer than their error bounds; such flips are counted and printed.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def lib():
    import grouped_expert_ffn_router_amd as m

    return m


def _dev(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _synthetic(name, T, H, E, k, dtype, seed):
    """Inputs with the generator's recipe for x and W_r; H need not be a multiple of 128 for f32/bf16."""
    if H % 128 == 0:
        wl = moe_inputs.get("tiny_fp32").replace(name=name, T=T, H=H, E=E, k=k, F=128, dtype=dtype, seed=seed)
        return moe_inputs.make_inputs(wl, with_weights=False)
    assert dtype == "f32"
    wl = moe_inputs.get("tiny_fp32").replace(name=name, T=T, H=H, E=E, k=k, F=128, dtype=dtype, seed=seed)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H), dtype=np.float32)
    w_r = (rng.standard_normal((H, E), dtype=np.float32) / np.float32(np.sqrt(H))).astype(np.float32)
    return moe_inputs.Inputs(wl, x, None, None, None, None, None, None, None, None, w_r)


CASES = {
    # the two layer shapes whose logits are defined as x W_r
    "tiny_fp32": lambda: moe_inputs.make_inputs(moe_inputs.get("tiny_fp32"), with_weights=False),
    "mixtral_bf16": lambda: moe_inputs.make_inputs(moe_inputs.get("mixtral_bf16"), with_weights=False),
    # fp8 activations (code value times the 128-column block scale), E = 16, ragged T
    "fp8_e16": lambda: _synthetic("fp8_e16", 203, 384, 16, 4, "fp8", 2001),
    # H not a multiple of the 64-column chunk, E = 3 (partial rows), k = E
    "f32_h136_e3": lambda: _synthetic("f32_h136_e3", 77, 136, 3, 3, "f32", 2002),
    # the largest E, k = 8; E = 1; an E that is not a power of two
    "bf16_e64": lambda: _synthetic("bf16_e64", 130, 256, 64, 8, "bf16", 2003),
    "f32_e1": lambda: _synthetic("f32_e1", 50, 128, 1, 1, "f32", 2004),
    "bf16_e33": lambda: _synthetic("bf16_e33", 100, 512, 33, 5, "bf16", 2005),
    # k > 8 picks from E = 48
    "f32_e48_k20": lambda: _synthetic("f32_e48_k20", 70, 256, 48, 20, "f32", 2007),
    # above 64 experts: the tiled logits kernel, then the route selection (E not a multiple of the 64-expert tile,
    # fp8 activations with 256 experts, the domain's 1024, a ragged token tile)
    "bf16_e100": lambda: _synthetic("bf16_e100", 300, 512, 100, 6, "bf16", 2008),
    "fp8_e256": lambda: _synthetic("fp8_e256", 257, 1024, 256, 8, "fp8", 2009),
    "f32_e1024": lambda: _synthetic("f32_e1024", 130, 256, 1024, 32, "f32", 2010),
    "f32_h136_e128": lambda: _synthetic("f32_h136_e128", 77, 136, 128, 4, "f32", 2011),
}


def _check_router(inp, logits_g, idx_g, w_g, label):
    wl = inp.wl
    ref, absdot = oracle.router_logits(inp)
    bound = (wl.H + 3) * U * absdot
    err = np.abs(logits_g.astype(np.float64) - ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    assert np.all(err <= bound), f"{label}: logits outside the fp32 bound (worst err/bound {worst:.3g})"
    # routing on the GPU's own logits: bit-exact picks, weights within 2 ulp of the fp64 oracle
    ridx, rw = oracle.route_topk(logits_g, wl.k)
    np.testing.assert_array_equal(idx_g, ridx)
    r32 = rw.astype(np.float32)
    assert np.all(np.abs(w_g.astype(np.float64) - r32.astype(np.float64)) <= 2 * np.spacing(np.abs(r32)))
    # against routing on the host's fp32 rounding of the exact logits: flips only at near-ties
    hidx, _ = oracle.route_topk(ref.astype(np.float32), wl.k)
    flips = np.nonzero(np.any(hidx != idx_g, axis=1))[0]
    for t in flips:
        j = int(np.argmax(hidx[t] != idx_g[t]))
        a, b = int(hidx[t, j]), int(idx_g[t, j])
        gap = abs(ref[t, a] - ref[t, b])
        assert gap <= bound[t, a] + bound[t, b] + 2 * np.spacing(np.float32(abs(ref[t, a]))), \
            f"{label}: token {t} flipped expert {a} -> {b} with fp64 gap {gap:.3g}"
    print(f"{label}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} {wl.dtype}: worst err/bound {worst:.3g}, "
          f"{len(flips)} near-tie flips vs host routing")
    return ref


@pytest.mark.parametrize("case", list(CASES))
def test_router_logits_and_routing_match_the_oracle(case):
    m = lib()
    inp = CASES[case]()
    wl = inp.wl
    print(f"case {case}", flush=True)
    x = _dev(inp.x, wl.dtype)
    xs = None if inp.x_scales is None else torch.from_numpy(inp.x_scales).cuda()
    wr = torch.from_numpy(inp.w_router).cuda()
    logits, idx, w = m.moe_router_topk(x, wr, wl.k, x_scales=xs)
    torch.cuda.synchronize()
    lg, ig, wg = logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    _check_router(inp, lg, ig, wg, case)
    # the same selection as moe_route_topk on these logits, bit for bit
    idx2, w2 = m.moe_route_topk(logits, wl.k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx2.cpu().numpy(), ig)
    np.testing.assert_array_equal(w2.cpu().numpy().view(np.uint32), wg.view(np.uint32))
    # no logits buffer (the one-kernel form, E <= 64): the same picks; above 64 experts it is required
    if wl.E <= 64:
        _, idx3, w3 = m.moe_router_topk(x, wr, wl.k, x_scales=xs, want_logits=False)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx3.cpu().numpy(), ig)
        np.testing.assert_array_equal(w3.cpu().numpy().view(np.uint32), wg.view(np.uint32))
    else:
        with pytest.raises(ValueError):
            m.moe_router_topk(x, wr, wl.k, x_scales=xs, want_logits=False)
    # a token's logits do not depend on T or on its position: the last rows alone give the same bits
    if wl.T > 9:
        s = wl.T - 9
        lg4, _, _ = m.moe_router_topk(x[s:], wr, wl.k, x_scales=None if xs is None else xs[s:])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(lg4.cpu().numpy().view(np.uint32), lg[s:].view(np.uint32))


def test_router_unaligned_router_matrix_and_zero_tokens():
    """W_r at a 4-byte (not 16-byte) offset takes the element-wise load path; T = 0 launches nothing."""
    m = lib()
    inp = _synthetic("f32_unaligned", 90, 256, 8, 2, "f32", 2006)
    x = torch.from_numpy(inp.x).cuda()
    buf = torch.zeros(inp.w_router.size + 1, dtype=torch.float32, device="cuda")
    buf[1:] = torch.from_numpy(inp.w_router.reshape(-1)).cuda()
    wr = buf[1:].view(inp.w_router.shape)
    assert wr.data_ptr() % 16 == 4
    logits, idx, w = m.moe_router_topk(x, wr, 2)
    torch.cuda.synchronize()
    _check_router(inp, logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), "unaligned W_r")
    lg0, i0, w0 = m.moe_router_topk(x[:0], wr, 2)
    torch.cuda.synchronize()
    assert lg0.shape == (0, 8) and i0.shape == (0, 2) and w0.shape == (0, 2)


def test_router_routes_the_mixtral_layer_like_its_host_logits():
    """The full layer on the mixtral shape, routed on the GPU from x W_r: the picks equal the host-logit picks
    except at near-ties, and the dispatch built from the GPU picks matches the oracle's on them."""
    m = lib()
    inp = CASES["mixtral_bf16"]()
    wl = inp.wl
    x = _dev(inp.x, wl.dtype)
    wr = torch.from_numpy(inp.w_router).cuda()
    _, idx, w = m.moe_router_topk(x, wr, wl.k, want_logits=False)
    disp = m.moe_dispatch_permute(x, idx, wl.E, gather=False)
    torch.cuda.synchronize()
    ig = idx.cpu().numpy()
    counts, offsets, rop, tor = oracle.dispatch(ig, wl.E)
    np.testing.assert_array_equal(disp.counts.cpu().numpy(), counts)
    np.testing.assert_array_equal(disp.row_of_pair.cpu().numpy(), rop)
    np.testing.assert_array_equal(disp.token_of_row.cpu().numpy(), tor)
    hidx, _ = oracle.route_topk(inp.logits, wl.k)
    frac = float(np.mean(np.any(hidx != ig, axis=1)))
    print(f"mixtral: {frac:.2e} of tokens routed differently from the host logits")
    assert frac < 1e-2
