"""moe_dispatch_permute_noalloc (the dispatch with the library's fixed scratch array instead of a workspace)
against moe_dispatch_permute on the same inputs: every output bit-exact, on calls in a row whose sizes shrink, so
a table entry left over from an earlier call would show.  The large calls take the multi-workgroup counting form,
which is the one that uses scratch memory."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _inputs(T, H, E, k, dtype, seed):
    rng = np.random.default_rng(seed)
    logits = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    xs = None
    if dtype == "fp8":
        x = torch.from_numpy(rng.integers(0, 255, size=(T, H), dtype=np.uint8)).cuda()
        x[x == 0x7F] = 0  # no NaN codes
        x[x == 0xFF] = 0
        xs = torch.from_numpy(rng.uniform(0.5, 2.0, size=(T, H // 128)).astype(np.float32)).cuda()
    else:
        x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16).cuda()
    return logits, x, xs


def _alloc(m, T, H, E, k, x, xs):
    R = T * k
    return m.Dispatch(
        counts=torch.empty(E, dtype=torch.int32, device="cuda"),
        offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
        row_of_pair=torch.empty(R, dtype=torch.int32, device="cuda"),
        token_of_row=torch.empty(R, dtype=torch.int32, device="cuda"),
        x_perm=torch.empty((R, H), dtype=x.dtype, device="cuda"),
        x_perm_scales=None if xs is None else torch.empty((R, H // 128), dtype=torch.float32, device="cuda"))


def test_noalloc_dispatch_matches_the_workspace_dispatch_on_calls_in_a_row():
    import grouped_expert_ffn_router_amd as m

    # (T, H, E, k, dtype): 65536 pairs, then 24000 pairs over 256 experts, then 20480 pairs over 32 experts (fewer
    # count tiles than the first call: the table's stride changes), then 2000 pairs (the one-workgroup form)
    cases = [(8192, 256, 32, 8, "bf16"), (3000, 256, 256, 8, "fp8"), (2560, 384, 32, 8, "bf16"),
             (500, 256, 16, 4, "bf16")]
    for i, (T, H, E, k, dt) in enumerate(cases):
        print(f"noalloc dispatch call {i}: T={T} H={H} E={E} k={k} {dt}", flush=True)
        logits, x, xs = _inputs(T, H, E, k, dt, seed=100 + i)
        idx, _ = m.moe_route_topk(logits, k)
        ref = m.moe_dispatch_permute(x, idx, E, x_scales=xs)
        got = m.moe_dispatch_permute_noalloc(x, idx, E, _alloc(m, T, H, E, k, x, xs), x_scales=xs)
        torch.cuda.synchronize()
        for name in ("counts", "offsets", "row_of_pair", "token_of_row"):
            assert torch.equal(getattr(got, name), getattr(ref, name)), (i, name)
        assert torch.equal(got.x_perm.view(torch.uint8), ref.x_perm.view(torch.uint8)), i
        if xs is not None:
            assert torch.equal(got.x_perm_scales, ref.x_perm_scales), i
        assert int(got.offsets[-1]) == T * k


def test_noalloc_dispatch_permutation_only_and_size_limit():
    import grouped_expert_ffn_router_amd as m

    T, H, E, k = 4096, 256, 64, 6
    logits, x, _ = _inputs(T, H, E, k, "bf16", seed=7)
    idx, _ = m.moe_route_topk(logits, k)
    ref = m.moe_dispatch_permute(x, idx, E, gather=False)
    out = _alloc(m, T, H, E, k, x, None)
    out.x_perm = None
    got = m.moe_dispatch_permute_noalloc(x, idx, E, out)
    torch.cuda.synchronize()
    for name in ("counts", "offsets", "row_of_pair", "token_of_row"):
        assert torch.equal(getattr(got, name), getattr(ref, name)), name
    # beyond the fixed scratch: refused on the host, nothing enqueued
    big = 1 << 18
    with pytest.raises(RuntimeError, match="more than the fixed"):
        m.moe_dispatch_permute_noalloc(x[:1].expand(big, H), idx[:1].expand(big, k).contiguous(), 256,
                                       _alloc(m, 1, H, 256, k, x, None))
