"""The layer captured in one HIP graph: no entry point synchronises, reads device memory on the host or records a
memset, so a whole layer (and a training step) can be captured once and replayed.

Each graph is replayed several times with eager work of the program and synchronisations between the replays, and
every replay must reproduce the eager result bit for bit (the kernels have no atomics and a fixed order)."""
import numpy as np
import pytest
import torch

import moe_inputs

pytestmark = pytest.mark.gpu


def lib():
    import grouped_expert_ffn_router_amd as m

    return m


def _dev(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _layer(inp, form="permuted", train=False):
    m = lib()
    wl = inp.wl
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[wl.dtype]
    sc = [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
          for a in (inp.s_gate, inp.s_up, inp.s_down)]
    return m.MoELayer(wl.T, wl.H, wl.E, wl.k, wl.F, tdt, *(_dev(a, wl.dtype) for a in (inp.w_gate, inp.w_up,
                                                                                    inp.w_down)),
                      *sc, form=form, train=train)


def _capture_and_check(run, outputs, replays=4):
    """run(): enqueue the work on the current stream; outputs(): tensors to compare."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on the capture stream (lazy initialisations happen outside the graph)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    for t in outputs():
        t.fill_(0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 22, device="cuda")
    for i in range(replays):
        for t in outputs():  # eager work between replays: clobber the outputs
            t.fill_(float(i + 1))
        scratch.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs(), ref):
            assert torch.equal(a, b), f"replay {i} differs from the eager result"
    return ref


@pytest.mark.parametrize("name,form", [("mixtral_bf16", "permuted"), ("dsv3_fp8", "gather"), ("skewed_bf16", "fused"),
                                       ("decode_bf16", "permuted")])
def test_layer_forward_in_one_graph(name, form):
    wl = moe_inputs.get(name)
    if wl.T * wl.H > 16384 * 4096 // 2:  # keep the weights' host generation short: half the tokens
        wl = wl.replace(T=wl.T // 2)
    inp = moe_inputs.make_inputs(wl)
    layer = _layer(inp, form=form)
    logits = torch.from_numpy(inp.logits).cuda()
    x = _dev(inp.x, wl.dtype)
    xs = None if inp.x_scales is None else torch.from_numpy(inp.x_scales).cuda()
    print(f"case {name} form={form}", flush=True)
    _capture_and_check(lambda: layer.forward(logits, x, xs),
                       lambda: [layer.out, layer.topk_idx, layer.topk_w, layer.disp.row_of_pair])


def test_training_step_in_one_graph():
    m = lib()
    wl = moe_inputs.Workload("graph_train", T=512, H=512, E=4, k=2, F=512, dtype="bf16", logits="zipf", seed=77)
    inp = moe_inputs.make_inputs(wl)
    layer = _layer(inp, train=True)
    logits = torch.from_numpy(inp.logits).cuda()
    x = _dev(inp.x, wl.dtype)
    dout = torch.randn((wl.T, wl.H), device="cuda").to(torch.bfloat16)

    def step():
        layer.route(logits)
        layer.dispatch(x)
        layer.forward_train()
        layer.combine()
        layer.backward(dout)

    _capture_and_check(step, lambda: [layer.out, layer.grads["dx"], layer.grads["dw_gate"], layer.grads["dw_down"],
                                      layer.grads["d_topk_w"], layer.grads["d_logits"]])


def test_router_in_one_graph():
    m = lib()
    inp = moe_inputs.make_inputs(moe_inputs.get("mixtral_bf16"), with_weights=False)
    wl = inp.wl
    x = _dev(inp.x, wl.dtype)
    wr = torch.from_numpy(inp.w_router).cuda()
    lg = torch.empty((wl.T, wl.E), device="cuda")
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), device="cuda")
    _capture_and_check(lambda: m.moe_router_topk(x, wr, wl.k, logits=lg, topk_idx=idx, topk_w=w),
                       lambda: [lg, idx, w])
