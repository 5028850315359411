#!/usr/bin/env python3
"""Tokens/s of one MoE layer on one MI355X: route, dispatch-permute, grouped SwiGLU FFN, combine.

A step is one pass of the whole layer over one batch of seeded synthetic inputs already resident in HBM.
Default workload: the DeepSeek-V3-shaped fp8 prefill on one GPU's share (T=8192 tokens, H=7168, 32 local experts,
top-8, F=2048; fp8 e4m3 activations and weights with fp32 block scales, bf16 output), the largest single-GPU
configuration; --workload selects the others (mixtral_bf16, skewed_bf16, decode_bf16, tiny_fp32).

Prints one JSON line with the layer throughput (K steps back to back, nothing recorded between the kernels), the
roofline of the dominant kernel (the gate/up grouped GEMM, against dense bf16 / fp8 MFMA peak), per-kernel
timings from HIP events recorded on the launch stream in a second pass of the same K steps, and the CPU oracle
timed on a bounded token sample on the host cores.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}  # dense MFMA (fp32: matrix fp32)
PEAK_HBM_GBS = 8000.0
METRIC = "MoE-layer tokens/s on 1 MI355X; permute/combine GB/s and grouped-GEMM MFMA %"
FORMS = ("permuted", "fused", "gather")  # --fused 0 / 1 / 2


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3_fp8")
    ap.add_argument("--cpu-baseline", type=int, default=1, help="0 skips the CPU oracle timing")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle token sample (0: sized for ~15 s)")
    ap.add_argument("--fused", type=int, default=0, choices=(0, 1, 2),
                    help="0: the permuted form (x_perm written by the dispatch); 1: the fused form (gather inside "
                         "the gate/up product, weighted pair-major slots); 2: the gather form (gather inside the "
                         "gate/up product, then the permuted down product and combine)")
    ap.add_argument("--router", type=int, default=0,
                    help="1: route from x W_r on the GPU (router GEMM fused with the top-k) instead of from the "
                         "stored logits; workloads whose logits are defined as x W_r only")
    ap.add_argument("--train", type=int, default=0,
                    help="1: a training step (forward keeping its activations, combine, then the backward pass for "
                         "a fixed synthetic dout); fp32 / bf16 workloads")
    ap.add_argument("--flush", type=int, default=0,
                    help="1: write a 1 GiB buffer before every step so each step starts with cold L2 and MALL; the "
                         "step time then comes from the HIP events around the step, not the wall clock")
    ap.add_argument("--graph", type=int, default=0,
                    help="1: capture one step in a HIP graph and time K replays of it (per-kernel times still come "
                         "from an evented eager pass)")
    ap.add_argument("--hbm-copy", type=int, default=1,
                    help="1: after the timed steps, time 1 GiB device copies (measured HBM bandwidth)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this library runs one GPU's share of the layer; --gpus {args.gpus} (WORLD_SIZE {world}) "
              "is not supported: run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import grouped_expert_ffn_router_amd as m
    import moe_inputs

    wl = moe_inputs.get(args.workload)
    dev = torch.device("cuda:0")
    inp = moe_inputs.make_inputs(wl)

    def up(a):
        a = np.ascontiguousarray(a)
        if wl.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[wl.dtype]
    x = up(inp.x)
    xs = None if inp.x_scales is None else torch.from_numpy(inp.x_scales).to(dev)
    logits = torch.from_numpy(inp.logits).to(dev)
    if args.router and inp.w_router is None:
        print(f"bench.py: --router 1 needs a workload whose logits are x W_r ({wl.name} has none)", file=sys.stderr)
        sys.exit(2)
    w_router = None if inp.w_router is None else torch.from_numpy(inp.w_router).to(dev)
    sc = [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
          for a in (inp.s_gate, inp.s_up, inp.s_down)]
    if args.train and (wl.dtype == "fp8" or args.fused):
        print("bench.py: --train 1 needs an fp32 / bf16 workload and the permuted form", file=sys.stderr)
        sys.exit(2)
    layer = m.MoELayer(wl.T, wl.H, wl.E, wl.k, wl.F, tdt, up(inp.w_gate), up(inp.w_up), up(inp.w_down), *sc,
                       e_lo=wl.e_lo, device=dev, form=FORMS[args.fused], train=bool(args.train))
    dout = None
    if args.train:
        g = torch.Generator(device="cpu").manual_seed(wl.seed + 1)
        dout = torch.randn((wl.T, wl.H), generator=g).to(tdt).to(dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    names = ["route", "dispatch", "ffn_gate_up", "ffn_down", "combine"]
    if args.train:
        names = ["route", "dispatch", "ffn_train", "combine", "backward"]

    def train_step(ev=None, st=None):
        stream_ = st or stream
        layer.route(logits, stream_)
        if ev: ev[1].record(stream_)
        layer.dispatch(x, xs, stream_)
        if ev: ev[2].record(stream_)
        layer.forward_train(stream_)
        if ev: ev[3].record(stream_)
        layer.combine(stream_)
        if ev: ev[4].record(stream_)
        layer.backward(dout, stream_)
        if ev: ev[5].record(stream_)

    def step(ev=None, st=None):
        stream_ = st or stream
        if args.train:
            return train_step(ev, st)
        if args.router:
            layer.route_x(x, w_router, xs, stream_)
        else:
            layer.route(logits, stream_)
        if ev: ev[1].record(stream_)
        layer.dispatch(x, xs, stream_)
        if ev: ev[2].record(stream_)
        layer.gate_up(stream_)
        if ev: ev[3].record(stream_)
        layer.down(stream_)
        if ev: ev[4].record(stream_)
        layer.combine(stream_)
        if ev: ev[5].record(stream_)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    flushbuf = torch.empty(1 << 28, dtype=torch.float32, device=dev) if args.flush else None
    elapsed = None
    if flushbuf is None:
        # the step time: K steps back to back with nothing recorded between the launches, so the figure is the
        # layer's own (the evented pass below reports its step time as well, for comparison)
        run = step
        if args.graph:
            # one step captured once (on a side stream, after the warm-up) and replayed: the launches become
            # graph nodes, so the host's per-launch work leaves the step
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step(st=side)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                step(st=torch.cuda.current_stream())
            torch.cuda.synchronize()
            for _ in range(3):
                g.replay()
            run = g.replay
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            run()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    # per-kernel times: the same K steps again, with an event after every launch on the launch stream
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        if flushbuf is not None:
            flushbuf.fill_(float(i))  # 1 GiB written: evicts the 4 MB L2s and the 256 MB MALL
        evs[i][0].record(stream)
        step(evs[i])
    torch.cuda.synchronize()
    elapsed_events = time.perf_counter() - t1
    if flushbuf is not None:
        # the wall clock includes the flushes: the step time is the events' first-to-last span instead
        elapsed = sum(evs[i][0].elapsed_time(evs[i][5]) for i in range(args.steps)) * 1e-3
        del flushbuf

    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    hbm_copy = None
    if args.hbm_copy:
        # a plain 1 GiB device-to-device copy: read + written bytes over its duration (median of 5)
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        times = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        hbm_copy = 2.0 * n / float(np.median(times[1:])) / 1e9
        del src, dst

    ms_per_step = elapsed * 1e3 / args.steps
    samples = {n: np.array([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]) * 1e3
               for j, n in enumerate(names)}  # microseconds per step
    per = {n: float(np.mean(v)) for n, v in samples.items()}
    spread = {n: {"median": float(np.median(v)), "p10": float(np.percentile(v, 10)),
                  "p90": float(np.percentile(v, 90))} for n, v in samples.items()}
    T, H, k, F = wl.T, wl.H, wl.k, wl.F
    R = T * k
    if args.train:
        return report_train(args, wl, inp, per, spread, elapsed, ms_per_step, hbm_copy, elapsed_events)
    b = moe_inputs.ELEM_BYTES[wl.dtype]
    bout = 4 if wl.dtype == "f32" else 2
    nsc = (H // 128) * 4 if wl.dtype == "fp8" else 0
    flops_gate_up = 4.0 * R * H * F
    flops_down = 2.0 * R * F * H
    # the fused and gather forms' dispatch writes only the permutation (T*k pairs: 4 B read, 8 B written)
    bytes_dispatch = R * 12 if args.fused else T * (H * b + nsc) + R * (H * b + nsc)
    bytes_combine = R * (H * 4 + 12) + T * H * bout
    # routing reads the logits (or x and W_r) and writes the picks
    bytes_route = (T * (H * b + nsc) + H * wl.E * 4 if args.router else T * wl.E * 4) + R * 8
    peak = PEAK_TFLOPS[wl.dtype]
    ach = flops_gate_up / (per["ffn_gate_up"] * 1e-6) / 1e12
    kernels = {
        "route_us": per["route"],
        "route_GBs": bytes_route / (per["route"] * 1e-6) / 1e9,
        "dispatch_us": per["dispatch"],
        "dispatch_GBs": bytes_dispatch / (per["dispatch"] * 1e-6) / 1e9,
        "ffn_gate_up_us": per["ffn_gate_up"],
        "ffn_gate_up_TFLOPs": ach,
        "ffn_down_us": per["ffn_down"],
        "ffn_down_TFLOPs": flops_down / (per["ffn_down"] * 1e-6) / 1e12,
        "combine_us": per["combine"],
        "combine_GBs": bytes_combine / (per["combine"] * 1e-6) / 1e9,
        "layer_us_events": sum(per.values()),
        "ms_per_step_evented_pass": elapsed_events * 1e3 / args.steps,
        "weights_GBs": 3.0 * wl.n_local * H * F * b / ((per["ffn_gate_up"] + per["ffn_down"]) * 1e-6) / 1e9,
        "us_median_p10_p90": spread,
    }
    for name in ("dispatch", "combine"):
        kernels[name + "_frac_of_8TBs"] = kernels[name + "_GBs"] / PEAK_HBM_GBS
        if hbm_copy:
            kernels[name + "_frac_of_copy"] = kernels[name + "_GBs"] / hbm_copy
    res = {
        "metric": METRIC,
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "H": H, "E": wl.E, "k": k, "F": F, "E_local": wl.n_local,
                   "path": FORMS[args.fused], "route_from": "x W_r" if args.router else "logits",
                   "caches": "flushed before every step (event-timed steps)" if args.flush else "warm",
                   "launch": "graph replay" if args.graph and not args.flush else "eager"},
        "roofline": {
            "bound": "mfma",
            "kernel": "grouped_gemm_kernel (gate/up + SwiGLU)",
            "achieved": ach,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": ach / peak,
            "traffic": None if args.fused else measured_traffic(wl.name),
            "algorithmic_flops_per_launch": flops_gate_up,
        },
        "kernels": kernels,
        "hbm_copy_GBs": hbm_copy,
        "device": device_facts(),
    }
    if args.cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_tokens)
    print(json.dumps(res))


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
KERNEL_SOURCES = ["grouped_expert_ffn_router_amd/csrc/ffn.hip", "grouped_expert_ffn_router_amd/csrc/gemm_tile.h",
                  "grouped_expert_ffn_router_amd/csrc/common.h"]


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def device_facts():
    """What the runtime reports for device 0 (name, architecture, compute units, memory) and rocminfo's peak
    engine clock of the first GPU agent (None if rocminfo is not available)."""
    import torch

    p = torch.cuda.get_device_properties(0)
    facts = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
             "memory_GiB": round(p.total_memory / 2**30, 1)}
    facts["max_clock_MHz"] = None
    import subprocess

    try:  # rocminfo's peak engine clock of the first gfx agent
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        gpu = False
        for line in out.splitlines():
            if "Name:" in line and "gfx" in line:
                gpu = True
            if gpu and "Max Clock Freq. (MHz):" in line:
                facts["max_clock_MHz"] = int(line.split(":")[1].split()[0])
                break
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    return facts


def measured_traffic(workload):
    """HBM bytes per launch of the gate/up grouped GEMM, from rocprofv3 FETCH_SIZE and WRITE_SIZE counters
    scaled by a plain copy's readings; None when the kernel sources changed after the counters were taken, or
    when the record is not physical (its bytes over the profiled launch duration above the 8 TB/s peak)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    w = rec.get("workloads", {}).get(workload)
    if w is None or w.get("gate_up_bytes_per_launch") is None:
        return None
    us = w.get("trace_avg_us")
    if not us or w["gate_up_bytes_per_launch"] / (us * 1e-6) > 8.0e12:
        return None
    return w["gate_up_bytes_per_launch"]


def cpu_baseline(wl, inp, n_tokens):
    """The CPU oracle as it stands, on the host cores: routing and the permutation for every token, the expert
    FFN + weighted sum for a seeded token sample; reported as layer tokens/s, and per part (route, permutation,
    FFN + combine) as tokens/s of that part alone."""
    import numpy as np

    import oracle

    if n_tokens <= 0:
        # about 15 s of work, sized from a short timed probe of the same routine (the probe is not reported)
        probe = np.arange(min(wl.T, 2 * oracle.num_threads()), dtype=np.int64)
        i0, w0 = oracle.route_topk(inp.logits[: len(probe)], wl.k)
        tp = time.perf_counter()
        oracle.moe_tokens(inp, i0, w0, tokens=probe)
        per_probe = (time.perf_counter() - tp) / len(probe)
        n_tokens = int(max(8, min(wl.T, 15.0 / max(per_probe, 1e-9))))
    rng = np.random.default_rng(1234)
    toks = np.sort(rng.choice(wl.T, size=min(n_tokens, wl.T), replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    idx, w = oracle.route_topk(inp.logits, wl.k)
    t1 = time.perf_counter()
    oracle.dispatch(idx, wl.E)
    t2 = time.perf_counter()
    oracle.moe_tokens(inp, idx, w, tokens=toks)
    t3 = time.perf_counter()
    per_route, per_perm, per_ffn = (t1 - t0) / wl.T, (t2 - t1) / wl.T, (t3 - t2) / len(toks)
    per_token_s = per_route + per_perm + per_ffn
    parts = {
        "route": {"tokens_per_s": 1.0 / per_route, "seconds": t1 - t0, "tokens": wl.T},
        "permutation": {"tokens_per_s": 1.0 / per_perm, "seconds": t2 - t1, "tokens": wl.T},
        "ffn_combine": {"tokens_per_s": 1.0 / per_ffn, "seconds": t3 - t2, "tokens": int(len(toks))},
    }
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": 1.0 / per_token_s, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "parts": parts,
            "cpu_model": cpu_model, "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"routing + permutation of all {wl.T} tokens, expert FFN + combine of {len(toks)} seeded tokens "
                      f"({t3 - t2:.1f} s), scaled to the layer",
            "seconds": t3 - t0}


def report_train(args, wl, inp, per, spread, elapsed, ms_per_step, hbm_copy, elapsed_events):
    """The training-step line: tokens/s of forward + backward, the backward's MFMA rate against the dense peak."""
    T, H, k, F = wl.T, wl.H, wl.k, wl.F
    R = T * k
    flops_fwd = 6.0 * R * H * F
    flops_bwd = 12.0 * R * H * F  # dh, dX (6 R H F) and the three weight products (6 R H F)
    peak = PEAK_TFLOPS[wl.dtype]
    bwd_tf = flops_bwd / (per["backward"] * 1e-6) / 1e12
    res = {
        "metric": "MoE-layer training tokens/s on 1 MI355X (forward keeping activations + backward)",
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "H": H, "E": wl.E, "k": k, "F": F, "E_local": wl.n_local,
                   "path": "train", "launch": "graph replay" if args.graph else "eager"},
        "roofline": {
            "bound": "mfma",
            "kernel": "backward (dgrad + wgrad grouped GEMMs, transposes, gathers), whole call",
            "achieved": bwd_tf,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": bwd_tf / peak,
            "traffic": None,
            "algorithmic_flops_per_launch": flops_bwd,
        },
        "kernels": {
            "route_us": per["route"], "dispatch_us": per["dispatch"], "ffn_train_us": per["ffn_train"],
            "ffn_train_TFLOPs": flops_fwd / (per["ffn_train"] * 1e-6) / 1e12, "combine_us": per["combine"],
            "backward_us": per["backward"], "backward_TFLOPs": bwd_tf, "us_median_p10_p90": spread,
            "ms_per_step_evented_pass": elapsed_events * 1e3 / args.steps,
        },
        "hbm_copy_GBs": hbm_copy,
        "device": device_facts(),
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()

