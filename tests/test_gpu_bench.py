"""bench.py's output contract on a real GPU, on the tiny fp32 workload (seconds per run): one JSON line with the
metric, the whole-job throughput, the roofline object of the dominant kernel and the CPU oracle baseline, for the
default form and for the gather, graph-replay, router and training options."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
METRIC = "MoE-layer tokens/s on 1 MI355X; permute/combine GB/s and grouped-GEMM MFMA %"
TRAIN_METRIC = "MoE-layer training tokens/s on 1 MI355X (forward keeping activations + backward)"


def _bench(*args):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_fp32", "--steps", "3", "--warmup",
           "1", "--hbm-copy", "0", *args]
    print("running", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def _common(d, steps=3, warmup=1, metric=METRIC):
    assert d["metric"] == metric and d["unit"] == "tokens/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - 256 / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]  # T tokens per step
    assert d["scaling"] == "weak" and d["vs_baseline"] is None and d["data"] == "synthetic"
    assert d["dtype"] == "f32" and d["config"]["workload"] == "tiny_fp32"
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 157.3
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    assert "traffic" in rf
    dev = d["device"]
    assert dev["compute_units"] > 0 and dev["memory_GiB"] > 0 and isinstance(dev["name"], str)


def test_default_line_with_the_cpu_baseline():
    d = _bench("--cpu-tokens", "32")
    _common(d)
    assert d["config"]["path"] == "permuted" and d["config"]["launch"] == "eager"
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert isinstance(cb["sample"], str) and cb["sample"]
    # the oracle's parts timed separately: route and permutation over every token, FFN + combine on the sample
    assert set(cb["parts"]) == {"route", "permutation", "ffn_combine"}
    assert all(p["tokens_per_s"] > 0 and p["seconds"] >= 0 for p in cb["parts"].values())
    assert cb["parts"]["route"]["tokens"] == 256 and cb["parts"]["ffn_combine"]["tokens"] == 32
    k = d["kernels"]
    for name in ("route_us", "dispatch_us", "ffn_gate_up_us", "ffn_down_us", "combine_us", "dispatch_GBs",
                 "combine_GBs", "ms_per_step_evented_pass"):
        assert k[name] > 0, name


@pytest.mark.parametrize("opts,path,launch", [(("--fused", "2", "--graph", "1"), "gather", "graph replay"),
                                              (("--fused", "1"), "fused", "eager"),
                                              (("--router", "1"), "permuted", "eager")])
def test_layer_options(opts, path, launch):
    d = _bench("--cpu-baseline", "0", *opts)
    _common(d)
    assert "cpu_baseline" not in d
    assert d["config"]["path"] == path and d["config"]["launch"] == launch
    if "--router" in opts:
        assert d["config"]["route_from"] == "x W_r"


def test_training_step_line():
    d = _bench("--cpu-baseline", "0", "--train", "1")
    _common(d, metric=TRAIN_METRIC)
    assert d["config"]["path"] == "train"
    assert d["kernels"]["backward_us"] > 0 and d["kernels"]["ffn_train_us"] > 0
