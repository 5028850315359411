"""Host-side behaviour that needs no GPU: the benchmark refuses runs on more than one GPU before touching one."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=120)


def test_bench_refuses_more_than_one_gpu():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_bench_refuses_a_multi_rank_launch():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "4", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "WORLD_SIZE 4" in r.stderr


def test_bench_reports_counter_traffic_only_for_the_counted_sources(tmp_path, monkeypatch):
    """roofline.traffic comes from the stored counter record only while the GEMM sources hash to the counted
    build, and only if the record is physical (its bytes over the traced launch duration within 8 TB/s)."""
    import json

    sys.path.insert(0, ROOT)
    import bench

    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    rec = {"source_sha256": bench.kernel_source_hash(),
           "workloads": {"dsv3_fp8": {"gate_up_bytes_per_launch": 6.0e9, "trace_avg_us": 2300.0},
                         "decode_bf16": {"gate_up_bytes_per_launch": 3.8e9, "trace_avg_us": 317.0}}}
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic("dsv3_fp8") == 6.0e9
    assert bench.measured_traffic("decode_bf16") is None  # 12 TB/s: not a physical reading
    assert bench.measured_traffic("mixtral_bf16") is None  # not counted
    rec["source_sha256"] = "0" * 64
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic("dsv3_fp8") is None  # sources changed since the counters were taken
    f.unlink()
    assert bench.measured_traffic("dsv3_fp8") is None
