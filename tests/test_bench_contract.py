"""bench.py's command-line contract and its JSON line (the GPU case runs a short bench)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("workload", ["tiny", "fp8", "decode"])
def test_bench_line(workload):
    print(f"[gpu-case] bench.py --workload {workload}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload,
                        "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--cold-runs", "1"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "device",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 3 and line["warmup"] == 1
    assert line["value"] > 0 and line["ms_per_step"] > 0
    roof = line["roofline"]
    if workload == "decode":
        assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
        assert line["unit"] == "GB/s" and line["config"]["splits"] >= 1
    else:
        assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
        assert roof["peak"] == (5000.0 if workload == "fp8" else 2500.0)
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "workload" in line["config"]
    for p in line["per_variant"]:
        assert p["min_launch_us"] <= p["median_launch_us"] and p["cold_avg_launch_us"] > 0


def test_one_core_oracle_rate():
    """The one-core oracle timing runs on the host, one BLAS thread, tiny config first."""
    sys.path.insert(0, ROOT)
    import bench
    from exact_attention_81_amd import synth

    out = bench.cpu_baseline_one_core([synth.workload("tiny")], max_heads=1, min_seconds=0.2)
    assert [o["workload"] for o in out] == [synth.workload("tiny").label()] * 2
    for o in out:
        assert o["cores"] == 1 and o["kind"] == "oracle" and o["unit"] == "TFLOP/s"
        assert o["value"] > 0 and o["heads"] >= 1


def test_committed_profiles_follow_kernel_sources(tmp_path, monkeypatch):
    """Traffic and counter figures are reported only while the kernel sources hash to
    the value recorded with them."""
    sys.path.insert(0, ROOT)
    import bench

    variant = "single:B4_H16_Nq2048_Nkv2048_d128x128_noncausal_bf16"
    (tmp_path / "attn_fwd_single_traffic.json").write_text(json.dumps(
        {"kernel_source_sha": "abc", "hbm_bytes_per_launch": 123.0}))
    (tmp_path / "attn_fwd_single_counters.json").write_text(json.dumps(
        {"kernel_source_sha": "abc", "per_variant": {variant: {"clock_ghz": 1.9}}}))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    assert bench.committed_traffic("single") == 123.0
    assert bench.committed_counters("single", variant)["clock_ghz"] == 1.9
    assert bench.committed_counters("single", "other variant") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "def")
    assert bench.committed_traffic("single") is None
    assert bench.committed_counters("single", variant) is None
