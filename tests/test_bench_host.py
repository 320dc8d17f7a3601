"""Host logic of bench.py (no GPU): the one-GPU guard, the roofline object, the
per-kernel statistics, and the rule that a counter measurement of HBM traffic is
reported only for the kernel source it was taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line for an unsupported count


def test_roofline_object():
    # 5.4989e11 flop in 0.5 ms is 1099.78 TFLOP/s, 0.4399 of 2.5 PF
    r = bench.roofline("prefill_bf16_kernel", "prefill_bf16_kernel<128>", "no-such-workload",
                       "mfma", 549890031616.0, 0.5)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(1099.78, abs=0.01)
    assert r["frac"] == pytest.approx(0.4399, abs=1e-4)
    assert r["traffic"] is None                 # nothing measured for that workload
    # 4,296,016,192 B in 0.65 ms is 6609.3 GB/s, 0.8262 of 8 TB/s
    r = bench.roofline("decode_split_kernel", "decode_split_kernel<bf16,128>", "x", "hbm",
                       4296016192, 0.65)
    assert r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(6609.26, abs=0.01)
    assert r["frac"] == pytest.approx(0.8262, abs=1e-4)


def test_stats_and_median():
    assert bench._median([3.0, 1.0, 2.0]) == 2.0
    assert bench._median([4.0, 1.0, 2.0, 3.0]) == 2.5
    s = bench.stats([1.0, 2.0, 4.0])
    assert s == {"median": 2.0, "mean": round(7 / 3, 4), "min": 1.0, "max": 4.0,
                 "spread": 1.5, "n": 3}


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    key = "prefill_bf16_kernel@some_workload"
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({key: {"src_sha": bench.src_sha("prefill_bf16_kernel"),
                                      "hbm_bytes_per_launch": 1234}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic("prefill_bf16_kernel", "some_workload") == 1234
    assert bench.traffic("prefill_bf16_kernel", "other_workload") is None
    # a measurement taken on another version of the kernel source is not reported
    path.write_text(json.dumps({key: {"src_sha": "0" * 16, "hbm_bytes_per_launch": 1234}}))
    assert bench.traffic("prefill_bf16_kernel", "some_workload") is None
    # nor is anything when the file is missing or unreadable
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic("prefill_bf16_kernel", "some_workload") is None


def test_committed_traffic_matches_committed_sources():
    """Every entry of profiles/traffic.json names a kernel bench.py knows and a
    source hash; the entries for the current sources are what bench.py reports."""
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t
    for key, v in t.items():
        kernel, workload = key.split("@", 1)
        assert kernel in bench.KERNEL_SOURCES
        assert len(v["src_sha"]) == 16
        assert v["hbm_bytes_per_launch"] > 0
        if v["src_sha"] == bench.src_sha(kernel):
            assert bench.traffic(kernel, workload) == v["hbm_bytes_per_launch"]
