"""Host-side pieces of bench.py that need no GPU: the one-GPU guard, the
traffic record's source check, and the CPU oracle baseline's record."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_follows_the_kernel_source(tmp_path, monkeypatch):
    current = bench.kernel_source_hash()
    assert len(current) == 16
    rec = {"kernel_source_hash": current, "hbm_bytes_per_launch": 123.0}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_some_workload.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: current)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("some_workload") == 123.0
    rec["kernel_source_hash"] = "0" * 16            # counters taken on other sources
    (prof / "traffic_some_workload.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("some_workload") is None
    assert bench.measured_traffic("no_record") is None


def test_committed_traffic_records_name_their_commands():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        if name.startswith("traffic_") and name.endswith(".json"):
            rec = json.load(open(os.path.join(ROOT, "profiles", name)))
            assert rec["commands"] and all("rocprofv3 --pmc" in c for c in rec["commands"])
            assert len(rec["kernel_source_hash"]) == 16


@pytest.mark.parametrize("procs", [1, 2])
def test_cpu_baseline_record(procs):
    wl = W.WORKLOADS["tiny_mrope"]
    inp = W.make_inputs(wl)
    r = bench.cpu_baseline(inp, wl, budget_s=0.3, procs=procs)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert r["cores"] == procs
    if procs > 1:
        assert r["one_thread"] > 0
