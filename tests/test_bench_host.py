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


def test_traffic_record_follows_the_kernel_and_its_sources(tmp_path, monkeypatch):
    current = bench.kernel_source_hash("qk_pipe_kernel")
    assert len(current) == 16 and current != bench.kernel_source_hash("qk_kernel")
    rec = {"kernel_family": "qk_pipe_kernel", "kernel_source_hash": current,
           "hbm_bytes_per_launch": 123.0}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_some_workload.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda fam: current)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    val, note = bench.measured_traffic("some_workload", "qk_pipe_kernel (rmsnorm_mrope_qk)")
    assert val == 123.0 and current in note and "L2<->fabric" in note
    # another kernel launched this run: the record does not apply
    assert bench.measured_traffic("some_workload", "qk_kernel")[0] is None
    rec["kernel_source_hash"] = "0" * 16            # counters taken on other sources
    (prof / "traffic_some_workload.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("some_workload", "qk_pipe_kernel")[0] is None
    assert bench.measured_traffic("no_record", "qk_pipe_kernel")[0] is None


def test_committed_traffic_records_name_their_commands_and_kernel():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        if name.startswith("traffic_") and name.endswith(".json"):
            rec = json.load(open(os.path.join(ROOT, "profiles", name)))
            assert rec["commands"] and all("rocprofv3 --pmc" in c or "bench.py" in c
                                           for c in rec["commands"])
            assert len(rec["kernel_source_hash"]) == 16
            assert rec["kernel_family"] in bench.KERNEL_SOURCES


@pytest.mark.parametrize("procs", [1, 2])
def test_cpu_baseline_record(procs):
    wl = W.WORKLOADS["tiny_mrope"]
    inp = W.make_inputs(wl)
    r = bench.cpu_baseline(inp, wl, budget_s=0.3, procs=procs)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert r["cores"] == procs
    assert r["cores_visible"] == len(os.sched_getaffinity(0))
    assert "1024-token chunks" in r["sample"] or "16-token chunks" in r["sample"]
    if procs > 1:
        assert r["one_thread"] > 0


@pytest.mark.parametrize("S_", [0, 4])
def test_trace_summary_splits_the_phases(tmp_path, S_):
    """The summary picks the dispatches of each phase in launch order: copy
    (settle + W + K), then the kernel rotating (settle + W + K) and on one
    set (settle + W + K); the settle count comes from the dispatch count."""
    W_, K_ = 2, 3
    CW, CK = bench.copy_counts(W_, K_)
    rows = []
    t = 1000
    names = ["void mrope::(anonymous namespace)::stream_copy_kernel(char const*, char*, "
             "unsigned long)"] * (S_ + CW + CK) + ["__amd_rocclr_fillBufferAligned"] + \
            ["void mrope::(anonymous namespace)::qk_kernel<true, 8, 0, true, 8, 0>(...)"] * \
            (2 * (S_ + W_ + K_))
    durs = [70] * S_ + [50] * CW + [40] * CK + [7] + [130] * S_ + [120] * W_ + [100] * K_ + \
        [125] * S_ + [110] * W_ + [90] * K_
    for i, (n, d) in enumerate(zip(names, durs)):
        rows.append({"Kernel_Name": n, "Start_Timestamp": str(t), "End_Timestamp": str(t + d * 1000)})
        t += d * 1000 + 500
    sub = tmp_path / "host" / "1"
    sub.mkdir(parents=True)
    with open(sub / "x_kernel_trace.csv", "w") as f:
        f.write("Kind,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for r in rows[::-1]:      # out of order on purpose: sorted by start time
            name, t0, t1 = r["Kernel_Name"], r["Start_Timestamp"], r["End_Timestamp"]
            f.write(f'KERNEL_DISPATCH,"{name}",{t0},{t1}\n')
    out = bench.summarize_trace(str(tmp_path), W_, K_)
    got = {(p["phase"], "copy" if "copy" in p["kernel"] else "kernel"): p for p in out["phases"]}
    assert got[("timed_rotating", "copy")]["mean_us"] == 40.0
    assert got[("timed_rotating", "kernel")]["mean_us"] == 100.0
    assert got[("timed_same_buffers", "kernel")]["mean_us"] == 90.0
    assert got[("timed_rotating", "kernel")]["dispatches"] == K_
    assert out["settle"] == S_
    if S_:
        assert got[("settle", "copy")]["mean_us"] == 70.0
        assert got[("settle_rotating", "kernel")]["mean_us"] == 130.0
        assert got[("settle_same_buffers", "kernel")]["dispatches"] == S_
    assert "unmatched" not in out


def test_settle_count_spans_about_200_ms():
    """About 200 ms of GPU time at 6 TB/s, whatever the step's size, within
    20 and 5000 steps."""
    for b in (6_336, 184_684_544, 453_246_976, 604_373_504, 906_231_808):
        n = bench.settle_count(b)
        assert 20 <= n <= 5000
        if 20 < n < 5000:
            assert 0.19 <= n * b / 6e12 <= 0.21


def test_trace_summary_cold_run(tmp_path):
    """A --cold run launches the kernel W + K times, each after a flush kernel
    the summary does not count."""
    W_, K_ = 2, 3
    rows, t = [], 1000
    for i in range(W_ + K_):
        for n, d in (("reduce_kernel<float>(...)", 300),
                     ("void mrope::(anonymous namespace)::qk_pipe_kernel<true, 8, true, 8, 0, 0>"
                      "(...)", 100 + (20 if i < W_ else i))):
            rows.append((n, t, t + d * 1000))
            t += d * 1000 + 500
    sub = tmp_path / "h"
    sub.mkdir()
    with open(sub / "x_kernel_trace.csv", "w") as f:
        f.write("Kind,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for n, t0, t1 in rows:
            f.write(f'KERNEL_DISPATCH,"{n}",{t0},{t1}\n')
    out = bench.summarize_trace(str(tmp_path), W_, K_, cold=True)
    got = {p["phase"]: p for p in out["phases"]}
    assert got["warmup"]["mean_us"] == 120.0
    assert got["timed_cold"]["dispatches"] == K_
    assert got["timed_cold"]["mean_us"] == 100 + (2 + 3 + 4) / 3
    assert "unmatched" not in out


def test_warmup_and_steps_are_exact(monkeypatch):
    """time_region runs exactly W untimed and K timed steps, cycling the sets."""
    calls = []

    class Ev:
        def __init__(self, **kw):
            pass

        def record(self, s=None):
            calls.append("ev")

        def elapsed_time(self, other):
            return 1.0

    class FakeCuda:
        Event = Ev

        @staticmethod
        def current_stream():
            return None

        @staticmethod
        def synchronize():
            pass

    import torch
    monkeypatch.setattr(torch, "cuda", FakeCuda)
    fns = [lambda i=i: calls.append(i) for i in range(3)]
    ms, _ = bench.time_region(fns, 4, 5)
    assert calls == [0, 1, 2, 0, "ev", 0, 1, 2, 0, 1, "ev"]
    assert ms == 1.0 / 5


def test_traffic_record_scales_each_counter_by_the_runs_copy(tmp_path):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the rotary kernel,
    scaled by what the same counter reads for the run's own copy phase."""
    wl = W.WORKLOADS["omni_text_prefill"]
    copy_bytes = wl.T * (wl.hq + wl.hk) * wl.D * 2
    kern = "void mrope::(anonymous namespace)::qk_pipe_kernel<true, 8, true, 8, 0, 2>(...)"
    copy = "void mrope::(anonymous namespace)::stream_copy_kernel(char const*, char*, ...)"

    def write(d, ctr, kern_kib, copy_kib):
        d.mkdir(parents=True)
        with open(d / "x_counter_collection.csv", "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            i = 0
            for name, kib in ((copy, copy_kib), (kern, kern_kib)):
                for _ in range(5):
                    i += 1
                    f.write(f'{i},"{name}",{ctr},{kib}\n')
            f.write(f'{i + 1},"__amd_rocclr_fillBufferAligned",{ctr},7\n')
    # fetch counter reads half the bytes (scale 2), write counter reads them all
    write(tmp_path / "f", "FETCH_SIZE", copy_bytes / 2048 * 1.01, copy_bytes / 2048)
    write(tmp_path / "w", "WRITE_SIZE", copy_bytes / 1024, copy_bytes / 1024)
    rec = bench.traffic_record(str(tmp_path / "f"), str(tmp_path / "w"), "omni_text_prefill")
    assert rec["kernel_family"] == "qk_pipe_kernel" and rec["kernel_dispatches"] == [5, 5]
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12 and abs(rec["write_scale"] - 1.0) < 1e-12
    assert abs(rec["hbm_read_bytes_per_launch"] - 1.01 * copy_bytes) < 1
    assert abs(rec["hbm_write_bytes_per_launch"] - copy_bytes) < 1
    assert rec["algorithmic_bytes_per_launch"] == wl.algorithmic_bytes()


def test_rotation_spans_four_times_the_mall():
    """The default rotation cycles through enough buffer sets (inputs and
    outputs of the fused call) to span 1 GiB; an explicit --rotate wins."""
    def per_set(name):
        wl = W.WORKLOADS[name]
        return 2 * wl.T * (wl.hq + wl.hk) * wl.D * (2 if wl.dtype == "bf16" else 4)
    for name in ("omni_text_prefill", "qwen35_partial_mixed", "chunked_video", "vision_2d"):
        n = bench.rotation_sets(0, per_set(name))
        assert n >= 3 and n * per_set(name) >= bench.ROTATION_SPAN
        assert n == 3 or (n - 1) * per_set(name) < bench.ROTATION_SPAN
    assert bench.rotation_sets(0, per_set("omni_text_prefill")) == 3
    assert bench.rotation_sets(0, per_set("chunked_video")) == 6
    assert bench.rotation_sets(5, per_set("chunked_video")) == 5
    assert bench.rotation_sets(0, 1) == bench.ROTATION_MAX_SETS == 16
