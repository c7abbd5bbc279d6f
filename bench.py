#!/usr/bin/env python3
"""Throughput of the fused RMSNorm + MRoPE hot path on one MI355X.

One step = one rmsnorm_mrope_qk call over the whole workload (cos/sin from
positions, per-head RMSNorm, rotation of every q and k head), inputs resident
in HBM.  Default workload: Omni-like text prefill, q[32768,32,128] and
k[32768,4,128] bf16, interleaved [24,20,20], theta 1e6, RMSNorm eps 1e-6.

Measures (HIP events on the stream the kernels are launched on):

* rotating (the reported value): step i works on buffer set i mod S (by
  default the fewest sets, at least 3, that span 1 GiB: 3 x 604 MB for the
  headline), launched back to back, so no step reads a line that an earlier
  step left in the 256 MB memory-side cache (MALL); the steady state of a
  stream of layers whose q/k come from HBM.  Python's garbage collector is
  off over the warm-up and timed steps.
* same_buffers: every step on one set, back to back (what the previous
  measure of this benchmark reported); workloads whose bytes fit the MALL
  are partly served from it here.
* copy_ceiling: mrope_stream_copy of the workload's bytes (the q/k bytes read
  are copied into as many bytes written), rotating over S sets the same way:
  the rate a plain copy of this size reaches under the same measure.

Order on the GPU: the copy ceiling (N settle + max(W, 50) warmup + max(K, 500)
timed copies), then the kernel rotating (N + W + K), then the kernel on one
buffer set (N + W + K); the profile summaries pick their dispatches by this
order (--trace-summary).  The N settle steps (about 200 ms of GPU time, the
same count in each phase, reported in the line) run back to back before the
requested W warm-up steps: once the load starts, the rotary kernels' steps
run up to 35% slower for some tens of milliseconds, then settle, so a short
run (W = 5, K = 20) would otherwise time that dip.

Prints one JSON line: Q+K tokens/s (value), achieved HBM bandwidth of the
kernel against the 8 TB/s peak (roofline), and the CPU oracle's rate on a
bounded sample of the same workload (cpu_baseline).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--rotate S] [--graph G] [--cold] [--cs-cache]
                  [--precision exact|dtype|fp32] [--cpu-procs P]
  python bench.py --pmc-summary DIR / --traffic-record FETCH_DIR WRITE_DIR
                  # counters of rocprofv3 --pmc runs of bench.py
  python bench.py --trace-summary DIR --workload NAME --steps K --warmup W
                  # per-phase kernel durations from a rocprofv3 kernel trace

Other workloads time the other entry points: the decode step (omni_decode),
the vision packed-qkv fusion (vision_qkv_planes[_bf16]) and the position
builder (mm_prompt_positions).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, vendor peak
DEFAULT_WORKLOAD = "omni_text_prefill"
# Device sources of each rotary kernel: a traffic record taken on a kernel
# holds only while these files are unchanged.
_CSRC = "vlm_multimodal_rotary_amd/csrc/"
KERNEL_SOURCES = {
    "qk_pipe_kernel": [_CSRC + "mrope_pipe.hip", _CSRC + "mrope_device.h",
                       _CSRC + "mrope_internal.h"],
    "qk_kernel": [_CSRC + "mrope_kernels.hip", _CSRC + "mrope_device.h",
                  _CSRC + "mrope_internal.h"],
}
KERNEL_SOURCES["stage_kernel"] = KERNEL_SOURCES["qk_kernel"]
KERNEL_SOURCES["flat_kernel"] = [_CSRC + "mrope_flat.hip", _CSRC + "mrope_device.h",
                                 _CSRC + "mrope_internal.h"]
KERNEL_SOURCES["planes_kernel"] = [_CSRC + "mrope_planes.hip", _CSRC + "mrope_device.h",
                                   _CSRC + "mrope_internal.h"]
# The machine's CPU share for one GPU: oracle worker pools stay within it
# whatever the affinity mask shows.
HOST_CORE_SHARE = 16
ORACLE_CHUNK = 1024           # tokens per oracle call (bounds its memory)


def kernel_family(name: str) -> str:
    """The rotary kernel a kernel name (or mrope_last_kernel's answer) names."""
    for k in ("qk_pipe_kernel", "qk_kernel", "flat_kernel", "stage_kernel", "planes_kernel"):
        if k in name:
            return k
    return ""


def kernel_source_hash(family: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """(bytes per launch, source note) from the committed rocprofv3 counter
    summary, or (None, reason) when there is none, it was taken on another
    kernel than `kernel` (the one this run launched), or that kernel's sources
    changed since.  The counters (FETCH_SIZE + WRITE_SIZE) count bytes between
    L2 and the memory fabric; lines served by the MALL are included."""
    rel = os.path.join("profiles", f"traffic_{workload}.json")
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None, f"no {rel}"
    with open(path) as f:
        rec = json.load(f)
    fam = kernel_family(kernel)
    if not fam or rec.get("kernel_family") != fam:
        return None, f"{rel} was taken on another kernel"
    h = kernel_source_hash(fam)
    if rec.get("kernel_source_hash") != h:
        return None, f"{rel} was taken on other kernel sources"
    return rec.get("hbm_bytes_per_launch"), (
        f"L2<->fabric bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy) from "
        f"{rel}, kernel source hash {h}; not measured in this run")


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def _oracle_chunks(q, k, pos, wl, wq, wk, precision, chunk):
    """Runs the oracle over consecutive chunks of the given tokens; returns
    the token count."""
    from oracle import mrope_oracle as O
    n = q.shape[0]
    for a in range(0, n, chunk):
        sl = slice(a, min(n, a + chunk))
        O.rmsnorm_mrope_qk(q[sl], k[sl], pos[:, sl], rotary_dim=wl.rotary_dim, theta=wl.theta,
                           section=wl.section, layout=wl.layout, wq=wq, wk=wk, eps=wl.eps,
                           dtype=wl.dtype, precision=precision)
    return n


def _oracle_worker(job):
    """One process of the multi-process oracle sample: from a common start
    time, walks its share of the workload chunk after chunk (starting over
    if time remains) until the deadline.  Returns (tokens done, seconds)."""
    q, k, pos, wl, wq, wk, precision, chunk, t_start, budget_s = job
    now = time.time()
    if now < t_start:
        time.sleep(t_start - now)
    start = time.perf_counter()
    done, a, n = 0, 0, q.shape[0]
    while True:
        sl = slice(a, min(n, a + chunk))
        done += _oracle_chunks(q[sl], k[sl], pos[:, sl], wl, wq, wk, precision, chunk)
        a = a + chunk if a + chunk < n else 0
        el = time.perf_counter() - start
        if el >= budget_s:
            return done, el


def host_cores():
    """(cores the pool uses, cores this process may run on)."""
    visible = len(os.sched_getaffinity(0))
    return min(visible, HOST_CORE_SHARE), visible


def cpu_baseline(inp, wl, budget_s: float = 6.0, precision: str = "exact", procs: int = 1):
    """The oracle as it stands on the same workload, 1024-token chunks
    streaming through it: one thread from the first token for about budget_s,
    then (procs > 1) one process per core, process i on the i-th contiguous
    share of the tokens, for about 20 s of CPU time in all.  The reported
    value is the aggregate rate of the processes."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    T = wl.T
    chunk = min(ORACLE_CHUNK, T)
    wq = inp["wq"] if wl.norm else None
    wk = inp["wk"] if wl.norm else None
    done, a = 0, 0
    start = time.perf_counter()
    while True:
        sl = slice(a, min(T, a + chunk))
        done += _oracle_chunks(inp["q"][sl], inp["k"][sl], inp["pos"][:, sl], wl, wq, wk,
                               precision, chunk)
        a = a + chunk if a + chunk < T else 0
        elapsed = time.perf_counter() - start
        if elapsed >= budget_s:
            break
    one = done / elapsed
    sample = (f"{done} tokens of {wl.name} in {chunk}-token chunks from token 0 on (all "
              f"{wl.hq}+{wl.hk} heads), {elapsed:.1f} s, one thread")
    used, visible = host_cores()
    if procs <= 1:
        return {"value": one, "unit": "tokens/s", "cores": 1, "cores_visible": visible,
                "kind": "oracle", "sample": sample}
    share = max(chunk, -(-T // procs))
    wall = max(1.0, 20.0 / procs)
    t_start = time.time() + 4.0
    jobs = []
    for i in range(procs):
        a = min(i * share, max(0, T - share))
        sl = slice(a, a + share)
        jobs.append((inp["q"][sl], inp["k"][sl], inp["pos"][:, sl], wl, wq, wk, precision, chunk,
                     t_start, wall))
    try:
        with ProcessPoolExecutor(procs, mp_context=mp.get_context("spawn")) as ex:
            futs = [ex.submit(_oracle_worker, j) for j in jobs]
            res = [f.result(timeout=wall + 180.0) for f in futs]
    except Exception as e:  # a worker died or never started: report the one thread
        return {"value": one, "unit": "tokens/s", "cores": 1, "cores_visible": visible,
                "kind": "oracle",
                "sample": f"{sample} (the {procs}-process sample failed: {type(e).__name__})"}
    agg = sum(d / e for d, e in res)
    toks = sum(d for d, _ in res)
    return {"value": agg, "unit": "tokens/s", "cores": procs, "cores_visible": visible,
            "kind": "oracle", "one_thread": one,
            "sample": f"{procs} processes from one start time, process i on the i-th share of "
                      f"{share} consecutive tokens, {chunk}-token chunks, for {wall:.2f} s each "
                      f"({toks} tokens in all; value = sum of their rates); {visible} cores "
                      f"visible, the pool kept to the box's share of {HOST_CORE_SHARE} per GPU; "
                      f"before them {sample}"}


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

SETTLE_S = 0.2              # seconds of back-to-back steps before each timed phase


def settle_count(step_bytes: int) -> int:
    """Untimed steps run back to back before the requested warm-up of each
    timed phase: about SETTLE_S of GPU time at 6 TB/s (at most 5000).
    After the load starts, the rotary kernels' dispatches run up to 35%
    slower for some tens of milliseconds, then settle (the plain copy shows
    no such dip); a run with a few warm-up steps and a few timed ones would
    otherwise time that dip.  A count from the step's bytes, so the trace
    summary can split the dispatches."""
    return int(min(5000, max(20, -(-SETTLE_S * 6e12 // max(1, step_bytes)))))


def time_region(fns, warmup: int, steps: int, settle: int = 0):
    """`settle` + W untimed steps, then exactly K timed ones; step i calls
    fns[i % len].
    HIP events on torch's current stream (the stream every call here
    launches on) bracket the K steps.  Returns (ms per step, wall ms per
    step).

    Python's cyclic garbage collector is off over the warm-up and timed
    steps, as `timeit` does: a full collection pauses the launching loop
    for tens of milliseconds (35 ms measured after the inputs are built),
    the queue of launches drains and the GPU idles, which read as a 30 %
    slower step in the first timed region of a process."""
    import gc
    import torch
    S = len(fns)
    was_on = gc.isenabled()
    gc.collect()
    gc.disable()
    try:
        for i in range(settle + warmup):
            fns[i % S]()
        stream = torch.cuda.current_stream()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            fns[i % S]()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    finally:
        if was_on:
            gc.enable()
    return ev0.elapsed_time(ev1) / steps, wall * 1e3 / steps


def time_graph(step, graph_steps: int, warmup: int, steps: int):
    """Capture graph_steps steps in one HIP graph and time replays of it
    (launch-bound workloads).  W untimed steps first; then ceil(K / G)
    replays.  Returns (ms per step, steps timed, wall ms per step)."""
    import torch
    for _ in range(warmup):
        step()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(graph_steps):
            step()
    graph.replay()
    torch.cuda.synchronize()
    runs = max(1, -(-steps // graph_steps))
    ms, wall = time_region([graph.replay], 0, runs)
    return ms / graph_steps, runs * graph_steps, wall / graph_steps


def time_steps_cold(step, warmup: int, steps: int, settle: int = 0):
    """Each timed step starts with no line of its inputs in L2 or the MALL:
    a 1 GiB scratch buffer is read (outside the timed interval; a read, so
    that no dirty line of the flush is written back inside the step) before
    it, and the step alone is bracketed by HIP events.  Returns the mean step
    time.  Per-step timing includes the launch's ramp-up and drain, which
    back-to-back timing overlaps."""
    import torch
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(settle + warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    wall0 = time.perf_counter()
    for e0, e1 in evs:
        torch.sum(scratch, dim=0, out=sink)
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps, wall * 1e3 / steps


def copy_ceiling(M, nbytes: int, sets: int, warmup: int, steps: int, settle: int = 0):
    """mrope_stream_copy of nbytes (read) into nbytes (written), rotating over
    `sets` source/destination pairs, back to back: the same measure as the
    kernel's rotating figure.  Returns the record for the JSON line."""
    import torch
    nbytes = (nbytes + 15) // 16 * 16
    pairs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1),
              torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(sets)]
    fns = [lambda s=s, d=d: M.stream_copy(s, d) for s, d in pairs]
    ms, _ = time_region(fns, warmup, steps, settle)
    del pairs
    torch.cuda.empty_cache()
    gbps = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "stream_copy_kernel (mrope_stream_copy)", "bytes_read": nbytes,
            "bytes_written": nbytes, "sets": sets, "settle": settle, "warmup": warmup,
            "steps": steps,
            "ms_per_copy": ms, "gbps": gbps, "frac_of_peak": gbps / HBM_PEAK_GBPS}


def copy_counts(warmup: int, steps: int):
    """(warmup, timed) copies of the copy-ceiling phase: at least 50 and 500,
    so that the ceiling is measured over at least 50 ms of traffic whatever
    --steps is."""
    return max(warmup, 50), max(steps, 500)


ROTATION_SPAN = 1 << 30     # bytes: four times the 256 MB MALL
ROTATION_MAX_SETS = 16      # small workloads: a bound, not the span


def rotation_sets(requested: int, bytes_per_set: int) -> int:
    """Buffer sets the rotating measure cycles through: `requested` when it
    is positive, else the fewest, at least 3, whose inputs and outputs
    together span 1 GiB, so that no step finds in the MALL the lines an
    earlier step left there (3 sets for the headline's 604 MB; 6 for
    chunked video's 184 MB, where 3 sets left part of each in the MALL),
    and at most 16."""
    if requested > 0:
        return requested
    return min(ROTATION_MAX_SETS, max(3, -(-ROTATION_SPAN // max(1, bytes_per_set))))


def measures(M, fns_sets, copy_bytes, args):
    """Copy ceiling, rotating and same-buffer figures of a step, in the order
    the trace summary expects.  fns_sets[i] runs the step on buffer set i."""
    n = settle_count(2 * copy_bytes)
    out = {"settle": n}
    out["copy"] = copy_ceiling(M, copy_bytes, len(fns_sets), *copy_counts(args.warmup, args.steps),
                               settle=n)
    out["rotating"] = time_region(fns_sets, args.warmup, args.steps, n)
    out["same"] = time_region(fns_sets[:1], args.warmup, args.steps, n)
    return out


def dispatch_plan(warmup: int, steps: int, cold: bool = False, settle: int = 0):
    """(kernel family, phase, dispatch count) in launch order, as measures()
    (or, with cold, time_steps_cold()) issues them."""
    if cold:
        return [("kernel", "settle", settle), ("kernel", "warmup", warmup),
                ("kernel", "timed_cold", steps)]
    cw, cs = copy_counts(warmup, steps)
    return [("copy", "settle", settle), ("copy", "warmup", cw), ("copy", "timed_rotating", cs),
            ("kernel", "settle_rotating", settle), ("kernel", "warmup_rotating", warmup),
            ("kernel", "timed_rotating", steps),
            ("kernel", "settle_same_buffers", settle), ("kernel", "warmup_same_buffers", warmup),
            ("kernel", "timed_same_buffers", steps)]


def settle_of_trace(n_kernel: int, warmup: int, steps: int, cold: bool) -> int:
    """The settle count of a traced run, from its rotary-kernel dispatches
    (one settle per timed phase: one phase cold, two otherwise)."""
    phases = 1 if cold else 2
    extra = n_kernel - phases * (warmup + steps)
    return extra // phases if extra > 0 and extra % phases == 0 else 0


def summarize_trace(trace_dir: str, warmup: int, steps: int, cold: bool = False) -> dict:
    """Per-phase durations of the kernels in a rocprofv3 kernel trace of a
    bench.py run (--no-cpu-baseline, same --steps/--warmup/--cold): dispatches
    of the copy kernel and of the rotary kernel, split by dispatch_plan()."""
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no *kernel_trace.csv under {trace_dir}")
    rows = []
    for p in paths:
        with open(p) as f:
            rows.extend(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))

    seq = {"copy": [], "kernel": []}
    names = {}
    for r in rows:
        fam = _family(r["Kernel_Name"])
        if fam is None:
            continue
        seq[fam].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        names.setdefault(fam, r["Kernel_Name"])
    out = {"trace_files": [os.path.relpath(p, trace_dir) for p in paths], "phases": []}
    pos = {"copy": 0, "kernel": 0}
    settle = settle_of_trace(len(seq["kernel"]), warmup, steps, cold)
    out["settle"] = settle
    for fam, phase, n in dispatch_plan(warmup, steps, cold, settle):
        d = seq[fam][pos[fam]:pos[fam] + n]
        pos[fam] += n
        if not d:
            continue
        ds = sorted(d)
        out["phases"].append({"kernel": names.get(fam, fam), "phase": phase, "dispatches": len(d),
                              "mean_us": sum(d) / len(d), "median_us": ds[len(ds) // 2],
                              "min_us": ds[0], "max_us": ds[-1]})
    for fam in seq:
        if pos[fam] != len(seq[fam]):
            out.setdefault("unmatched", {})[fam] = len(seq[fam]) - pos[fam]
    return out


def _pmc_rows(pmc_dir: str):
    paths = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no *counter_collection.csv under {pmc_dir}")
    rows = []
    for p in paths:
        with open(p) as f:
            rows.extend(csv.DictReader(f))
    return rows, paths


def _family(name: str):
    if "stream_copy_kernel" in name:
        return "copy"
    return "kernel" if kernel_family(name) else None


def summarize_counters(pmc_dir: str) -> dict:
    """Per kernel family (the rotary kernel, the copy kernel) and counter of a
    rocprofv3 --pmc run of bench.py: the median over the family's dispatches
    of the counter's value per dispatch (rows of one dispatch summed)."""
    rows, paths = _pmc_rows(pmc_dir)
    per = {}
    names = {}
    for r in rows:
        fam = _family(r["Kernel_Name"])
        if fam is None:
            continue
        key = (fam, r["Counter_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        names.setdefault(fam, r["Kernel_Name"])
    out = {"files": [os.path.relpath(p, pmc_dir) for p in paths], "families": {}}
    by = {}
    for (fam, ctr, _), v in per.items():
        by.setdefault((fam, ctr), []).append(v)
    for (fam, ctr), vals in sorted(by.items()):
        vals.sort()
        rec = out["families"].setdefault(fam, {"kernel": names[fam]})
        rec[ctr] = {"median": vals[len(vals) // 2], "dispatches": len(vals)}
    return out


def traffic_record(fetch_dir: str, write_dir: str, workload: str) -> dict:
    """HBM-side traffic of the rotary kernel from two rocprofv3 --pmc runs of
    bench.py (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).  Each counter is
    scaled by what it reads for the run's own copy phase, a plain copy of
    known size (the q/k bytes read into as many written): scale = bytes /
    (KiB * 1024)."""
    import workloads as W
    wl = W.WORKLOADS.get(workload) or W.VISION_QKV_WORKLOADS[workload]
    if workload in W.WORKLOADS:
        copy_bytes = 2 * wl.T * (wl.hq + wl.hk) * wl.D * wl.elem_bytes // 2
    else:
        copy_bytes = wl.T * 3 * wl.heads * wl.D * (2 if wl.dtype == "bf16" else 4)
    copy_bytes = (copy_bytes + 15) // 16 * 16
    f = summarize_counters(fetch_dir)["families"]
    w = summarize_counters(write_dir)["families"]
    kf, cf = f["kernel"]["FETCH_SIZE"]["median"], f["copy"]["FETCH_SIZE"]["median"]
    kw, cw = w["kernel"]["WRITE_SIZE"]["median"], w["copy"]["WRITE_SIZE"]["median"]
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    rd, wr = kf * 1024 * fs, kw * 1024 * ws
    alg = wl.algorithmic_bytes()
    fam = kernel_family(f["kernel"]["kernel"])
    return {"kernel": f["kernel"]["kernel"], "workload": workload, "kernel_family": fam,
            "kernel_sources": KERNEL_SOURCES[fam], "kernel_source_hash": kernel_source_hash(fam),
            "kernel_fetch_kib_per_dispatch": kf, "kernel_write_kib_per_dispatch": kw,
            "kernel_dispatches": [f["kernel"]["FETCH_SIZE"]["dispatches"],
                                  w["kernel"]["WRITE_SIZE"]["dispatches"]],
            "copy_bytes": copy_bytes, "copy_kernel": f["copy"]["kernel"],
            "copy_fetch_kib_per_dispatch": cf, "copy_write_kib_per_dispatch": cw,
            "fetch_scale": fs, "write_scale": ws,
            "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
            "hbm_bytes_per_launch": rd + wr, "algorithmic_bytes_per_launch": alg,
            "traffic_over_algorithmic": (rd + wr) / alg}


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def build_cache(M, dim: int, theta: float, rows: int):
    """The cos/sin cache by position, built once; its build time (HIP events,
    median of 5 builds) goes into the JSON line beside the step time."""
    import torch
    cache = M.mrope_cos_sin_cache(dim, theta, rows)
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        M.mrope_cos_sin_cache(dim, theta, rows, out=cache)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return cache, {"rows": rows, "dim": dim, "bytes": rows * dim * 4,
                   "build_ms": sorted(times)[2]}


def bench_positions(args):
    """One step = one mrope_rope_index call (two kernels at this size, three
    past the fused pass's limits) over the batch; one buffer set (1.3 MB)."""
    import torch
    import workloads as W
    import vlm_multimodal_rotary_amd as M

    wl = W.POSITION_WORKLOADS[args.workload]
    types, mask, images, videos = W.mm_prompt_batch(wl)
    td, md = torch.from_numpy(types).cuda(), torch.from_numpy(mask).cuda()
    gi, gv = torch.from_numpy(images).cuda(), torch.from_numpy(videos).cuda()
    B, L = types.shape
    lib = M.load()
    ws_bytes = lib.mrope_rope_index_workspace_size(B, L, gi.shape[0], gv.shape[0])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    pos = torch.empty((3, B * L), dtype=torch.int32, device="cuda")
    delta = torch.empty(B, dtype=torch.int32, device="cuda")
    status = torch.empty(1, dtype=torch.int32, device="cuda")

    def step():
        M.rope_index_into(td, md, gi, gv, 2, pos, delta, status, ws)

    if args.graph > 0:
        ms, n, wall_ms = time_graph(step, args.graph, args.warmup, args.steps)
    else:
        (ms, wall_ms), n = time_region([step], args.warmup, args.steps), args.steps
    assert int(status.item()) == 0
    alg = wl.algorithmic_bytes()
    gbps = alg / (ms * 1e-3) / 1e9
    line = {
        "metric": "position-table tokens/s (mrope_rope_index)",
        "value": wl.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": n,
        "warmup": args.warmup, "ms_per_step": ms, "wall_ms_per_step": wall_ms,
        "graph_steps": args.graph, "measure": "same_buffers", "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic (seeded chat-style multimodal prompts)",
        "config": {"workload": wl.name, "batch": B, "seq_len": L, "images": int(gi.shape[0]),
                   "videos": int(gv.shape[0]), "merge": 2},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None, "algorithmic_bytes": alg,
                     "kernel": f"{M.last_kernel()} (mrope_rope_index, one step)"},
    }
    if not args.no_cpu_baseline:
        from oracle import positions_oracle as PO
        start = time.perf_counter()
        reps = 0
        while time.perf_counter() - start < 10.0:
            PO.get_rope_index(types, images, videos, mask)
            reps += 1
        el = time.perf_counter() - start
        line["cpu_baseline"] = {"value": reps * wl.T / el, "unit": "tokens/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{reps} full batches of {wl.T} slots, {el:.1f} s, "
                                          "one thread"}
    print(json.dumps(line), flush=True)


def line_measures(meas, alg_bytes, units):
    """The rotating / same-buffer / copy records of the JSON line."""
    (ms_r, wall_r), (ms_s, wall_s) = meas["rotating"], meas["same"]
    cp = meas["copy"]
    rec = {
        "rotating": {"ms_per_step": ms_r, "wall_ms_per_step": wall_r,
                     "gbps": alg_bytes / (ms_r * 1e-3) / 1e9,
                     "frac": alg_bytes / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "units_per_s": units / (ms_r * 1e-3)},
        "same_buffers": {"ms_per_step": ms_s, "wall_ms_per_step": wall_s,
                         "gbps": alg_bytes / (ms_s * 1e-3) / 1e9,
                         "frac": alg_bytes / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "units_per_s": units / (ms_s * 1e-3)},
        "copy_ceiling": dict(cp, kernel_frac_of_copy=cp["ms_per_copy"] / ms_r),
        "settle": settle_record(meas["settle"]),
    }
    return rec


def settle_record(n: int):
    return {"steps_per_phase": n,
            "note": "untimed back-to-back steps before the requested warm-up of each timed "
                    "phase (copy, rotating, one buffer set), about 200 ms of GPU time: after "
                    "the load starts the rotary kernels run up to 35% slower for some tens of "
                    "milliseconds before they settle"}


def bench_vision_qkv(args):
    """One step = one mrope_vision_qkv call: packed qkv in, rotated q/k and
    copied v in per-head planes out; rotating over buffer sets."""
    import numpy as np
    import torch
    import workloads as W
    import vlm_multimodal_rotary_amd as M

    wl = W.VISION_QKV_WORKLOADS[args.workload]
    inp = W.make_vision_qkv_inputs(wl)
    n = wl.T
    flat = inp["qkv"].reshape(n, -1)
    if wl.dtype == "bf16":
        qkv0 = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        qkv0 = torch.from_numpy(flat).cuda()
    qkv0 = qkv0.reshape(n, 3, wl.heads, wl.D)
    pos = torch.from_numpy(inp["pos"]).cuda()
    shape = (wl.heads, n, wl.D)
    cache, cache_info = None, None
    if args.cs_cache:
        cache, cache_info = build_cache(M, wl.rotary_dim // 2, wl.theta,
                                        int(inp["pos"].max()) + 1)
    sets = []
    n_sets = rotation_sets(args.rotate, 2 * qkv0.numel() * qkv0.element_size())
    for i in range(n_sets):
        qkv = qkv0 if i == 0 else qkv0.clone()
        outs = tuple(torch.empty(shape, dtype=qkv0.dtype, device="cuda") for _ in range(3))
        sets.append((qkv, outs))

    def make_step(qkv, outs):
        def step():
            M.vision_qkv(qkv, pos, wl.rotary_dim, wl.theta, q_out=outs[0], k_out=outs[1],
                         v_out=outs[2], precision=args.precision, cs_cache=cache)
        return step

    fns = [make_step(*s) for s in sets]
    meas = measures(M, fns, qkv0.numel() * qkv0.element_size(), args)
    kernel = M.last_kernel()
    alg = wl.algorithmic_bytes()
    rec = line_measures(meas, alg, n)
    ms = rec["rotating"]["ms_per_step"]
    gbps = rec["rotating"]["gbps"]
    traffic, traffic_note = ((None, "not taken for this precision or the cache")
                             if args.precision != "exact" or args.cs_cache
                             else measured_traffic(wl.name, kernel))
    line = {
        "metric": "vision patches/s, packed qkv to rotated head-major planes (mrope_vision_qkv)",
        "value": n / (ms * 1e-3), "unit": "patches/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms,
        "wall_ms_per_step": rec["rotating"]["wall_ms_per_step"],
        "measure": f"rotating over {n_sets} buffer sets", "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded normal qkv, merge-block patch positions)",
        "config": {"workload": wl.name, "patches": n, "heads": wl.heads, "D": wl.D,
                   "rotary_dim": wl.rotary_dim, "theta": wl.theta, "layout": "vision_2d",
                   "output": "head-major planes", "precision": args.precision,
                   "cs_cache": cache_info},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic,
                     "traffic_note": traffic_note, "algorithmic_bytes": alg,
                     "kernel": f"{kernel} (mrope_vision_qkv)"},
        **rec,
    }
    if not args.no_cpu_baseline:
        from oracle import mrope_oracle as O
        chunk, done, t0 = ORACLE_CHUNK, 0, 0
        start = time.perf_counter()
        while time.perf_counter() - start < 12.0:
            sl = slice(t0, min(n, t0 + chunk))
            O.vision_qkv(inp["qkv"][sl], inp["pos"][:, sl], rotary_dim=wl.rotary_dim,
                         theta=wl.theta, dtype=wl.dtype, precision=args.precision)
            done += sl.stop - sl.start
            t0 = sl.stop if sl.stop < n else 0
        el = time.perf_counter() - start
        line["cpu_baseline"] = {"value": done / el, "unit": "patches/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{done} patches in {chunk}-patch chunks from patch 0 "
                                          f"on, {el:.1f} s, one thread"}
    print(json.dumps(line), flush=True)


def cpu_baseline_decode(inp, wl, budget_s: float = 10.0, precision: str = "exact"):
    """The oracle's decode step on groups of 8 consecutive sequences of the
    same batch (their q, k, cache rows and lengths), until about budget_s of
    CPU time; single thread."""
    from oracle import mrope_oracle as O
    group = 8
    B = wl.batch
    done = 0
    b0 = 0
    start = time.perf_counter()
    while True:
        rows = slice(b0 * wl.new_tokens, (b0 + group) * wl.new_tokens)
        O.mrope_decode_qk(inp["q"][rows], inp["k"][rows], inp["cache_len"][b0:b0 + group],
                          wl.new_tokens, inp["rope_delta"][b0:b0 + group],
                          inp["k_cache"][b0:b0 + group], rotary_dim=wl.rotary_dim,
                          theta=wl.theta, wq=inp["wq"], wk=inp["wk"], eps=wl.eps,
                          dtype=wl.dtype, precision=precision)
        done += group * wl.new_tokens
        b0 = (b0 + group) % (B - group + 1)
        elapsed = time.perf_counter() - start
        if elapsed >= budget_s:
            break
    return {"value": done / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} decode tokens (groups of {group} sequences with their cache "
                      f"rows) of {wl.name}, {elapsed:.1f} s, one thread"}


def bench_decode(args, wl, inp, dev):
    """One step = one mrope_decode_qk call (one buffer set: the step moves
    9.4 MB, latency-bound)."""
    import torch
    import vlm_multimodal_rotary_amd as M
    q, k = dev(inp["q"]), dev(inp["k"])
    wq, wk = dev(inp["wq"]), dev(inp["wk"])
    q_out = torch.empty_like(q)
    cache_len, rope_delta, k_cache = (dev(inp["cache_len"]), dev(inp["rope_delta"]),
                                      dev(inp["k_cache"]))

    def step():
        M.mrope_decode_qk(q, k, cache_len, rope_delta, wl.new_tokens, wl.rotary_dim,
                          wl.theta, k_cache, wq=wq, wk=wk, eps=wl.eps, q_out=q_out,
                          precision=args.precision)

    if args.graph > 0:
        ms, n, wall_ms = time_graph(step, args.graph, args.warmup, args.steps)
    else:
        (ms, wall_ms), n = time_region([step], args.warmup, args.steps), args.steps
    alg = wl.algorithmic_bytes()
    gbps = alg / (ms * 1e-3) / 1e9
    line = {
        "metric": "decode tokens/s, mrope_decode_qk", "value": wl.T / (ms * 1e-3),
        "unit": "tokens/s", "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": ms,
        "wall_ms_per_step": wall_ms, "graph_steps": args.graph, "measure": "same_buffers",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded normal q/k, cache lengths and rope deltas)",
        "config": {"workload": wl.name, "batch": wl.batch, "new_tokens": wl.new_tokens,
                   "hq": wl.hq, "hk": wl.hk, "D": wl.D, "rotary_dim": wl.rotary_dim,
                   "theta": wl.theta, "cache_rows": wl.capacity, "rmsnorm": wl.norm,
                   "precision": args.precision},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "traffic_note": "not taken for decode", "algorithmic_bytes": alg,
                     "kernel": f"{M.last_kernel()} (mrope_decode_qk)"},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(inp, wl, precision=args.precision)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=0,
                    help="buffer sets the rotating measure cycles through (default: the fewest, "
                         "at least 3, that span 1 GiB, so no step finds its inputs in the 256 MB "
                         "MALL; 3 = 1.8 GB for the headline)")
    ap.add_argument("--cold", action="store_true",
                    help="instead: read a 1 GiB scratch buffer before every timed step (evicts "
                         "L2 and the 256 MB MALL) and time each step alone with HIP events")
    ap.add_argument("--cs-cache", action="store_true",
                    help="gather cos/sin from a cache by position (built once before the timed "
                         "steps; its build time is reported separately)")
    ap.add_argument("--precision", default="exact", choices=["exact", "dtype", "fp32"],
                    help="rotation rounding: exact (default), dtype (cos/sin cast to the "
                         "tensor dtype, bf16 tensor ops) or fp32 (fp32 tensor ops)")
    ap.add_argument("--cpu-procs", type=int, default=0,
                    help="processes for the oracle's multi-process sample (default: the "
                         "cores this process may run on, within the box's share of 16; "
                         "1 = one thread only)")
    ap.add_argument("--graph", type=int, default=0,
                    help="decode and position workloads: capture this many steps in one HIP "
                         "graph and time graph replays")
    ap.add_argument("--trace-summary", default="",
                    help="print per-phase kernel durations of a rocprofv3 kernel trace "
                         "directory of a bench.py run with the same --steps/--warmup/--cold")
    ap.add_argument("--pmc-summary", default="",
                    help="print per-kernel medians of every counter of a rocprofv3 --pmc "
                         "directory of a bench.py run")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the traffic record of --workload from a FETCH_SIZE and a "
                         "WRITE_SIZE rocprofv3 --pmc run of bench.py")
    args = ap.parse_args()

    if args.trace_summary:
        print(json.dumps(summarize_trace(args.trace_summary, args.warmup, args.steps, args.cold),
                         indent=1))
        return
    if args.pmc_summary:
        print(json.dumps(summarize_counters(args.pmc_summary), indent=1))
        return
    if args.traffic_record:
        print(json.dumps(traffic_record(*args.traffic_record, args.workload), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this hot path has no exchange step, and "
              "every run here uses a single MI355X. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.rotate < 0:
        print("--steps >= 1, --warmup >= 0 and --rotate >= 0 are required", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    import vlm_multimodal_rotary_amd as M

    if args.workload in W.POSITION_WORKLOADS:
        bench_positions(args)
        return
    if args.workload in W.VISION_QKV_WORKLOADS:
        bench_vision_qkv(args)
        return
    decode = args.workload in W.DECODE_WORKLOADS
    wl = W.DECODE_WORKLOADS[args.workload] if decode else W.WORKLOADS[args.workload]
    inp = W.make_decode_inputs(wl) if decode else W.make_inputs(wl)

    def dev(a):
        if a is None:
            return None
        if wl.dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    if decode:
        bench_decode(args, wl, inp, dev)
        return

    q0, k0 = dev(inp["q"]), dev(inp["k"])
    wq, wk = dev(inp["wq"]), dev(inp["wk"])
    pos = dev(inp["pos"])
    cache, cache_info = None, None
    if args.cs_cache:
        rows = int(inp["pos"].max()) + 1
        dim = wl.rotary_dim // 2 if wl.layout == "vision_2d" else wl.rotary_dim
        cache, cache_info = build_cache(M, dim, wl.theta, rows)
    sets = []
    n_sets = rotation_sets(args.rotate, 2 * (q0.numel() + k0.numel()) * q0.element_size())
    for i in range(n_sets):
        q, k = (q0, k0) if i == 0 else (q0.clone(), k0.clone())
        sets.append((q, k, torch.empty_like(q), torch.empty_like(k)))

    def make_step(q, k, q_out, k_out):
        def step():
            M.rmsnorm_mrope_qk(q, k, pos, wl.rotary_dim, wl.theta, wl.section, wl.layout,
                               wq=wq, wk=wk, eps=wl.eps, q_out=q_out, k_out=k_out,
                               precision=args.precision, cs_cache=cache)
        return step

    fns = [make_step(*s) for s in sets]
    alg_bytes = wl.algorithmic_bytes()
    qk_bytes = (q0.numel() + k0.numel()) * q0.element_size()
    if args.cold:
        settle = settle_count(2 * qk_bytes)
        ms, wall_ms = time_steps_cold(fns[0], args.warmup, args.steps, settle)
        rec = {"settle": settle_record(settle)}
        measure = "cold: 1 GiB read before each step, each step timed alone"
    else:
        rec = line_measures(measures(M, fns, qk_bytes, args), alg_bytes, wl.T)
        ms, wall_ms = rec["rotating"]["ms_per_step"], rec["rotating"]["wall_ms_per_step"]
        measure = f"rotating over {n_sets} buffer sets, back to back"
    kernel = M.last_kernel()

    achieved_gbps = alg_bytes / (ms * 1e-3) / 1e9
    traffic, traffic_note = ((None, "not taken for this precision or the cache")
                             if args.precision != "exact" or args.cs_cache
                             else measured_traffic(wl.name, kernel))
    config = {"workload": wl.name, "T": wl.T, "hq": wl.hq, "hk": wl.hk, "D": wl.D,
              "rotary_dim": wl.rotary_dim, "theta": wl.theta, "layout": wl.layout,
              "section": list(wl.section), "rmsnorm": wl.norm, "precision": args.precision}
    if cache_info:
        config["cs_cache"] = cache_info
    line = {
        "metric": "Q+K tokens/s and achieved HBM GB/s (% of peak), fused RMSNorm+MRoPE",
        "value": wl.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "wall_ms_per_step": wall_ms,
        "measure": measure,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded normal q/k, N(1,0.1) weights, workload position tables)",
        "config": config,
        "hbm_gbps": achieved_gbps,
        "roofline": {"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "traffic_note": traffic_note,
                     "algorithmic_bytes": alg_bytes,
                     "kernel": f"{kernel} (rmsnorm_mrope_qk)"},
        **rec,
    }
    if not args.no_cpu_baseline:
        used, _ = host_cores()
        line["cpu_baseline"] = cpu_baseline(inp, wl, precision=args.precision,
                                            procs=args.cpu_procs or used)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
