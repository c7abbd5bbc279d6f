#!/usr/bin/env python3
"""Throughput of the fused RMSNorm + MRoPE hot path on one MI355X.

One step = one rmsnorm_mrope_qk call over the whole workload (cos/sin from
positions, per-head RMSNorm, rotation of every q and k head), inputs resident
in HBM.  Default workload: Omni-like text prefill, q[32768,32,128] and
k[32768,4,128] bf16, interleaved [24,20,20], theta 1e6, RMSNorm eps 1e-6.

Prints one JSON line: Q+K tokens/s (value), achieved HBM bandwidth of the
kernel against the 8 TB/s peak (roofline), and the CPU oracle's rate on a
bounded sample of the same workload (cpu_baseline: one thread, then one
process per core).

Warmup is at least W steps and at least --min-warmup-s seconds: the first
tens of milliseconds of sustained HBM traffic run at a different clock state,
and the timed K steps are meant to see the steady state.  Each step is one
kernel launch on torch's current stream, timed with HIP events on that stream.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--graph G] [--cold] [--cs-cache] [--precision exact|dtype|fp32]
                  [--cpu-procs P]
  python bench.py --copy-calib BYTES   # plain device copy, for counter scaling

Other workloads time the other entry points the same way: the decode step
(omni_decode), the vision packed-qkv fusion (vision_qkv_planes[_bf16]) and
the position builder (mm_prompt_positions).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, vendor peak
DEFAULT_WORKLOAD = "omni_text_prefill"
KERNEL_SOURCES = ["vlm_multimodal_rotary_amd/csrc/mrope_kernels.hip",
                  "vlm_multimodal_rotary_amd/csrc/mrope_api.cpp",
                  "vlm_multimodal_rotary_amd/csrc/mrope_internal.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _oracle_fused_windows(q, k, pos, wl, wq, wk, precision, chunk):
    from oracle import mrope_oracle as O
    for i in range(q.shape[0] // chunk):
        sl = slice(i * chunk, (i + 1) * chunk)
        O.rmsnorm_mrope_qk(q[sl], k[sl], pos[:, sl], rotary_dim=wl.rotary_dim, theta=wl.theta,
                           section=wl.section, layout=wl.layout, wq=wq, wk=wk, eps=wl.eps,
                           dtype=wl.dtype, precision=precision)


def _oracle_worker(job):
    """One process of the multi-process oracle sample: from a common start
    time, repeats the oracle over its own token windows until the deadline.
    Returns (tokens done, seconds)."""
    q, k, pos, wl, wq, wk, precision, chunk, t_start, budget_s = job
    now = time.time()
    if now < t_start:
        time.sleep(t_start - now)
    start = time.perf_counter()
    done = 0
    while True:
        _oracle_fused_windows(q, k, pos, wl, wq, wk, precision, chunk)
        done += q.shape[0]
        el = time.perf_counter() - start
        if el >= budget_s:
            return done, el


def cpu_baseline(inp, wl, budget_s: float = 8.0, precision: str = "exact", procs: int = 1):
    """The oracle as it stands, on consecutive 64-token windows of the same
    workload: one thread for about budget_s, then (procs > 1) one process per
    core, each on its own 8 windows, for about 20 s of CPU time in all.  The
    reported value is the aggregate rate of the processes."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    T = wl.T
    chunk = min(64, T)
    wq = inp["wq"] if wl.norm else None
    wk = inp["wk"] if wl.norm else None
    done = 0
    start = time.perf_counter()
    t0 = 0
    while True:
        sl = slice(t0, t0 + chunk)
        _oracle_fused_windows(inp["q"][sl], inp["k"][sl], inp["pos"][:, sl], wl, wq, wk,
                              precision, chunk)
        done += chunk
        t0 = (t0 + chunk) % (T - chunk + 1)
        elapsed = time.perf_counter() - start
        if elapsed >= budget_s:
            break
    one = done / elapsed
    sample = (f"{done} tokens ({done // chunk} windows of {chunk} consecutive tokens, all "
              f"{wl.hq}+{wl.hk} heads) of {wl.name}, {elapsed:.1f} s, one thread")
    if procs <= 1:
        return {"value": one, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                "sample": sample}
    per = min(8, T // chunk) * chunk
    stride = max(per, (T - per) // procs)
    wall = max(1.0, 20.0 / procs)
    t_start = time.time() + 4.0
    jobs = []
    for i in range(procs):
        a = min(i * stride, T - per)
        jobs.append((inp["q"][a:a + per], inp["k"][a:a + per], inp["pos"][:, a:a + per], wl,
                     wq, wk, precision, chunk, t_start, wall))
    try:
        with ProcessPoolExecutor(procs, mp_context=mp.get_context("spawn")) as ex:
            futs = [ex.submit(_oracle_worker, j) for j in jobs]
            res = [f.result(timeout=wall + 120.0) for f in futs]
    except Exception as e:  # a worker died or never started: report the one thread
        return {"value": one, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                "sample": f"{sample} (the {procs}-process sample failed: {type(e).__name__})"}
    agg = sum(d / e for d, e in res)
    toks = sum(d for d, _ in res)
    return {"value": agg, "unit": "tokens/s", "cores": procs, "kind": "oracle",
            "one_thread": one,
            "sample": f"{procs} processes from one start time, each repeating {per // chunk} windows of "
                      f"{chunk} tokens for {wall:.1f} s ({toks} tokens in all; value = sum of "
                      f"their rates); before them {sample}"}


def time_steps(step, args, stream=None):
    """Warm up (at least W steps and --min-warmup-s), optionally capture
    --graph steps in one HIP graph, then time K steps with HIP events on the
    launching stream.  Returns (ms per step, steps timed, warmup steps, wall
    ms per step)."""
    import torch
    t_warm = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_warm < args.min_warmup_s:
        for _ in range(50):
            step()
        done += 50
        torch.cuda.synchronize()
    runner = step
    per_run = 1
    if args.graph > 0:
        # Capture G steps once; each replay launches them back to back without
        # host overhead.  The captured launches are plain kernel launches.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.graph):
                step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        runner = graph.replay
        per_run = args.graph
    runs = max(1, args.steps // per_run)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(runs):
        runner()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    n = runs * per_run
    return ev0.elapsed_time(ev1) / n, n, done, wall * 1e3 / n


def time_steps_cold(step, args):
    """Each timed step starts with no line of its inputs in L2 or the 256 MB
    MALL: a 1 GiB scratch read (outside the timed interval; a read, so that
    no dirty line of the flush is written back inside the step) precedes
    it, and the step alone is bracketed by HIP events.  Returns the mean
    step time.  The step's own writes may then stay in the MALL past the
    end of the step, which back-to-back timing does not allow."""
    import torch
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(max(3, args.warmup // 50)):
        step()
    torch.cuda.synchronize()
    n = max(1, min(args.steps, 500))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    wall0 = time.perf_counter()
    for e0, e1 in evs:
        torch.sum(scratch, dim=0, out=sink)
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total = sum(e0.elapsed_time(e1) for e0, e1 in evs)
    return total / n, n, 0, wall * 1e3 / n


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
    """One step = one mrope_rope_index call (two kernels at this size, three past the
    fused pass's limits) over the batch."""
    import numpy as np
    import torch
    import workloads as W
    import vlm_multimodal_rotary_amd as M
    from vlm_multimodal_rotary_amd import _lib
    import ctypes

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
    P = ctypes.c_void_p

    def step():
        _lib.check(lib.mrope_rope_index(
            P(td.data_ptr()), P(md.data_ptr()), B, L, P(gi.data_ptr()), gi.shape[0],
            P(gv.data_ptr()), gv.shape[0], 2, P(pos.data_ptr()), B * L, P(delta.data_ptr()),
            P(status.data_ptr()), P(ws.data_ptr()), ws_bytes,
            P(torch.cuda.current_stream().cuda_stream)))

    ms, n, warm, wall_ms = time_steps(step, args)
    assert int(status.item()) == 0
    alg = wl.algorithmic_bytes()
    gbps = alg / (ms * 1e-3) / 1e9
    line = {
        "metric": "position-table tokens/s (mrope_rope_index)",
        "value": wl.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": n,
        "warmup": warm, "ms_per_step": ms, "wall_ms_per_step": wall_ms,
        "graph_steps": args.graph, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32",
        "data": "synthetic (seeded chat-style multimodal prompts)",
        "config": {"workload": wl.name, "batch": B, "seq_len": L, "images": int(gi.shape[0]),
                   "videos": int(gv.shape[0]), "merge": 2},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None, "algorithmic_bytes": alg,
                     "kernel": "rope_index_summarize + rope_index_carry + rope_index_apply "
                               "(one step)"},
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


def bench_vision_qkv(args):
    """One step = one mrope_vision_qkv call: packed qkv in, rotated q/k and
    copied v in per-head planes out."""
    import numpy as np
    import torch
    import workloads as W
    import vlm_multimodal_rotary_amd as M

    wl = W.VISION_QKV_WORKLOADS[args.workload]
    inp = W.make_vision_qkv_inputs(wl)
    n = wl.T
    flat = inp["qkv"].reshape(n, -1)
    if wl.dtype == "bf16":
        qkv = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        qkv = torch.from_numpy(flat).cuda()
    qkv = qkv.reshape(n, 3, wl.heads, wl.D)
    pos = torch.from_numpy(inp["pos"]).cuda()
    shape = (wl.heads, n, wl.D)
    qo, ko, vo = (torch.empty(shape, dtype=qkv.dtype, device="cuda") for _ in range(3))
    cache, cache_info = None, None
    if args.cs_cache:
        cache, cache_info = build_cache(M, wl.rotary_dim // 2, wl.theta,
                                        int(inp["pos"].max()) + 1)

    def step():
        M.vision_qkv(qkv, pos, wl.rotary_dim, wl.theta, q_out=qo, k_out=ko, v_out=vo,
                     precision=args.precision, cs_cache=cache)

    ms, n_timed, warm, wall_ms = time_steps(step, args)
    alg = wl.algorithmic_bytes()
    gbps = alg / (ms * 1e-3) / 1e9
    line = {
        "metric": "vision patches/s, packed qkv to rotated head-major planes (mrope_vision_qkv)",
        "value": n / (ms * 1e-3), "unit": "patches/s", "n_gpus": 1, "steps": n_timed,
        "warmup": warm, "ms_per_step": ms, "wall_ms_per_step": wall_ms,
        "graph_steps": args.graph, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded normal qkv, merge-block patch positions)",
        "config": {"workload": wl.name, "patches": n, "heads": wl.heads, "D": wl.D,
                   "rotary_dim": wl.rotary_dim, "theta": wl.theta, "layout": "vision_2d",
                   "output": "head-major planes", "precision": args.precision,
                   "cs_cache": cache_info},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": measured_traffic(wl.name)
                     if args.precision == "exact" and not args.cs_cache else None,
                     "algorithmic_bytes": alg,
                     "kernel": f"{M.last_kernel()} (mrope_vision_qkv)"},
    }
    if not args.no_cpu_baseline:
        from oracle import mrope_oracle as O
        chunk, done, t0 = 64, 0, 0
        start = time.perf_counter()
        while time.perf_counter() - start < 12.0:
            sl = slice(t0, t0 + chunk)
            O.vision_qkv(inp["qkv"][sl], inp["pos"][:, sl], rotary_dim=wl.rotary_dim,
                         theta=wl.theta, dtype=wl.dtype, precision=args.precision)
            done += chunk
            t0 = (t0 + chunk) % (n - chunk + 1)
        el = time.perf_counter() - start
        line["cpu_baseline"] = {"value": done / el, "unit": "patches/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{done} patches ({done // chunk} windows of {chunk}), "
                                          f"{el:.1f} s, one thread"}
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


def copy_calib(nbytes: int, steps: int):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "steps": steps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--min-warmup-s", type=float, default=0.5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="write a 1 GiB scratch buffer before every timed step (evicts L2 and the "
                         "256 MB MALL) and time each step alone with HIP events")
    ap.add_argument("--cs-cache", action="store_true",
                    help="gather cos/sin from a cache by position (built once before the timed "
                         "steps; its build time is reported separately)")
    ap.add_argument("--precision", default="exact", choices=["exact", "dtype", "fp32"],
                    help="rotation rounding: exact (default), dtype (cos/sin cast to the "
                         "tensor dtype, bf16 tensor ops) or fp32 (fp32 tensor ops)")
    ap.add_argument("--cpu-procs", type=int, default=0,
                    help="processes for the oracle's multi-process sample (default: the "
                         "cores this process may run on, at most 16; 1 = one thread only)")
    ap.add_argument("--copy-calib", type=int, default=0)
    ap.add_argument("--graph", type=int, default=0,
                    help="capture this many steps in one HIP graph and time graph replays "
                         "(for launch-bound workloads)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this hot path has no exchange step, and "
              "every run here uses a single MI355X. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calib(args.copy_calib, args.steps)
        return

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

    q, k = dev(inp["q"]), dev(inp["k"])
    wq, wk = dev(inp["wq"]), dev(inp["wk"])
    q_out = torch.empty_like(q)
    if decode:
        cache_len, rope_delta, k_cache = (dev(inp["cache_len"]), dev(inp["rope_delta"]),
                                          dev(inp["k_cache"]))

        def step():
            M.mrope_decode_qk(q, k, cache_len, rope_delta, wl.new_tokens, wl.rotary_dim,
                              wl.theta, k_cache, wq=wq, wk=wk, eps=wl.eps, q_out=q_out,
                              precision=args.precision)
    else:
        pos = dev(inp["pos"])
        k_out = torch.empty_like(k)
        cache = None
        if args.cs_cache:
            rows = int(inp["pos"].max()) + 1
            dim = wl.rotary_dim // 2 if wl.layout == "vision_2d" else wl.rotary_dim
            cache, cache_info = build_cache(M, dim, wl.theta, rows)

        def step():
            M.rmsnorm_mrope_qk(q, k, pos, wl.rotary_dim, wl.theta, wl.section, wl.layout,
                               wq=wq, wk=wk, eps=wl.eps, q_out=q_out, k_out=k_out,
                               precision=args.precision, cs_cache=cache)

    if args.cold:
        ms, n_timed, done, wall_ms = time_steps_cold(step, args)
    else:
        ms, n_timed, done, wall_ms = time_steps(step, args)   # one kernel launch per step

    alg_bytes = wl.algorithmic_bytes()
    achieved_gbps = alg_bytes / (ms * 1e-3) / 1e9
    traffic = measured_traffic(wl.name) if args.precision == "exact" else None
    if decode:
        config = {"workload": wl.name, "batch": wl.batch, "new_tokens": wl.new_tokens,
                  "hq": wl.hq, "hk": wl.hk, "D": wl.D, "rotary_dim": wl.rotary_dim,
                  "theta": wl.theta, "cache_rows": wl.capacity, "rmsnorm": wl.norm,
                  "precision": args.precision}
    else:
        config = {"workload": wl.name, "T": wl.T, "hq": wl.hq, "hk": wl.hk, "D": wl.D,
                  "rotary_dim": wl.rotary_dim, "theta": wl.theta, "layout": wl.layout,
                  "section": list(wl.section), "rmsnorm": wl.norm,
                  "precision": args.precision}
    line = {
        "metric": ("decode tokens/s, mrope_decode_qk" if decode else
                   "Q+K tokens/s and achieved HBM GB/s (% of peak), fused RMSNorm+MRoPE"),
        "value": wl.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n_timed,
        "warmup": done,
        "ms_per_step": ms,
        "wall_ms_per_step": wall_ms,
        "graph_steps": args.graph,
        "cold": args.cold,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded normal q/k, N(1,0.1) weights, workload position tables)",
        "config": config,
        "hbm_gbps": achieved_gbps,
        "roofline": {"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes": alg_bytes,
                     "kernel": f"{M.last_kernel()} (mrope_decode_qk)" if decode
                     else f"{M.last_kernel()} (rmsnorm_mrope_qk)"},
    }
    if not decode and args.cs_cache:
        line["config"]["cs_cache"] = cache_info
        line["roofline"]["traffic"] = None
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = (cpu_baseline_decode(inp, wl, precision=args.precision) if decode
                                else cpu_baseline(inp, wl, precision=args.precision,
                                                  procs=args.cpu_procs or
                                                  min(len(os.sched_getaffinity(0)), 16)))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
