"""The oracle over token chunks in worker processes, for full-size parity.

The GPU tests hand each worker a chunk of the inputs and the GPU's outputs for
the same tokens; the worker runs the oracle on the chunk and returns what the
comparison found (values compared, values that differ, the largest
difference).  Only numpy and the oracle are imported here: the workers are
spawned interpreters that never touch the GPU.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

CHUNK = 1024


def pool_size() -> int:
    """Workers: the cores this process may run on, within the 16 a GPU machine
    gives one GPU."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def make_pool() -> ProcessPoolExecutor:
    return ProcessPoolExecutor(pool_size(), mp_context=mp.get_context("spawn"))


def compare(got: np.ndarray, want: np.ndarray, dtype: str):
    """(values, values that differ, largest difference): bf16 in ulps
    (ordered integers of the bit patterns, +0 == -0), binary32 as the
    absolute difference (values that differ = not bit-equal)."""
    assert got.shape == want.shape, (got.shape, want.shape)
    if dtype == "bf16":
        def ordered(bits):
            b = bits.astype(np.int64)
            mag = b & 0x7FFF
            return np.where(b & 0x8000, -mag, mag)
        d = np.abs(ordered(got) - ordered(want))
        return int(d.size), int(np.count_nonzero(d)), float(d.max()) if d.size else 0.0
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    n_off = int(np.count_nonzero(got.view(np.uint32) != want.view(np.uint32)))
    return int(err.size), n_off, float(err.max()) if err.size else 0.0


def fused_chunk(job):
    """Oracle rmsnorm_mrope_qk on one chunk against the GPU's q and k rows."""
    from oracle import mrope_oracle as O
    kw, q, k, pos, wq, wk, precision, gq, gk = job
    oq, ok = O.rmsnorm_mrope_qk(q, k, pos, wq=wq, wk=wk, precision=precision, **kw)
    return compare(gq, oq, kw["dtype"]), compare(gk, ok, kw["dtype"])


def vision_chunk(job):
    """Oracle vision_qkv on one chunk of patches against the GPU's planes."""
    from oracle import mrope_oracle as O
    kw, qkv, pos, gq, gk, gv = job
    oq, ok, ov = O.vision_qkv(qkv, pos, **kw)
    return (compare(gq, oq, kw["dtype"]), compare(gk, ok, kw["dtype"]),
            (int(gv.size), int(np.count_nonzero(gv.view(np.uint8) != ov.view(np.uint8))), 0.0))


def merge(results):
    """Sum the per-chunk comparisons of one output."""
    n = sum(r[0] for r in results)
    off = sum(r[1] for r in results)
    worst = max((r[2] for r in results), default=0.0)
    return n, off, worst
