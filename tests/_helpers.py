"""Shared test helpers: device transfer and the parity comparisons."""
from __future__ import annotations

import sys

import numpy as np


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a failing run says where)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a, dtype: str, device="cuda"):
    import torch
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.int32:
        t = torch.from_numpy(np.ascontiguousarray(a))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def from_dev(t):
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_ordered(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> integers whose differences count ulps (+0 == -0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_bf16_close(got: np.ndarray, want: np.ndarray, max_ulp: int = 1, what: str = ""):
    assert got.shape == want.shape, (got.shape, want.shape)
    d = np.abs(bf16_ordered(got) - bf16_ordered(want))
    worst = int(d.max()) if d.size else 0
    n_off = int(np.count_nonzero(d))
    print(f"[parity] {what}: {d.size} bf16 values, {n_off} off by >0 ulp, max {worst} ulp",
          flush=True)
    assert worst <= max_ulp, f"{what}: max {worst} ulp > {max_ulp} ({n_off} values differ)"
    return n_off, worst


def assert_f32_close(got: np.ndarray, want: np.ndarray, atol: float = 1e-5, what: str = ""):
    assert got.shape == want.shape, (got.shape, want.shape)
    g = got.astype(np.float64)
    w = want.astype(np.float64)
    err = np.abs(g - w)
    worst = float(err.max()) if err.size else 0.0
    n_off = int(np.count_nonzero(got.view(np.uint32) != want.view(np.uint32)))
    print(f"[parity] {what}: {err.size} f32 values, {n_off} not bit-equal, max abs {worst:.3g}",
          flush=True)
    assert worst <= atol, f"{what}: max abs error {worst} > {atol}"
    return n_off, worst


def assert_close(got, want, dtype: str, what: str = ""):
    if dtype == "bf16":
        return assert_bf16_close(got, want, 1, what)
    return assert_f32_close(got, want, 1e-5, what)
