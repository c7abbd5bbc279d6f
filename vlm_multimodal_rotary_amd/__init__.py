"""Python binding of the MI355X multimodal rotary library (libmrope.so).

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI in include/mrope.h.  Tensors are torch device tensors, token-major
[T, heads, D] with contiguous heads (any token stride); work is enqueued on
torch's current stream.  There is no CPU path: calling these without the
built library or without a GPU raises.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from ._lib import (DTYPE_BF16, DTYPE_F32, LAYOUTS, PRECISIONS, MropeError, check,  # noqa: F401
                   float_array, int_array, load)

__all__ = ["mrope_inv_freq", "mrope_axis_table", "mrope_cos_sin", "mrope_cos_sin_cache", "rms_norm",
           "apply_rotary_qk", "rmsnorm_mrope_qk", "mrope_decode_qk", "vision_qkv", "rope_index",
           "vision_pos_ids", "last_kernel", "MropeError", "load"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise MropeError(_lib.MROPE_EUNSUPPORTED, f"unsupported dtype {t.dtype}")


def _layout_code(layout) -> int:
    return LAYOUTS[layout] if isinstance(layout, str) else int(layout)


def _precision_code(precision) -> int:
    if isinstance(precision, str):
        if precision not in PRECISIONS:
            raise MropeError(_lib.MROPE_EINVAL, f"precision must be one of {list(PRECISIONS)}")
        return PRECISIONS[precision]
    return int(precision)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _heads_view(x, name):
    """Check a [T, heads, D] view with contiguous heads; return its token stride."""
    if x.dim() != 3:
        raise MropeError(_lib.MROPE_EINVAL, f"{name} must be [T, heads, D], got {tuple(x.shape)}")
    T, H, D = x.shape
    if x.numel() == 0:
        return H * D
    if D > 1 and x.stride(2) != 1:
        raise MropeError(_lib.MROPE_EINVAL, f"{name} last dim must be contiguous")
    if H > 1 and x.stride(1) != D:
        raise MropeError(_lib.MROPE_EINVAL, f"{name} heads must be contiguous (stride D)")
    return x.stride(0) if T > 1 else H * D


def mrope_inv_freq(dim: int, theta: float) -> np.ndarray:
    """theta^(-2i/dim) for i < dim/2 as float32 (host)."""
    out = np.zeros(max(1, dim // 2), dtype=np.float32)
    check(load().mrope_inv_freq(int(dim), float(theta),
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return out[: dim // 2]


def mrope_axis_table(half: int, section, layout) -> np.ndarray:
    """Axis (0/1/2) read by each frequency column j < half (host)."""
    out = np.zeros(max(1, half), dtype=np.uint8)
    sec = list(section) if section is not None else []
    check(load().mrope_axis_table(int(half), int_array(sec), len(sec), _layout_code(layout),
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))))
    return out[:half]


def mrope_cos_sin(pos, inv_freq, section, layout, rotary_dim: int, cos_out=None, sin_out=None):
    """cos, sin [T, rotary_dim] float32 on pos's device from int32 positions [n_axes, T]."""
    torch = _torch()
    n_axes, T = pos.shape
    if pos.dtype != torch.int32:
        raise MropeError(_lib.MROPE_EINVAL, "positions must be int32")
    if cos_out is None:
        cos_out = torch.empty((T, rotary_dim), dtype=torch.float32, device=pos.device)
    if sin_out is None:
        sin_out = torch.empty((T, rotary_dim), dtype=torch.float32, device=pos.device)
    sec = list(section) if section is not None else []
    inv = float_array(np.asarray(inv_freq, dtype=np.float32).reshape(-1))
    pos_stride = pos.stride(0) if n_axes > 1 else T
    if T > 0 and pos.stride(1) != 1:
        raise MropeError(_lib.MROPE_EINVAL, "positions must be contiguous along T")
    check(load().mrope_cos_sin(_ptr(pos), pos_stride, n_axes, T, inv, int_array(sec), len(sec),
                               _layout_code(layout), int(rotary_dim), _ptr(cos_out),
                               _ptr(sin_out), cos_out.stride(0) if T > 0 else rotary_dim,
                               _stream(pos)))
    return cos_out, sin_out


def rms_norm(x, w, eps: float, out=None):
    """Per-head RMSNorm of x [T, heads, D] with weight w [D] (dtype of x)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    T, H, D = x.shape
    check(load().rms_norm(_ptr(x), _heads_view(x, "x"), T, H, D, _ptr(w), float(eps),
                          _dtype_code(x), _ptr(out), _heads_view(out, "out"), _stream(x)))
    return out


def apply_rotary_qk(q, k, cos, sin, rotary_dim: int, q_out=None, k_out=None,
                    precision="exact"):
    """Split-half rotation of q [T, hq, D] and k [T, hk, D] with cos/sin [T, rotary_dim].

    precision: "exact" (one rounding of the binary32 result), "dtype" (cos/sin
    cast to the tensor dtype, every tensor operation rounded to it) or "fp32"
    (binary32 tensor operations, one cast at the end).
    """
    torch = _torch()
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    T, hq, D = q.shape
    hk = k.shape[1]
    check(load().apply_rotary_qk(_ptr(q), _heads_view(q, "q"), hq, _ptr(k), _heads_view(k, "k"),
                                 hk, T, D, int(rotary_dim), _ptr(cos), _ptr(sin),
                                 cos.stride(0) if T > 0 else rotary_dim, _dtype_code(q),
                                 _precision_code(precision), _ptr(q_out),
                                 _heads_view(q_out, "q_out"), _ptr(k_out),
                                 _heads_view(k_out, "k_out"), _stream(q)))
    return q_out, k_out


def mrope_cos_sin_cache(dim: int, theta: float, rows: int, device="cuda", out=None):
    """cos/sin table by position [rows, dim/2, 2] float32 (cos, sin) for
    inv_freq = mrope_inv_freq(dim, theta); dim = rotary_dim for text layouts,
    rotary_dim/2 for the vision layout."""
    torch = _torch()
    if out is None:
        out = torch.empty((rows, dim // 2, 2), dtype=torch.float32, device=device)
    check(load().mrope_cos_sin_cache(int(dim), float(theta), int(rows), _ptr(out), _stream(out)))
    return out


def rmsnorm_mrope_qk(q, k, pos, rotary_dim: int, theta: float, section, layout,
                     wq=None, wk=None, eps: float = 1e-6, q_out=None, k_out=None,
                     precision="exact", cs_cache=None):
    """Fused per-head RMSNorm (if weights are given) + MRoPE on q and k.

    pos: int32 [n_axes, T] on the device (3 axes for interleaved, 2 for
    vision_2d, len(section) for chunked).  precision as in apply_rotary_qk.
    cs_cache: optional table from mrope_cos_sin_cache (same theta), read for
    positions inside it.
    """
    torch = _torch()
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    T, hq, D = q.shape
    hk = k.shape[1]
    n_axes = pos.shape[0]
    if pos.dtype != torch.int32:
        raise MropeError(_lib.MROPE_EINVAL, "positions must be int32")
    if T > 0 and pos.stride(1) != 1:
        raise MropeError(_lib.MROPE_EINVAL, "positions must be contiguous along T")
    pos_stride = pos.stride(0) if n_axes > 1 else T
    sec = list(section) if section is not None else []
    check(load().rmsnorm_mrope_qk_cached(
        _ptr(q), _heads_view(q, "q"), hq, _ptr(k), _heads_view(k, "k"), hk, T, D,
        int(rotary_dim), _ptr(pos), pos_stride, n_axes, int_array(sec), len(sec),
        _layout_code(layout), float(theta), _ptr(wq), _ptr(wk), float(eps), _dtype_code(q),
        _precision_code(precision), _ptr(q_out), _heads_view(q_out, "q_out"), _ptr(k_out),
        _heads_view(k_out, "k_out"), _ptr(cs_cache), 0 if cs_cache is None else cs_cache.shape[0],
        _stream(q)))
    return q_out, k_out


def mrope_decode_qk(q, k, cache_len, rope_delta, new_tokens: int, rotary_dim: int, theta: float,
                    k_cache, wq=None, wk=None, eps: float = 1e-6, q_out=None,
                    precision="exact"):
    """One decode step: q, k [batch*new_tokens, heads, D]; cache_len and
    rope_delta (or None) int32 [batch] on the device; k_cache [batch,
    capacity, hk, D] receives the rotated k at rows cache_len[b] + i.
    precision as in apply_rotary_qk.  Returns q_out (k_cache is updated in
    place)."""
    torch = _torch()
    q_out = torch.empty_like(q) if q_out is None else q_out
    T, hq, D = q.shape
    hk = k.shape[1]
    batch = cache_len.shape[0]
    if cache_len.dtype != torch.int32 or (rope_delta is not None and rope_delta.dtype != torch.int32):
        raise MropeError(_lib.MROPE_EINVAL, "cache_len and rope_delta must be int32")
    if batch * new_tokens != T:
        raise MropeError(_lib.MROPE_EINVAL, "q rows must equal batch * new_tokens")
    if k_cache.dim() != 4 or k_cache.shape[2] != hk or k_cache.shape[3] != D:
        raise MropeError(_lib.MROPE_EINVAL, "k_cache must be [batch, capacity, hk, D]")
    if k_cache.stride(3) != 1 or (hk > 1 and k_cache.stride(2) != D):
        raise MropeError(_lib.MROPE_EINVAL, "k_cache rows must be contiguous")
    check(load().mrope_decode_qk(
        _ptr(q), _heads_view(q, "q"), hq, _ptr(k), _heads_view(k, "k"), hk, batch,
        int(new_tokens), D, int(rotary_dim), _ptr(cache_len), _ptr(rope_delta), float(theta),
        _ptr(wq), _ptr(wk), float(eps), _dtype_code(q), _precision_code(precision), _ptr(q_out),
        _heads_view(q_out, "q_out"),
        _ptr(k_cache), k_cache.stride(0), k_cache.stride(1), k_cache.shape[1], _stream(q)))
    return q_out


def vision_qkv(qkv, pos, rotary_dim: int, theta: float, q_out=None, k_out=None, v_out=None,
               precision="exact", head_major: bool = True, with_v: bool = True, cs_cache=None):
    """Vision rotary on a packed qkv [n, 3, heads, D] (token stride free, the
    rest contiguous): q and k rotated with the 2-D (row, col) positions pos
    int32 [2, n], v copied.  Outputs are per-head planes [heads, n, D] (or
    token-major [n, heads, D] with head_major=False)."""
    torch = _torch()
    if qkv.dim() != 4 or qkv.shape[1] != 3:
        raise MropeError(_lib.MROPE_EINVAL, "qkv must be [n, 3, heads, D]")
    n, _, H, D = qkv.shape
    if n > 0 and (qkv.stride(3) != 1 or qkv.stride(2) != D or qkv.stride(1) != H * D):
        raise MropeError(_lib.MROPE_EINVAL, "qkv must be contiguous within a token")
    shape = (H, n, D) if head_major else (n, H, D)
    q_out = torch.empty(shape, dtype=qkv.dtype, device=qkv.device) if q_out is None else q_out
    k_out = torch.empty(shape, dtype=qkv.dtype, device=qkv.device) if k_out is None else k_out
    if with_v and v_out is None:
        v_out = torch.empty(shape, dtype=qkv.dtype, device=qkv.device)
    for t in (q_out, k_out) + ((v_out,) if with_v else ()):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise MropeError(_lib.MROPE_EINVAL, f"outputs must be contiguous {shape}")
    hs, ts = (n * D, D) if head_major else (D, H * D)
    if pos.dtype != torch.int32 or (n > 0 and pos.stride(1) != 1):
        raise MropeError(_lib.MROPE_EINVAL, "positions must be int32, contiguous along n")
    check(load().mrope_vision_qkv(
        _ptr(qkv), qkv.stride(0) if n > 0 else 3 * H * D, n, H, D, int(rotary_dim), _ptr(pos),
        pos.stride(0) if n > 0 else n, float(theta), _dtype_code(qkv), _precision_code(precision),
        _ptr(q_out), _ptr(k_out), _ptr(v_out) if with_v else None, hs, ts, _ptr(cs_cache),
        0 if cs_cache is None else cs_cache.shape[0], _stream(qkv)))
    return q_out, k_out, (v_out if with_v else None)


def _int32_device(t, name, shape_len):
    torch = _torch()
    if t.dtype != torch.int32 or not t.is_contiguous() or t.dim() != shape_len:
        raise MropeError(_lib.MROPE_EINVAL, f"{name} must be a contiguous int32 tensor "
                                            f"with {shape_len} dims")
    return t


def _raise_on_status(status):
    s = int(status.item())
    if s:
        bits = [msg for bit, msg in _lib.POS_FLAGS.items() if s & bit]
        raise MropeError(_lib.MROPE_EINVAL, "position builder: " + "; ".join(bits))


def rope_index(mm_token_type, image_grid_thw=None, video_grid_thw=None, attention_mask=None,
               merge: int = 2, check: bool = True):
    """3-axis positions and rope_deltas of a batch (get_rope_index) on the GPU.

    mm_token_type, attention_mask: int32 [B, L] on the device (0 text, 1
    image, 2 video; mask nonzero = valid).  Grids: int32 [n, 3] (t, h, w)
    before merging.  Returns (pos int32 [3, B*L], rope_delta int32 [B],
    status int32 [1]); with check=True the call waits for the status word and
    raises on a nonzero one.
    """
    torch = _torch()
    _int32_device(mm_token_type, "mm_token_type", 2)
    B, L = mm_token_type.shape
    dev = mm_token_type.device
    if attention_mask is not None:
        _int32_device(attention_mask, "attention_mask", 2)
    ni = 0 if image_grid_thw is None else _int32_device(image_grid_thw, "image_grid_thw", 2).shape[0]
    nv = 0 if video_grid_thw is None else _int32_device(video_grid_thw, "video_grid_thw", 2).shape[0]
    lib = load()
    ws_bytes = lib.mrope_rope_index_workspace_size(B, L, ni, nv)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    pos = torch.empty((3, B * L), dtype=torch.int32, device=dev)
    delta = torch.empty(B, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    check_rc = lib.mrope_rope_index(_ptr(mm_token_type), _ptr(attention_mask), B, L,
                                    _ptr(image_grid_thw), ni, _ptr(video_grid_thw), nv, int(merge),
                                    _ptr(pos), B * L, _ptr(delta), _ptr(status), _ptr(workspace),
                                    ws_bytes, _stream(mm_token_type))
    _lib.check(check_rc)
    if check:
        _raise_on_status(status)
    return pos, delta, status


def vision_pos_ids(grid_thw, n_tokens: int, merge: int = 2, check: bool = True):
    """(row, col) of every vision patch (rot_pos_emb order): int32 [2, n_tokens]."""
    torch = _torch()
    _int32_device(grid_thw, "grid_thw", 2)
    pos = torch.empty((2, n_tokens), dtype=torch.int32, device=grid_thw.device)
    status = torch.empty(1, dtype=torch.int32, device=grid_thw.device)
    _lib.check(load().mrope_vision_pos_ids(_ptr(grid_thw), grid_thw.shape[0], int(merge),
                                           int(n_tokens), _ptr(pos), max(int(n_tokens), 1),
                                           _ptr(status), _stream(grid_thw)))
    if check:
        _raise_on_status(status)
    return pos, status


def last_kernel() -> str:
    """Name of the kernel the last q/k call on this thread launched
    ("qk_kernel", "flat_kernel" or "stage_kernel"; "" before any)."""
    return load().mrope_last_kernel().decode()
