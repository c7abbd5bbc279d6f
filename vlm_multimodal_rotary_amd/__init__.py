"""Python binding of the MI355X multimodal rotary library (libmrope.so).

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI in include/mrope.h.  Tensors are torch device tensors, token-major
[T, heads, D] with contiguous heads (any token stride); work is enqueued on
torch's current stream.  There is no CPU path: calling these without the
built library or without a GPU raises.

The C ABI sizes every buffer from the sizes passed to it, so the binding
checks each tensor against them before any pointer reaches the library:
device (every tensor on the same GPU), dtype, shape and layout.  A mismatch
raises MropeError(MROPE_EINVAL) and nothing is launched.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from ._lib import (DTYPE_BF16, DTYPE_F32, LAYOUTS, PRECISIONS, MropeError, check,  # noqa: F401
                   float_array, int_array, load)

__all__ = ["mrope_inv_freq", "mrope_axis_table", "mrope_cos_sin", "mrope_cos_sin_cache", "rms_norm",
           "apply_rotary_qk", "rmsnorm_mrope_qk", "mrope_decode_qk", "vision_qkv", "rope_index",
           "rope_index_into", "rope_index_workspace_size", "vision_pos_ids", "stream_copy",
           "last_kernel", "MropeError", "load"]


_TORCH = None


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch
        _TORCH = torch
    return _TORCH


def _einval(msg: str):
    return MropeError(_lib.MROPE_EINVAL, msg)


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
            raise _einval(f"precision must be one of {list(PRECISIONS)}")
        return PRECISIONS[precision]
    return int(precision)


def _ptr(t):
    return None if t is None else t.data_ptr()


_RAW_STREAM = None


def _stream(t):
    """torch's current stream on t's GPU (torch's raw-handle query when it has
    one: the stream object costs about 2 us per call)."""
    global _RAW_STREAM
    torch = _torch()
    if _RAW_STREAM is None:
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _RAW_STREAM:
        return ctypes.c_void_p(_RAW_STREAM(t.get_device()))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


# ---------------------------------------------------------------------------
# Argument checks (no launch happens before all of them pass)
# ---------------------------------------------------------------------------

# Device types whose tensors the library may be handed (a HIP device shows as
# "cuda" in torch).
_GPU_DEVICE_TYPES = ("cuda",)


def _on_gpu(t, name, device=None):
    """t must be a tensor on a GPU, and on `device` when given (a torch.device,
    or a tensor whose GPU it must share)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise _einval(f"{name} must be a torch tensor, got {type(t).__name__}")
    if not t.is_cuda and t.device.type not in _GPU_DEVICE_TYPES:
        raise _einval(f"{name} must be on the GPU, got device {t.device}")
    if device is not None:
        if isinstance(device, torch.Tensor):
            if t.get_device() != device.get_device():
                raise _einval(f"{name} is on {t.device}, the other tensors on {device.device}")
        elif t.device != device:
            raise _einval(f"{name} is on {t.device}, the other tensors on {device}")
    return t


def _like(t, name, ref, ref_name, shape=None):
    """t on ref's device with ref's dtype (and the given shape)."""
    _on_gpu(t, name, ref)
    if t.dtype != ref.dtype:
        raise _einval(f"{name} has dtype {t.dtype}, {ref_name} has {ref.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise _einval(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _heads_view(x, name):
    """Check a [T, heads, D] view with contiguous heads; return its token stride."""
    shape = x.shape
    if len(shape) != 3:
        raise _einval(f"{name} must be [T, heads, D], got {tuple(shape)}")
    T, H, D = shape
    if T == 0 or H == 0 or D == 0:
        return H * D
    st = x.stride()
    if D > 1 and st[2] != 1:
        raise _einval(f"{name} last dim must be contiguous")
    if H > 1 and st[1] != D:
        raise _einval(f"{name} heads must be contiguous (stride D)")
    return st[0] if T > 1 else H * D


def _weight(w, name, ref):
    """An RMSNorm weight: contiguous [D] with ref's dtype, on ref's device."""
    _like(w, name, ref, "q", (ref.shape[2],))
    if not w.is_contiguous():
        raise _einval(f"{name} must be contiguous")
    return w


def _int32_vec(t, name, device, length=None):
    torch = _torch()
    _on_gpu(t, name, device)
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
        raise _einval(f"{name} must be a contiguous int32 vector")
    if length is not None and t.shape[0] != length:
        raise _einval(f"{name} has {t.shape[0]} entries, expected {length}")
    return t


def _positions(pos, T, n_axes_expected, device):
    """int32 [n_axes, T] positions, contiguous along T; returns the axis stride."""
    torch = _torch()
    _on_gpu(pos, "pos", device)
    if pos.dtype != torch.int32:
        raise _einval("positions must be int32")
    if pos.dim() != 2 or pos.shape[1] != T:
        raise _einval(f"positions must be [n_axes, T={T}], got {tuple(pos.shape)}")
    if n_axes_expected is not None and pos.shape[0] != n_axes_expected:
        raise _einval(f"positions have {pos.shape[0]} axes, the layout reads {n_axes_expected}")
    st = pos.stride()
    if T > 1 and st[1] != 1:
        raise _einval("positions must be contiguous along T")
    return st[0] if pos.shape[0] > 1 else T


def _n_axes(layout, section):
    lay = _layout_code(layout)
    if lay == _lib.LAYOUT_INTERLEAVED:
        return 3
    if lay == _lib.LAYOUT_VISION_2D:
        return 2
    return len(list(section)) if section is not None else None


def _cs_table(t, name, T, rotary_dim, device):
    """A cos/sin table: float32 [T, >= rotary_dim], last dim contiguous."""
    torch = _torch()
    _on_gpu(t, name, device)
    if t.dtype != torch.float32 or t.dim() != 2 or t.shape[0] != T or t.shape[1] < rotary_dim:
        raise _einval(f"{name} must be float32 [T={T}, >= {rotary_dim}], got "
                      f"{t.dtype} {tuple(t.shape)}")
    if t.numel() > 0 and t.stride(1) != 1:
        raise _einval(f"{name} must be contiguous along its last dim")
    return t.stride(0) if T > 1 else max(rotary_dim, t.shape[1])


def _cos_sin_cache(cache, n_freq, device):
    """A cos/sin cache: contiguous float32 [rows, n_freq, 2]; returns rows."""
    torch = _torch()
    if cache is None:
        return 0
    _on_gpu(cache, "cs_cache", device)
    if (cache.dtype != torch.float32 or cache.dim() != 3 or cache.shape[1] != n_freq
            or cache.shape[2] != 2 or not cache.is_contiguous()):
        raise _einval(f"cs_cache must be a contiguous float32 [rows, {n_freq}, 2] table, got "
                      f"{cache.dtype} {tuple(cache.shape)}")
    return cache.shape[0]


def _qk_pair(q, k, q_out, k_out):
    """q [T, hq, D] and k [T, hk, D] of one dtype on one GPU; outputs of the
    same shapes (created when None).  Returns (q_out, k_out, T, hq, hk, D)."""
    torch = _torch()
    _on_gpu(q, "q")
    if q.dim() != 3:
        raise _einval(f"q must be [T, heads, D], got {tuple(q.shape)}")
    T, hq, D = q.shape
    _like(k, "k", q, "q")
    if k.dim() != 3 or k.shape[0] != T or k.shape[2] != D:
        raise _einval(f"k must be [T={T}, heads, D={D}], got {tuple(k.shape)}")
    hk = k.shape[1]
    q_out = torch.empty_like(q) if q_out is None else _like(q_out, "q_out", q, "q", q.shape)
    k_out = torch.empty_like(k) if k_out is None else _like(k_out, "k_out", k, "k", k.shape)
    return q_out, k_out, T, hq, hk, D


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------

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
    _on_gpu(pos, "pos")
    if pos.dim() != 2:
        raise _einval(f"positions must be [n_axes, T], got {tuple(pos.shape)}")
    n_axes, T = pos.shape
    pos_stride = _positions(pos, T, None, pos.device)
    if cos_out is None:
        cos_out = torch.empty((T, rotary_dim), dtype=torch.float32, device=pos.device)
    if sin_out is None:
        sin_out = torch.empty((T, rotary_dim), dtype=torch.float32, device=pos.device)
    cs_ts = _cs_table(cos_out, "cos_out", T, rotary_dim, pos.device)
    if _cs_table(sin_out, "sin_out", T, rotary_dim, pos.device) != cs_ts:
        raise _einval("cos_out and sin_out must have the same token stride")
    sec = list(section) if section is not None else []
    inv = np.asarray(inv_freq, dtype=np.float32).reshape(-1)
    half = int(rotary_dim) // 2
    need = half // 2 if _layout_code(layout) == _lib.LAYOUT_VISION_2D else half
    if inv.shape[0] < need:
        raise _einval(f"inv_freq has {inv.shape[0]} entries, the layout reads {need}")
    check(load().mrope_cos_sin(_ptr(pos), pos_stride, n_axes, T, float_array(inv),
                               int_array(sec), len(sec), _layout_code(layout), int(rotary_dim),
                               _ptr(cos_out), _ptr(sin_out), cs_ts, _stream(pos)))
    return cos_out, sin_out


def rms_norm(x, w, eps: float, out=None):
    """Per-head RMSNorm of x [T, heads, D] with weight w [D] (dtype of x)."""
    torch = _torch()
    _on_gpu(x, "x")
    xs = _heads_view(x, "x")
    T, H, D = x.shape
    _weight(w, "w", x)
    out = torch.empty_like(x) if out is None else _like(out, "out", x, "x", x.shape)
    check(load().rms_norm(_ptr(x), xs, T, H, D, _ptr(w), float(eps), _dtype_code(x), _ptr(out),
                          _heads_view(out, "out"), _stream(x)))
    return out


def apply_rotary_qk(q, k, cos, sin, rotary_dim: int, q_out=None, k_out=None,
                    precision="exact"):
    """Split-half rotation of q [T, hq, D] and k [T, hk, D] with cos/sin [T, rotary_dim].

    precision: "exact" (one rounding of the binary32 result), "dtype" (cos/sin
    cast to the tensor dtype, every tensor operation rounded to it) or "fp32"
    (binary32 tensor operations, one cast at the end).
    """
    q_out, k_out, T, hq, hk, D = _qk_pair(q, k, q_out, k_out)
    cs_ts = _cs_table(cos, "cos", T, rotary_dim, q.device)
    if _cs_table(sin, "sin", T, rotary_dim, q.device) != cs_ts:
        raise _einval("cos and sin must have the same token stride")
    check(load().apply_rotary_qk(_ptr(q), _heads_view(q, "q"), hq, _ptr(k), _heads_view(k, "k"),
                                 hk, T, D, int(rotary_dim), _ptr(cos), _ptr(sin), cs_ts,
                                 _dtype_code(q), _precision_code(precision), _ptr(q_out),
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
    if _cos_sin_cache(out, dim // 2, out.device if isinstance(out, torch.Tensor) else None) != rows:
        raise _einval(f"out must have {rows} rows")
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
    q_out, k_out, T, hq, hk, D = _qk_pair(q, k, q_out, k_out)
    pos_stride = _positions(pos, T, _n_axes(layout, section), q)
    n_axes = pos.shape[0]
    if (wq is None) != (wk is None):
        raise _einval("wq and wk must both be given or both be None")
    if wq is not None:
        _weight(wq, "wq", q)
        _weight(wk, "wk", q)
    half = int(rotary_dim) // 2
    n_freq = half // 2 if _layout_code(layout) == _lib.LAYOUT_VISION_2D else half
    rows = _cos_sin_cache(cs_cache, n_freq, q)
    sec = list(section) if section is not None else []
    check(load().rmsnorm_mrope_qk_cached(
        _ptr(q), _heads_view(q, "q"), hq, _ptr(k), _heads_view(k, "k"), hk, T, D,
        int(rotary_dim), _ptr(pos), pos_stride, n_axes, int_array(sec), len(sec),
        _layout_code(layout), float(theta), _ptr(wq), _ptr(wk), float(eps), _dtype_code(q),
        _precision_code(precision), _ptr(q_out), _heads_view(q_out, "q_out"), _ptr(k_out),
        _heads_view(k_out, "k_out"), _ptr(cs_cache), rows, _stream(q)))
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
    _on_gpu(q, "q")
    if q.dim() != 3:
        raise _einval(f"q must be [T, heads, D], got {tuple(q.shape)}")
    T, hq, D = q.shape
    _like(k, "k", q, "q")
    if k.dim() != 3 or k.shape[0] != T or k.shape[2] != D:
        raise _einval(f"k must be [T={T}, heads, D={D}], got {tuple(k.shape)}")
    hk = k.shape[1]
    q_out = torch.empty_like(q) if q_out is None else _like(q_out, "q_out", q, "q", q.shape)
    _on_gpu(cache_len, "cache_len", q)
    if cache_len.dim() != 1:
        raise _einval("cache_len must be an int32 vector [batch]")
    batch = cache_len.shape[0]
    _int32_vec(cache_len, "cache_len", q)
    if rope_delta is not None:
        _int32_vec(rope_delta, "rope_delta", q, batch)
    if batch * new_tokens != T:
        raise _einval("q rows must equal batch * new_tokens")
    _like(k_cache, "k_cache", q, "q")
    if k_cache.dim() != 4 or k_cache.shape[0] != batch or k_cache.shape[2] != hk \
            or k_cache.shape[3] != D:
        raise _einval(f"k_cache must be [batch={batch}, capacity, hk={hk}, D={D}], got "
                      f"{tuple(k_cache.shape)}")
    if k_cache.stride(3) != 1 or (hk > 1 and k_cache.stride(2) != D):
        raise _einval("k_cache rows must be contiguous")
    if (wq is None) != (wk is None):
        raise _einval("wq and wk must both be given or both be None")
    if wq is not None:
        _weight(wq, "wq", q)
        _weight(wk, "wk", q)
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
    _on_gpu(qkv, "qkv")
    if qkv.dim() != 4 or qkv.shape[1] != 3:
        raise _einval("qkv must be [n, 3, heads, D]")
    n, _, H, D = qkv.shape
    if n > 0 and (qkv.stride(3) != 1 or qkv.stride(2) != D or qkv.stride(1) != H * D):
        raise _einval("qkv must be contiguous within a token")
    shape = (H, n, D) if head_major else (n, H, D)
    q_out = torch.empty(shape, dtype=qkv.dtype, device=qkv.device) if q_out is None else q_out
    k_out = torch.empty(shape, dtype=qkv.dtype, device=qkv.device) if k_out is None else k_out
    if with_v and v_out is None:
        v_out = torch.empty(shape, dtype=qkv.dtype, device=qkv.device)
    for nm, t in (("q_out", q_out), ("k_out", k_out)) + ((("v_out", v_out),) if with_v else ()):
        _like(t, nm, qkv, "qkv", shape)
        if not t.is_contiguous():
            raise _einval(f"{nm} must be contiguous {shape}")
    hs, ts = (n * D, D) if head_major else (D, H * D)
    pos_stride = _positions(pos, n, 2, qkv.device)
    rows = _cos_sin_cache(cs_cache, int(rotary_dim) // 4, qkv.device)
    check(load().mrope_vision_qkv(
        _ptr(qkv), qkv.stride(0) if n > 0 else 3 * H * D, n, H, D, int(rotary_dim), _ptr(pos),
        pos_stride, float(theta), _dtype_code(qkv), _precision_code(precision),
        _ptr(q_out), _ptr(k_out), _ptr(v_out) if with_v else None, hs, ts, _ptr(cs_cache),
        rows, _stream(qkv)))
    return q_out, k_out, (v_out if with_v else None)


def _int32_device(t, name, shape_len, device=None, cols=None):
    torch = _torch()
    _on_gpu(t, name, device)
    if t.dtype != torch.int32 or not t.is_contiguous() or t.dim() != shape_len:
        raise _einval(f"{name} must be a contiguous int32 tensor with {shape_len} dims")
    if cols is not None and t.shape[-1] != cols:
        raise _einval(f"{name} must have {cols} columns, got {tuple(t.shape)}")
    return t


def _raise_on_status(status):
    s = int(status.item())
    if s:
        bits = [msg for bit, msg in _lib.POS_FLAGS.items() if s & bit]
        raise _einval("position builder: " + "; ".join(bits))


def _rope_index_inputs(mm_token_type, image_grid_thw, video_grid_thw, attention_mask):
    _int32_device(mm_token_type, "mm_token_type", 2)
    B, L = mm_token_type.shape
    dev = mm_token_type.device
    if attention_mask is not None:
        _int32_device(attention_mask, "attention_mask", 2, dev)
        if tuple(attention_mask.shape) != (B, L):
            raise _einval(f"attention_mask must be [{B}, {L}]")
    ni = 0 if image_grid_thw is None else _int32_device(image_grid_thw, "image_grid_thw", 2, dev,
                                                         3).shape[0]
    nv = 0 if video_grid_thw is None else _int32_device(video_grid_thw, "video_grid_thw", 2, dev,
                                                         3).shape[0]
    return B, L, ni, nv, dev


def rope_index_workspace_size(batch: int, seq_len: int, n_images: int, n_videos: int) -> int:
    """Bytes of device workspace rope_index_into needs for these sizes."""
    return int(load().mrope_rope_index_workspace_size(int(batch), int(seq_len), int(n_images),
                                                      int(n_videos)))


def rope_index_into(mm_token_type, attention_mask, image_grid_thw, video_grid_thw, merge: int,
                    pos, rope_delta, status, workspace):
    """mrope_rope_index into caller buffers: pos int32 [3, B*L], rope_delta
    int32 [B], status int32 [1], workspace uint8 of at least
    rope_index_workspace_size bytes.  Does not wait for the status word."""
    torch = _torch()
    B, L, ni, nv, dev = _rope_index_inputs(mm_token_type, image_grid_thw, video_grid_thw,
                                           attention_mask)
    _int32_device(pos, "pos", 2, dev)
    if pos.shape[0] != 3 or pos.shape[1] != B * L:
        raise _einval(f"pos must be [3, {B * L}]")
    _int32_vec(rope_delta, "rope_delta", dev, B)
    _int32_vec(status, "status", dev, 1)
    _on_gpu(workspace, "workspace", dev)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise _einval("workspace must be a contiguous uint8 tensor")
    check(load().mrope_rope_index(_ptr(mm_token_type), _ptr(attention_mask), B, L,
                                  _ptr(image_grid_thw), ni, _ptr(video_grid_thw), nv, int(merge),
                                  _ptr(pos), B * L, _ptr(rope_delta), _ptr(status),
                                  _ptr(workspace), workspace.numel(), _stream(mm_token_type)))


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
    B, L, ni, nv, dev = _rope_index_inputs(mm_token_type, image_grid_thw, video_grid_thw,
                                           attention_mask)
    ws_bytes = rope_index_workspace_size(B, L, ni, nv)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    pos = torch.empty((3, B * L), dtype=torch.int32, device=dev)
    delta = torch.empty(B, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    rope_index_into(mm_token_type, attention_mask, image_grid_thw, video_grid_thw, merge, pos,
                    delta, status, workspace)
    if check:
        _raise_on_status(status)
    return pos, delta, status


def vision_pos_ids(grid_thw, n_tokens: int, merge: int = 2, check: bool = True):
    """(row, col) of every vision patch (rot_pos_emb order): int32 [2, n_tokens]."""
    torch = _torch()
    _int32_device(grid_thw, "grid_thw", 2, None, 3)
    pos = torch.empty((2, n_tokens), dtype=torch.int32, device=grid_thw.device)
    status = torch.empty(1, dtype=torch.int32, device=grid_thw.device)
    _lib.check(load().mrope_vision_pos_ids(_ptr(grid_thw), grid_thw.shape[0], int(merge),
                                           int(n_tokens), _ptr(pos), max(int(n_tokens), 1),
                                           _ptr(status), _stream(grid_thw)))
    if check:
        _raise_on_status(status)
    return pos, status


def stream_copy(src, dst):
    """Plain streaming device copy of src's bytes into dst (mrope_stream_copy):
    the copy rate the benchmark reports beside each kernel.  Both contiguous,
    on one GPU, with the same byte size (a multiple of 16)."""
    _on_gpu(src, "src")
    _on_gpu(dst, "dst", src.device)
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise _einval("src and dst must be contiguous")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise _einval("src and dst must have the same byte size")
    check(load().mrope_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(src)))
    return dst


def last_kernel() -> str:
    """Name of the kernel the last q/k call on this thread launched
    ("qk_kernel", "qk_pipe_kernel", "flat_kernel" or "stage_kernel"; "" before
    any)."""
    return load().mrope_last_kernel().decode()
