"""CPU oracle for multimodal rotary position embedding (MRoPE) with an optional
per-head RMSNorm in front of it.

TEST INFRASTRUCTURE ONLY.  This module defines what the GPU path must compute.
It is imported by the test suite, by the entry point's smoke check and by the
benchmark's CPU-baseline leg, and by nothing else.  It shares no code with the
HIP library and imports nothing from it.

Everything is evaluated in float64 with the rounding points written out:

* ``fl32(v)``  round-to-nearest-even of a real (held in float64) to binary32;
* ``bf(v)``    round-to-nearest-even of a binary32 to bfloat16.

Sources (the pages, cited by page title and section):

* "Interleaved Rotary Position Embedding" (taking-lying-flat blog, RoPE post):
  the ``inv_freq`` listing under "RoPE", the ``rotate_half`` /
  ``apply_rotary_pos_emb`` listing with partial rotary, the
  ``recomposition_frequencies`` axis selection under "Interleaved MRoPE",
  and the ``get_rope_index`` position builder.
* "M01 · RMSNorm and multimodal RoPE (interleaved / chunked)" (nano-vllm-omni
  drills): the numeric conventions of RMSNorm, the interleaved rule, the
  chunked layout table, the shape trace and the worked numbers.
* "Qwen3-VL" annotated source (frankmowj blog): ``Qwen3VLTextRotaryEmbedding``
  (fp32 angles, ``cat(f, f)``, cos/sin), ``apply_rotary_pos_emb_vision`` and
  ``rot_pos_emb`` (the 2-D vision variant).
* cortiq-engine ``qwen3vis.rs``: ``rope_angles`` (18 row + 18 column
  frequencies with exponent denominator 36) and ``attention`` (split-half
  rotation over the whole 72-dim head).

Readings where the pages leave a step open:

1. ``inv_freq`` is the binary32 value nearest to theta**(-2i/d), evaluated in
   float64 and rounded once.
2. The angle is the binary32 product of float32(position) and the binary32
   ``inv_freq`` entry, rounded once (the Qwen3-VL listing forces float32 with
   autocast off).
3. cos/sin of that binary32 angle are evaluated in float64 and rounded once to
   binary32; ``attention_scaling`` is 1 for the default rope type.
4. RMSNorm: ``r = fl32(1/sqrt(sum(x^2)/D + eps))`` with the sum taken exactly
   (``math.fsum``), ``n = fl32(x*r)``, then the cast back to the input dtype,
   then the weight multiply, then the cast to the input dtype again.
5. The rotation of a bf16 tensor uses the binary32 cos/sin (as the vision
   listing does) and rounds once: ``bf(fl32(exact))``.  The products are exact
   in float64 and the sum is rounded once to float64 before that.
6. An interleaved section whose rule would give an axis fewer columns than its
   section entry is rejected (assertion), as is a section that does not sum to
   rotary_dim/2.
7. Rotation precision "dtype" (M01 drill shape trace, the apply_rotary row,
   and its broadcast note: for bf16 input cos/sin are cast to x.dtype before
   the multiplies, as HF does): every tensor operation of
   ``x*cos + rotate_half(x)*sin`` rounds to x.dtype, and a bf16 operation
   computes in binary32 before it rounds (the tensor arithmetic of PyTorch).
   So ``bf(fl32(bf(x*c_b) + bf(-x2*s_b)))`` with ``c_b = bf(cos)``.
8. Rotation precision "fp32" (Qwen3-VL ``apply_rotary_pos_emb_vision``):
   q/k and cos/sin are upcast to binary32, each product and the sum rounds
   to binary32, and the result is cast to x.dtype once at the end.  For
   binary32 input "dtype" and "fp32" are the same arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

LAYOUT_CHUNKED = 0
LAYOUT_INTERLEAVED = 1
LAYOUT_VISION_2D = 2

_LAYOUT_NAMES = {"chunked": LAYOUT_CHUNKED, "interleaved": LAYOUT_INTERLEAVED,
                 "vision_2d": LAYOUT_VISION_2D}


def layout_id(layout) -> int:
    if isinstance(layout, str):
        return _LAYOUT_NAMES[layout]
    return int(layout)


# ---------------------------------------------------------------------------
# Rounding helpers
# ---------------------------------------------------------------------------

def fl32(v):
    """Round float64 value(s) to the nearest binary32 (ties to even)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def bf16_bits_to_f64(bits):
    """Decode bfloat16 bit patterns (uint16) to float64; exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x):
    """Round binary32 value(s) to bfloat16 bit patterns, nearest, ties to even.

    The low 16 bits of the binary32 pattern are the discarded part: round up
    when they exceed half of a bf16 unit, or equal it and the kept part is
    odd.  A carry out of the mantissa moves to the next binade (or to
    infinity), which is the correct rounding.  NaN stays NaN (quiet bit set).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    kept = (u >> np.uint32(16)).astype(np.uint32)
    dropped = u & np.uint32(0xFFFF)
    half = np.uint32(0x8000)
    up = (dropped > half) | ((dropped == half) & ((kept & np.uint32(1)) == np.uint32(1)))
    out = kept + up.astype(np.uint32)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    out = np.where(nan, kept | np.uint32(0x0040), out)
    return out.astype(np.uint16)


def bf(v):
    """fl32 then round to bfloat16; returns the bf16 value as float64."""
    return bf16_bits_to_f64(f32_to_bf16_bits(fl32(v)))


def decode(x, dtype: str):
    """Stored representation -> exact float64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def encode(v, dtype: str):
    """Float64 values -> stored representation, rounding as the dtype requires.

    bf16: bf(fl32(v)) as uint16 bit patterns; f32: fl32(v).
    """
    if dtype == "bf16":
        return f32_to_bf16_bits(fl32(v))
    if dtype == "f32":
        return fl32(v)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Frequencies and the per-column axis table
# ---------------------------------------------------------------------------

def inv_freq(dim: int, theta: float) -> np.ndarray:
    """``inv[i] = theta ** (-2 i / dim)`` for ``i < dim/2``, as binary32.

    RoPE post, "RoPE" section (the inv_freq listing: frequencies from
    ``arange(0, dim, 2) / dim``); M01 drill, ``rope_inv_freq`` and its
    worked values.  ``dim`` is the rotary dimension for text layouts (the
    partial-rotary listing computes frequencies over the rotated slice only)
    and half the head dimension for the vision layout (qwen3vis.rs
    ``rope_angles``).
    """
    assert dim > 0 and dim % 2 == 0 and theta > 0
    return np.array([np.float32(float(theta) ** (-(2.0 * i) / dim)) for i in range(dim // 2)],
                    dtype=np.float32)


def axis_table(half: int, section, layout) -> np.ndarray:
    """Axis (0 = T/row, 1 = H/col, 2 = W) used by each frequency column j < half.

    * interleaved (M01 drill rule; RoPE post ``recomposition_frequencies``;
      Qwen3-VL ``apply_interleaved_mrope``): column j takes H when
      ``j % 3 == 1 and j < 3*s_h``, W when ``j % 3 == 2 and j < 3*s_w``,
      T otherwise.
    * chunked (M01 drill layout table, acos probe step 3): consecutive ranges
      of s_t, s_h, s_w columns; each axis supplies the *same* column range.
    * vision 2-D (qwen3vis.rs ``rope_angles``; Qwen3-VL ``rot_pos_emb``):
      the first half/2 columns read the row, the rest the column.
    """
    lay = layout_id(layout)
    axis = np.zeros(half, dtype=np.uint8)
    if lay == LAYOUT_INTERLEAVED:
        s = list(section)
        assert len(s) == 3 and sum(s) == half, "section must have 3 entries summing to half"
        for j in range(half):
            if j % 3 == 1 and j < 3 * s[1]:
                axis[j] = 1
            elif j % 3 == 2 and j < 3 * s[2]:
                axis[j] = 2
        counts = [int(np.sum(axis == a)) for a in range(3)]
        assert counts == s, f"interleaved rule gives {counts} columns, section says {s}"
    elif lay == LAYOUT_CHUNKED:
        s = list(section)
        assert 1 <= len(s) <= 3 and sum(s) == half and min(s) >= 0
        j = 0
        for a, n in enumerate(s):
            axis[j:j + n] = a
            j += n
    elif lay == LAYOUT_VISION_2D:
        assert half % 2 == 0
        axis[half // 2:] = 1
    else:
        raise ValueError(layout)
    return axis


def column_inv(half: int, theta: float, layout, rotary_dim: int) -> np.ndarray:
    """The binary32 inverse frequency that column j < half multiplies.

    Text layouts use ``inv_freq(rotary_dim)`` (one entry per column).  The
    vision layout uses ``inv_freq(half)`` (half/2 entries) twice: once for the
    row angles, once for the column angles.
    """
    lay = layout_id(layout)
    if lay == LAYOUT_VISION_2D:
        inv = inv_freq(half, theta)
        return np.array([inv[j % (half // 2)] for j in range(half)], dtype=np.float32)
    return inv_freq(rotary_dim, theta)


def n_axes_of(layout, section) -> int:
    lay = layout_id(layout)
    if lay == LAYOUT_INTERLEAVED:
        return 3
    if lay == LAYOUT_VISION_2D:
        return 2
    return len(section)


# ---------------------------------------------------------------------------
# Angles and cos/sin
# ---------------------------------------------------------------------------

def angles(pos, axis, invc) -> np.ndarray:
    """``a[t, j] = fl32(float32(pos[axis[j], t]) * invc[j])``, shape [T, half].

    M01 drill shape trace rows 4-5 (broadcast product, then pick one axis per
    column, a copy with no new arithmetic); Qwen3-VL text rotary ``forward``
    (float32 with autocast disabled).  The product of two binary32 values is
    exact in float64, so ``fl32`` of it is the binary32 product.
    """
    pos = np.asarray(pos)
    p32 = pos.astype(np.float32).astype(np.float64)          # [n_axes, T]
    picked = p32[np.asarray(axis, dtype=np.int64), :].T       # [T, half]
    return fl32(picked * np.asarray(invc, dtype=np.float32).astype(np.float64)[None, :])


def cos_sin_half(pos, axis, invc):
    """fl32(cos(a)), fl32(sin(a)) for every (token, column < half)."""
    a = angles(pos, axis, invc).astype(np.float64)
    return fl32(np.cos(a)), fl32(np.sin(a))


def mrope_cos_sin(pos, inv, section, layout, rotary_dim):
    """cos, sin of shape [T, rotary_dim], binary32, columns j and j+half equal.

    M01 drill ``mrope_cos_sin(inv_freq, positions[3,T], section, interleaved)``
    and shape-trace rows 5-7: select an axis per column, ``cat([f, f])``, then
    cos/sin.  ``inv`` is taken as given (binary32, one entry per column for
    text layouts, half/2 entries for the vision layout) so the acos probe with
    ``inv = ones`` can run.
    """
    half = rotary_dim // 2
    axis = axis_table(half, section, layout)
    inv = np.asarray(inv, dtype=np.float32)
    if layout_id(layout) == LAYOUT_VISION_2D:
        invc = np.array([inv[j % (half // 2)] for j in range(half)], dtype=np.float32)
    else:
        assert inv.shape == (half,)
        invc = inv
    c, s = cos_sin_half(pos, axis, invc)
    return np.concatenate([c, c], axis=1), np.concatenate([s, s], axis=1)


def cos_sin_cache(dim: int, theta: float, rows: int) -> np.ndarray:
    """cos/sin by position value, [rows, dim/2, 2] binary32 (cos, sin).

    RoPE post, "method 2" under the Qwen3-VL rotary: the binary32 outer
    product of arange(rows) and inv_freq, whose cos/sin are gathered by
    position afterwards; the angle fl32(p * inv[i]) is the same product the
    per-token path forms, so the gathered values equal ``cos_sin_half``'s.
    """
    inv = inv_freq(dim, theta).astype(np.float64)
    p = np.arange(rows, dtype=np.float64)
    ang = fl32(p[:, None] * inv[None, :]).astype(np.float64)
    return np.stack([fl32(np.cos(ang)), fl32(np.sin(ang))], axis=-1)


# ---------------------------------------------------------------------------
# RMSNorm and rotation
# ---------------------------------------------------------------------------

def rms_scale(row, eps: float) -> float:
    """``r = fl32(1 / sqrt(sum(x^2)/D + eps))`` for one row, eps as binary32.

    The squares of bf16/fp32 values are exact in float64 and ``math.fsum``
    rounds their sum once, so r is the binary32 value of the float64
    evaluation of the M01 drill formula (eps inside the square root).
    """
    row = np.asarray(row, dtype=np.float64)
    ssq = math.fsum(row * row)
    eps64 = float(np.float32(eps))
    return float(np.float32(1.0 / math.sqrt(ssq / row.shape[0] + eps64)))


def rms_norm_values(x, w, eps: float, dtype: str):
    """Per-row RMSNorm over the last axis; returns float64 values on the dtype grid.

    M01 drill numeric conventions: ``y = w * x / sqrt(mean(x^2) + eps)``,
    normalised in fp32, cast back to the input dtype, *then* multiplied by
    the weight; eps sits inside the square root.  ``x`` and ``w`` are exact
    float64 values of the stored inputs.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    D = x.shape[-1]
    rows = x.reshape(-1, D)
    out = np.empty_like(rows)
    for i in range(rows.shape[0]):
        row = rows[i]
        r = rms_scale(row, eps)
        n = fl32(row * r).astype(np.float64)    # x*r is exact in float64
        if dtype == "bf16":
            out[i] = bf(bf(n) * w)              # bf16*bf16 is exact in binary32
        else:
            out[i] = fl32(n * w)
    return out.reshape(x.shape)


def rotate_half(x):
    """``rotate_half([a, b]) = [-b, a]`` over the last axis (RoPE post listing)."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    return np.concatenate([-x[..., h:], x[..., :h]], axis=-1)


def apply_rotary_values(y, cos, sin, rotary_dim: int):
    """``y_rot * cos + rotate_half(y_rot) * sin`` on the first rotary_dim dims,
    the rest passed through (RoPE post ``apply_rotary_pos_emb`` with partial
    rotary; M01 drill ``apply_rotary`` with cos/sin broadcast over heads).

    ``y`` is [T, heads, D] float64; ``cos``/``sin`` are [T, rotary_dim]
    binary32 tables.  Returns float64 values, each the float64-rounded exact
    result (products of a bf16/fp32 value and a binary32 value are exact in
    float64, so only the sum rounds).  Pass-through dims are copied.
    """
    y = np.asarray(y, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float32).astype(np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float32).astype(np.float64)[:, None, :]
    rot = y[..., :rotary_dim]
    out = y.copy()
    out[..., :rotary_dim] = rot * c + rotate_half(rot) * s
    return out


PRECISIONS = ("exact", "dtype", "fp32")


def apply_rotary_tensor_ops(y, cos, sin, rotary_dim: int, dtype: str, precision: str):
    """The rotation as a sequence of tensor operations, each rounded.

    precision "dtype": cos/sin cast to x.dtype first, then the two products
    and their sum each rounded to x.dtype (M01 drill, apply_rotary row of the
    shape trace).  precision "fp32": cos/sin and y in binary32, the products
    and the sum each rounded to binary32 (Qwen3-VL vision rotary); the cast
    to x.dtype happens when the result is encoded.

    ``y`` holds exact float64 values of the stored input; products of two
    values of at most 24 significant bits are exact in float64, and the sum
    of two binary32 values rounded in float64 and then to binary32 equals the
    sum rounded once (53 >= 2*24 + 2), so ``fl32`` after the float64
    operation is the binary32 operation.
    """
    if precision == "dtype":
        rnd = bf if dtype == "bf16" else fl32
    elif precision == "fp32":
        rnd = fl32
    else:
        raise ValueError(precision)
    y = np.asarray(y, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float32).astype(np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float32).astype(np.float64)[:, None, :]
    if precision == "dtype":
        c = np.asarray(rnd(c), dtype=np.float64)
        s = np.asarray(rnd(s), dtype=np.float64)
    rot = y[..., :rotary_dim]
    p1 = np.asarray(rnd(rot * c), dtype=np.float64)
    p2 = np.asarray(rnd(rotate_half(rot) * s), dtype=np.float64)
    out = y.copy()
    out[..., :rotary_dim] = rnd(p1 + p2)
    return out


def rotary_values(y, cos, sin, rotary_dim: int, dtype: str, precision: str = "exact"):
    """The rotation in the requested precision (float64 values; encode rounds)."""
    if precision == "exact":
        return apply_rotary_values(y, cos, sin, rotary_dim)
    return apply_rotary_tensor_ops(y, cos, sin, rotary_dim, dtype, precision)


# ---------------------------------------------------------------------------
# Entry points mirroring the library's operations (stored representations)
# ---------------------------------------------------------------------------

def rms_norm(x, w, eps: float, dtype: str):
    """RMSNorm of x[T, heads, D] with weight w[D] shared by all heads."""
    y = rms_norm_values(decode(x, dtype), decode(w, dtype), eps, dtype)
    return encode(y, dtype)


def apply_rotary_qk(q, k, cos, sin, rotary_dim: int, dtype: str, precision: str = "exact"):
    """Rotate q[T, hq, D] and k[T, hk, D] with the same per-token cos/sin."""
    qo = encode(rotary_values(decode(q, dtype), cos, sin, rotary_dim, dtype, precision), dtype)
    ko = encode(rotary_values(decode(k, dtype), cos, sin, rotary_dim, dtype, precision), dtype)
    return qo, ko


def rmsnorm_mrope_qk(q, k, pos, *, rotary_dim: int, theta: float, section, layout,
                     wq=None, wk=None, eps: float = 0.0, dtype: str = "bf16",
                     precision: str = "exact"):
    """The fused hot path: optional per-head RMSNorm, then MRoPE, on q and k.

    The RMSNorm output is on the dtype grid (cast back) before the rotation,
    exactly as the unfused composition rms_norm -> apply_rotary would give.
    Positions ``pos`` are [n_axes, T] integers.
    """
    half = rotary_dim // 2
    axis = axis_table(half, section, layout)
    invc = column_inv(half, theta, layout, rotary_dim)
    c, s = cos_sin_half(pos, axis, invc)
    cos = np.concatenate([c, c], axis=1)
    sin = np.concatenate([s, s], axis=1)
    qv, kv = decode(q, dtype), decode(k, dtype)
    if wq is not None:
        qv = rms_norm_values(qv, decode(wq, dtype), eps, dtype)
        kv = rms_norm_values(kv, decode(wk, dtype), eps, dtype)
    qo = encode(rotary_values(qv, cos, sin, rotary_dim, dtype, precision), dtype)
    ko = encode(rotary_values(kv, cos, sin, rotary_dim, dtype, precision), dtype)
    return qo, ko


# ---------------------------------------------------------------------------
# Vision tower: packed qkv to per-head planes
# ---------------------------------------------------------------------------

def vision_qkv(qkv, pos, *, rotary_dim: int, theta: float, dtype: str = "f32",
               precision: str = "exact"):
    """The vision attention's rotary step on a packed projection.

    cortiq-engine ``qwen3vis.rs`` (``attention``): the projection is
    [n, 3, heads, hd] with the head axis innermost; q and k of every head are
    rotated split-half over the head with the patch's (row, col) angles and
    laid out as per-head planes [heads, n, hd] for the attention kernel; v is
    copied into its plane unchanged.  The rotation is this oracle's fused
    path for the vision 2-D layout (no RMSNorm), so the planes are the
    token-major results transposed.  Returns (q, k, v) planes in the stored
    representation.
    """
    qkv = np.asarray(qkv)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    qo, ko = rmsnorm_mrope_qk(q, k, pos, rotary_dim=rotary_dim, theta=theta, section=None,
                              layout=LAYOUT_VISION_2D, dtype=dtype, precision=precision)
    return (np.ascontiguousarray(qo.transpose(1, 0, 2)), np.ascontiguousarray(ko.transpose(1, 0, 2)),
            np.ascontiguousarray(v.transpose(1, 0, 2)))


# ---------------------------------------------------------------------------
# Decode: positions from the cache length, rotated K appended to a KV cache
# ---------------------------------------------------------------------------

def decode_positions(cache_len, new_tokens: int, rope_delta=None) -> np.ndarray:
    """Positions of the new tokens of a decode step, flattened [B * new_tokens].

    RoPE post, "Qwen3.5: MRoPE call chain" (``compute_3d_position_ids``): once
    ``rope_deltas`` are stored and the cache is non-empty, the positions are
    recovered from the sequence index counted from the cache length, expanded
    to all three axes, plus each sample's ``rope_deltas`` (the next rotary
    position minus the valid sequence length, from ``get_rope_index``).
    Token i of sample b gets ``cache_len[b] + i + rope_delta[b]``.
    """
    cache_len = np.asarray(cache_len, dtype=np.int64)
    B = cache_len.shape[0]
    delta = np.zeros(B, dtype=np.int64) if rope_delta is None else np.asarray(rope_delta, np.int64)
    i = np.arange(new_tokens, dtype=np.int64)
    return (cache_len[:, None] + i[None, :] + delta[:, None]).reshape(-1)


def mrope_decode_qk(q, k, cache_len, new_tokens: int, rope_delta, k_cache, *, rotary_dim: int,
                    theta: float, wq=None, wk=None, eps: float = 0.0, dtype: str = "bf16",
                    precision: str = "exact"):
    """One decode step: RMSNorm + rotary on q and k of B * new_tokens tokens
    whose positions follow ``decode_positions`` (text positions: the same on
    every axis, so the rotation is 1-D RoPE whatever the section), then the
    rotated k of token (b, i) is written to ``k_cache[b, cache_len[b] + i]``.

    ``k_cache`` is [B, capacity, hk, D] in the stored representation; rows at
    or past the capacity are not written.  Returns (q_out, new k_cache).
    """
    pos = decode_positions(cache_len, new_tokens, rope_delta)
    half = rotary_dim // 2
    qo, ko = rmsnorm_mrope_qk(q, k, pos.reshape(1, -1), rotary_dim=rotary_dim, theta=theta,
                              section=(half,), layout=LAYOUT_CHUNKED, wq=wq, wk=wk, eps=eps,
                              dtype=dtype, precision=precision)
    cache = np.array(k_cache, copy=True)
    cap = cache.shape[1]
    for b in range(len(cache_len)):
        for i in range(new_tokens):
            slot = int(cache_len[b]) + i
            if slot < cap:
                cache[b, slot] = ko[b * new_tokens + i]
    return qo, cache
