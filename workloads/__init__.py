"""Seeded synthetic workloads for the fused RMSNorm + multimodal rotary path.

This module only *generates inputs*: random tensors and integer position
tables.  It holds none of the method's arithmetic (no frequencies, angles,
norms or rotations), so both the CPU oracle and the GPU path can consume the
same arrays without sharing code.

Five workloads, shaped after the models the pages describe:

* ``tiny_mrope``            q[16,2,16], k[16,1,16] fp32, interleaved [4,2,2],
                            positions uniform in [0,32); no RMSNorm.
* ``omni_text_prefill``     q[32768,32,128], k[32768,4,128] bf16, interleaved
                            [24,20,20], theta 1e6, text-only positions, RMSNorm.
* ``qwen35_partial_mixed``  q[16384,24,256], k[16384,4,256] bf16, rotary_dim 64,
                            interleaved [11,11,10], theta 1e7, 512 text tokens,
                            one 24x32 merged image grid, then text; RMSNorm.
* ``chunked_video``         q[11264,28,128], k[11264,4,128] bf16, chunked
                            [16,24,24], theta 1e6, 1024 text + a 16x24x24 video
                            grid + 1024 text; no RMSNorm.
* ``vision_2d``             q,k[32768,16,72] fp32, vision 2-D layout, theta 1e4,
                            8 images of 64x64 patches in 2x2 merge-block order.

Random draws: ``numpy.random.default_rng(seed)`` with seed = the workload's
index (1..5); draw order q, k, w_q, w_k, then positions (tiny_mrope only).
q and k are standard normal binary32 draws; for bf16 workloads they are
rounded to bfloat16 (nearest, ties to even, by torch's CPU conversion).
RMSNorm weights are 1 + 0.1 * standard normal, rounded the same way.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    dtype: str            # "bf16" or "f32"
    T: int
    hq: int
    hk: int
    D: int
    rotary_dim: int
    theta: float
    layout: str           # "interleaved" | "chunked" | "vision_2d"
    section: tuple
    norm: bool
    eps: float = 1e-6
    description: str = ""

    @property
    def n_axes(self) -> int:
        return {"interleaved": 3, "chunked": len(self.section), "vision_2d": 2}[self.layout]

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def algorithmic_bytes(self, T: int | None = None) -> int:
        """HBM bytes one fused call must move: read and write every q/k
        element once, read the int32 positions, read the two weight vectors."""
        T = self.T if T is None else T
        qk = 2 * T * (self.hq + self.hk) * self.D * self.elem_bytes
        pos = 4 * self.n_axes * T
        w = 2 * self.D * self.elem_bytes if self.norm else 0
        return qk + pos + w


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_mrope", 1, "f32", 16, 2, 1, 16, 16, 1e4, "interleaved", (4, 2, 2), False,
                 description="Tiny MRoPE, T=16, D=16, interleaved [4,2,2], random positions"),
        Workload("omni_text_prefill", 2, "bf16", 32768, 32, 4, 128, 128, 1e6, "interleaved",
                 (24, 20, 20), True,
                 description="Omni-like text prefill, T=32768, 32/4 heads x 128, RMSNorm"),
        Workload("qwen35_partial_mixed", 3, "bf16", 16384, 24, 4, 256, 64, 1e7, "interleaved",
                 (11, 11, 10), True,
                 description="Qwen3.5-like partial rotary 64 of 256, text+image+text, RMSNorm"),
        Workload("chunked_video", 4, "bf16", 11264, 28, 4, 128, 128, 1e6, "chunked",
                 (16, 24, 24), False,
                 description="Chunked MRoPE on text+video(16x24x24)+text, T=11264"),
        Workload("vision_2d", 5, "f32", 32768, 16, 16, 72, 72, 1e4, "vision_2d", (18, 18), False,
                 description="Vision-tower 2-D RoPE, 8 images of 64x64 patches, 16 heads x 72"),
    ]
}


# ---------------------------------------------------------------------------
# Position builders (integer bookkeeping only)
# ---------------------------------------------------------------------------

def text_positions(n: int, start: int = 0) -> np.ndarray:
    """Text tokens advance by one on all three axes."""
    p = np.arange(start, start + n, dtype=np.int64)
    return np.stack([p, p, p])


def vision_segment_positions(start: int, grid_t: int, grid_h: int, grid_w: int,
                             time_interval: int = 1) -> np.ndarray:
    """(t, h, w) of a merged visual grid, width fastest, height next, time
    slowest; every axis offset by the segment start.  The RoPE post's
    ``get_vision_position_ids`` (meshgrid with 'ij' indexing)."""
    t = start + np.arange(grid_t, dtype=np.int64) * time_interval
    h = start + np.arange(grid_h, dtype=np.int64)
    w = start + np.arange(grid_w, dtype=np.int64)
    tt, hh, ww = np.meshgrid(t, h, w, indexing="ij")
    return np.stack([tt.reshape(-1), hh.reshape(-1), ww.reshape(-1)])


def rope_index(segments, merge: int = 2):
    """3-axis position table for a sequence of segments.

    ``segments`` is a list of ``("text", n)`` or ``("image", (t, h, w))`` with
    the grid before spatial merging.  A visual segment takes positions from
    ``vision_segment_positions`` on the merged grid and then advances the
    running position by max(h, w) // merge (the RoPE post's
    ``get_rope_index``: advance by the longer merged side, not by the token
    count).  Returns (positions [3, L], rope_delta = max + 1 - L).
    """
    cur = 0
    parts = []
    for kind, arg in segments:
        if kind == "text":
            parts.append(text_positions(arg, cur))
            cur += arg
        elif kind == "image":
            t, h, w = arg
            parts.append(vision_segment_positions(cur, t, h // merge, w // merge))
            cur += max(h, w) // merge
        else:
            raise ValueError(kind)
    pos = np.concatenate(parts, axis=1)
    return pos, int(pos.max()) + 1 - pos.shape[1]


def vision_patch_positions(n_images: int, h: int, w: int, merge: int = 2) -> np.ndarray:
    """(row, col) per patch for n_images h x w patch grids, emitted in
    merge x merge block order (block row, block col, intra row, intra col),
    as the Qwen3-VL ``rot_pos_emb`` and qwen3vis.rs ``rope_angles`` emit them."""
    rows, cols = [], []
    for _ in range(n_images):
        for by in range(h // merge):
            for bx in range(w // merge):
                for iy in range(merge):
                    for ix in range(merge):
                        rows.append(by * merge + iy)
                        cols.append(bx * merge + ix)
    return np.stack([np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)])


def workload_positions(wl: Workload, rng: np.random.Generator | None = None) -> np.ndarray:
    """int32 positions [n_axes, T] of a named workload."""
    if wl.name == "tiny_mrope":
        assert rng is not None
        pos = rng.integers(0, 32, size=(3, wl.T))
    elif wl.name == "omni_text_prefill":
        pos = text_positions(wl.T)
    elif wl.name == "qwen35_partial_mixed":
        # 512 text tokens, one image whose patch grid is 48x64 (24x32 merged),
        # then text up to T tokens.
        n_img = 24 * 32
        pos, _ = rope_index([("text", 512), ("image", (1, 48, 64)),
                             ("text", wl.T - 512 - n_img)])
    elif wl.name == "chunked_video":
        # 1024 text tokens, one video segment on a merged 16x24x24 grid, then
        # text resuming at the segment start + max(h, w) (= max position + 1).
        head = text_positions(1024)
        vid = vision_segment_positions(1024, 16, 24, 24)
        tail = text_positions(wl.T - 1024 - vid.shape[1], 1024 + 24)
        pos = np.concatenate([head, vid, tail], axis=1)
    elif wl.name == "vision_2d":
        pos = vision_patch_positions(8, 64, 64)
    else:
        raise KeyError(wl.name)
    assert pos.shape == (wl.n_axes, wl.T), (pos.shape, wl.n_axes, wl.T)
    return np.ascontiguousarray(pos.astype(np.int32))


def vision_cu_seqlens(n_images: int = 8, patches: int = 64 * 64) -> np.ndarray:
    """Cumulative patch counts per image (carried for completeness; the
    rotation does not read it)."""
    return np.arange(0, (n_images + 1) * patches, patches, dtype=np.int32)


# ---------------------------------------------------------------------------
# Tensors
# ---------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns (uint16), nearest-even, via torch CPU."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def make_inputs(wl: Workload | str, T: int | None = None, seed: int | None = None,
                pos_offset: int = 0) -> dict:
    """Seeded inputs for a workload.

    ``T`` (optional) shrinks the token count for small parity runs: the
    random tensors are then drawn at the smaller shape, and positions are the
    columns [pos_offset, pos_offset + T) of the full table (tiny_mrope draws
    its own).  Returns a dict with q, k (uint16 bf16 bits or float32), wq, wk
    (or None), pos (int32 [n_axes, T]) and the workload record.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    full_T = wl.T
    T = full_T if T is None else int(T)
    rng = np.random.default_rng(wl.index if seed is None else seed)
    q = rng.standard_normal((T, wl.hq, wl.D), dtype=np.float32)
    k = rng.standard_normal((T, wl.hk, wl.D), dtype=np.float32)
    wq = wk = None
    if wl.norm:
        wq = (1.0 + 0.1 * rng.standard_normal(wl.D)).astype(np.float32)
        wk = (1.0 + 0.1 * rng.standard_normal(wl.D)).astype(np.float32)
    if wl.name == "tiny_mrope":
        pos = rng.integers(0, 32, size=(3, T)).astype(np.int32)
    else:
        pos = workload_positions(wl)[:, pos_offset:pos_offset + T]
        assert pos.shape[1] == T, "pos_offset + T exceeds the workload"
    out = dict(q=_store(q, wl.dtype), k=_store(k, wl.dtype),
               wq=None if wq is None else _store(wq, wl.dtype),
               wk=None if wk is None else _store(wk, wl.dtype),
               pos=np.ascontiguousarray(pos, dtype=np.int32), workload=wl, T=T)
    return out


def random_qk(rng: np.random.Generator, T: int, hq: int, hk: int, D: int, dtype: str,
              scale: float = 1.0):
    """Free-form seeded q, k for edge-case tests (same recipe as the workloads)."""
    q = (scale * rng.standard_normal((T, hq, D))).astype(np.float32)
    k = (scale * rng.standard_normal((T, hk, D))).astype(np.float32)
    return _store(q, dtype), _store(k, dtype)


def random_weight(rng: np.random.Generator, D: int, dtype: str):
    return _store((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32), dtype)


# ---------------------------------------------------------------------------
# Decode steps
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    index: int
    dtype: str
    batch: int            # sequences
    new_tokens: int       # tokens appended per sequence
    hq: int
    hk: int
    D: int
    rotary_dim: int
    theta: float
    capacity: int         # KV-cache rows per sequence
    norm: bool
    eps: float = 1e-6
    description: str = ""

    @property
    def T(self) -> int:
        return self.batch * self.new_tokens

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def algorithmic_bytes(self) -> int:
        """Read q and k, write q_out and the k-cache rows, read cache_len and
        rope_delta, read the two weight vectors."""
        qk = self.T * (2 * self.hq + 2 * self.hk) * self.D * self.elem_bytes
        meta = 2 * 4 * self.batch
        w = 2 * self.D * self.elem_bytes if self.norm else 0
        return qk + meta + w


DECODE_WORKLOADS = {
    w.name: w for w in [
        DecodeWorkload("omni_decode", 6, "bf16", 512, 1, 32, 4, 128, 128, 1e6, 1024, True,
                       description="Omni-like decode: 512 sequences x 1 new token, "
                                   "k appended to a 1024-row cache"),
    ]
}


def make_decode_inputs(wl: DecodeWorkload | str, batch: int | None = None,
                       new_tokens: int | None = None, capacity: int | None = None,
                       seed: int | None = None) -> dict:
    """Seeded decode-step inputs: q, k [batch*new_tokens, heads, D], weights,
    cache_len uniform in [0, capacity - new_tokens], rope_delta uniform in
    [-300, 0] (a prompt with visual segments advances its positions by less
    than its token count), and a random k_cache [batch, capacity, hk, D]."""
    if isinstance(wl, str):
        wl = DECODE_WORKLOADS[wl]
    B = wl.batch if batch is None else batch
    n = wl.new_tokens if new_tokens is None else new_tokens
    cap = wl.capacity if capacity is None else capacity
    rng = np.random.default_rng(wl.index if seed is None else seed)
    q = rng.standard_normal((B * n, wl.hq, wl.D), dtype=np.float32)
    k = rng.standard_normal((B * n, wl.hk, wl.D), dtype=np.float32)
    wq = wk = None
    if wl.norm:
        wq = (1.0 + 0.1 * rng.standard_normal(wl.D)).astype(np.float32)
        wk = (1.0 + 0.1 * rng.standard_normal(wl.D)).astype(np.float32)
    cache_len = rng.integers(0, max(1, cap - n + 1), size=B).astype(np.int32)
    rope_delta = rng.integers(-300, 1, size=B).astype(np.int32)
    cache = rng.standard_normal((B, cap, wl.hk, wl.D), dtype=np.float32)
    return dict(q=_store(q, wl.dtype), k=_store(k, wl.dtype),
                wq=None if wq is None else _store(wq, wl.dtype),
                wk=None if wk is None else _store(wk, wl.dtype),
                cache_len=cache_len, rope_delta=rope_delta, k_cache=_store(cache, wl.dtype),
                workload=wl, batch=B, new_tokens=n, capacity=cap)


def random_mm_batch(rng, B: int, L: int, pad: bool = True, merge: int = 2):
    """Random mixed-modality batch for the position builders: token types
    [B, L] (0 text, 1 image, 2 video), attention mask [B, L], and the image /
    video grids (t, h, w) the batch consumes in order.  Each sample is a
    sequence of whole units -- a text run; an image followed by a text token;
    a video whose single-slice runs are separated by timestamp text -- padded
    on the left or with a hole near the start.  Grids are small (h, w even,
    at most 6) so that many runs fit."""
    types = np.zeros((B, L), dtype=np.int64)
    mask = np.zeros((B, L), dtype=np.int64)
    images, videos = [], []
    for b in range(B):
        budget = L - (int(rng.integers(0, L // 4 + 1)) if pad else 0)
        flat = []
        for _ in range(max(200, L // 2)):
            if len(flat) >= budget:
                break
            r = rng.random()
            if r < 0.45:
                unit, img, vid = [0] * int(rng.integers(1, 12)), None, None
            elif r < 0.75:
                t, h, w = 1, 2 * int(rng.integers(1, 4)), 2 * int(rng.integers(1, 4))
                unit = [1] * ((h // merge) * (w // merge)) + [0]
                img, vid = (t, h, w), None
            else:
                t, h, w = int(rng.integers(1, 4)), 2 * int(rng.integers(1, 3)), 2 * int(rng.integers(1, 3))
                unit = []
                for _ in range(t):
                    unit += [0] * int(rng.integers(1, 3)) + [2] * ((h // merge) * (w // merge))
                unit += [0]
                img, vid = None, (t, h, w)
            if len(flat) + len(unit) > budget:
                continue
            flat += unit
            if img:
                images.append(img)
            if vid:
                videos.append(vid)
        valid = len(flat)
        hole = L - valid
        if rng.random() < 0.5 or hole == 0:
            types[b, hole:] = flat
            mask[b, hole:] = 1
        else:
            # a hole inside the first text stretch (or at the start)
            cut = 0
            while cut < valid and flat[cut] == 0 and cut < 3:
                cut += 1
            types[b, :cut] = flat[:cut]
            mask[b, :cut] = 1
            types[b, cut + hole:] = flat[cut:]
            mask[b, cut + hole:] = 1
    return types, mask, images, videos


@dataclasses.dataclass(frozen=True)
class PositionWorkload:
    """A batch of multimodal prompts for the position builder."""
    name: str
    index: int
    batch: int
    seq_len: int
    description: str = ""

    @property
    def T(self) -> int:
        return self.batch * self.seq_len

    def algorithmic_bytes(self) -> int:
        # token types and mask read once (int32), three int32 positions
        # written, one delta per sample
        return self.T * (4 + 4 + 12) + 4 * self.batch


POSITION_WORKLOADS = {
    w.name: w for w in [
        PositionWorkload("mm_prompt_positions", 7, 8, 8192,
                         description="8 prompts x 8192 slots: system text, a 48x64-patch image, "
                                     "text, a 4-slice 32x32 video with timestamps, text, left "
                                     "padding"),
    ]
}


def mm_prompt_batch(wl: PositionWorkload | str, seed: int | None = None):
    """Seeded batch of chat-style multimodal prompts: per sample, a system
    text run, one image (1, 48, 64) -> 768 slots, a text run, one video of 4
    slices (4, 32, 32) -> 4 runs of 256 slots each preceded by 3 timestamp
    tokens, then text, with 0..1023 tokens of left padding.  Returns types,
    mask [B, L] int32 and the image / video grids in batch order."""
    if isinstance(wl, str):
        wl = POSITION_WORKLOADS[wl]
    rng = np.random.default_rng(wl.index if seed is None else seed)
    B, L = wl.batch, wl.seq_len
    types = np.zeros((B, L), dtype=np.int32)
    mask = np.zeros((B, L), dtype=np.int32)
    images, videos = [], []
    for b in range(B):
        pad = int(rng.integers(0, 1024))
        sys_len = int(rng.integers(50, 400))
        mid = int(rng.integers(20, 300))
        seq = [0] * sys_len + [1] * 768 + [0] * mid
        for _ in range(4):
            seq += [0] * 3 + [2] * 256
        seq += [0] * (L - pad - len(seq))
        types[b, pad:] = seq
        mask[b, pad:] = 1
        images.append((1, 48, 64))
        videos.append((4, 32, 32))
    return types, mask, np.array(images, dtype=np.int32), np.array(videos, dtype=np.int32)


@dataclasses.dataclass(frozen=True)
class VisionQKVWorkload:
    """Packed vision qkv [n, 3, heads, D] rotated into per-head planes."""
    name: str
    index: int
    dtype: str
    n_images: int
    side: int             # patches per image side (before merging)
    heads: int
    D: int
    rotary_dim: int
    theta: float
    description: str = ""

    @property
    def T(self) -> int:
        return self.n_images * self.side * self.side

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def algorithmic_bytes(self) -> int:
        # read q, k, v of every patch once, write the three planes once,
        # read the (row, col) positions
        return 2 * self.T * 3 * self.heads * self.D * self.elem_bytes + 8 * self.T


VISION_QKV_WORKLOADS = {
    w.name: w for w in [
        VisionQKVWorkload("vision_qkv_planes", 8, "f32", 8, 64, 16, 72, 72, 1e4,
                          description="Vision tower packed qkv of 8 images x 64x64 patches, "
                                      "16 heads x 72, to head-major planes (q, k rotated)"),
        VisionQKVWorkload("vision_qkv_planes_bf16", 9, "bf16", 8, 64, 16, 72, 72, 1e4,
                          description="The same in bfloat16"),
    ]
}


def make_vision_qkv_inputs(wl: VisionQKVWorkload | str, n: int | None = None,
                           seed: int | None = None) -> dict:
    """Seeded packed qkv [n, 3, heads, D] (standard normal, stored in the
    workload dtype) and the patches' (row, col) positions [2, n] in
    merge-block order (the first n patches of the workload's images)."""
    if isinstance(wl, str):
        wl = VISION_QKV_WORKLOADS[wl]
    n = wl.T if n is None else n
    rng = np.random.default_rng(wl.index if seed is None else seed)
    qkv = rng.standard_normal((n, 3, wl.heads, wl.D), dtype=np.float32)
    pos = vision_patch_positions(wl.n_images, wl.side, wl.side)
    reps = -(-n // pos.shape[1])
    pos = np.tile(pos, (1, reps))[:, :n].astype(np.int32)
    return dict(qkv=_store(qkv, wl.dtype), pos=np.ascontiguousarray(pos), T=n, workload=wl)
