"""CPU oracle for the position builders of multimodal rotary embedding.

TEST INFRASTRUCTURE ONLY.  Imported by the test suite and the benchmark's
CPU-baseline leg, never by the library.  Shares no code with the HIP path.

Two builders, written from the pages in their order of steps:

* ``get_rope_index`` -- the 3-axis (T, H, W) position table of a batch of
  mixed text / image / video token sequences and the per-sample
  ``rope_deltas`` ("Interleaved Rotary Position Embedding", the
  ``get_rope_index()`` walkthrough: prepare the grids, filter padding and
  split into segments, advance positions, flatten the vision grid, write back,
  return the deltas; checked against its single-batch L = 10 table).
* ``vision_pos_ids`` -- the (row, col) coordinate of every vision patch in
  the order the vision tower emits patches ("Qwen3-VL" source walkthrough,
  ``rot_pos_emb``: merge-block order, repeated per frame).

Plain Python loops over segments and numpy ``arange``/``meshgrid`` for the
coordinates; every result is an exact integer.

Readings where the pages leave a step open:

1. Token types other than 0 (text), 1 (image) and 2 (video) have no grid
   iterator in the walkthrough; they are an error here.
2. A visual segment whose token count differs from its grid's slot count, or
   one with no grid left in its iterator, is an error (the walkthrough's
   concatenation and write-back could not succeed).
3. A sample with no valid token gets rope_delta 0 (the walkthrough's maximum
   over an empty table is undefined).
4. Vision grids must have h and w divisible by the merge size (otherwise the
   listing's patch count t*h*w and its coordinate count disagree).
"""
from __future__ import annotations

import itertools

import numpy as np

TEXT, IMAGE, VIDEO = 0, 1, 2


class PositionError(ValueError):
    """The inputs describe a sequence the walkthrough cannot build."""


def expand_video_grids(video_grid_thw):
    """Each video of t temporal slices becomes t grids with temporal length 1
    (the walkthrough splits videos by timestamps into per-slice segments)."""
    if video_grid_thw is None or len(video_grid_thw) == 0:
        return np.zeros((0, 3), dtype=np.int64)
    g = np.asarray(video_grid_thw, dtype=np.int64).reshape(-1, 3)
    out = np.repeat(g, g[:, 0], axis=0)
    out[:, 0] = 1
    return out


def vision_segment_ids(start: int, grid_thw, merge: int, temporal_merge: int = 1,
                       time_interval: int = 1) -> np.ndarray:
    """[3, n] positions of one visual segment starting at ``start``.

    The grid is given before spatial merging; the slot grid is
    (t // temporal_merge, h // merge, w // merge).  T = t_index *
    time_interval + start, H = row + start, W = col + start, flattened with
    the width fastest, then the height, then the time.
    """
    t, h, w = (int(v) for v in grid_thw)
    gt, gh, gw = t // temporal_merge, h // merge, w // merge
    pt = np.arange(gt, dtype=np.int64) * time_interval
    ph = np.arange(gh, dtype=np.int64) + start
    pw = np.arange(gw, dtype=np.int64) + start
    tt, hh, ww = np.meshgrid(pt, ph, pw, indexing="ij")
    ids = np.stack([tt, hh, ww], axis=0).reshape(3, -1)
    ids[0] += start
    return ids


def get_rope_index(mm_token_type, image_grid_thw=None, video_grid_thw=None,
                   attention_mask=None, merge: int = 2):
    """3-axis positions [3, B, L] and rope_deltas [B] (int64).

    ``mm_token_type`` is [B, L] with 0 text, 1 image, 2 video.  Grids are
    [n, 3] (t, h, w) before spatial merging; one image iterator and one video
    iterator are shared by the whole batch and consumed in sample order, then
    in order of appearance.  Padding (attention_mask 0) is removed before the
    segments are formed and keeps position 0.
    """
    types = np.asarray(mm_token_type, dtype=np.int64)
    if types.ndim != 2:
        raise PositionError("mm_token_type must be [B, L]")
    B, L = types.shape
    mask = None if attention_mask is None else np.asarray(attention_mask).astype(bool)
    videos = expand_video_grids(video_grid_thw)
    images = (np.zeros((0, 3), dtype=np.int64) if image_grid_thw is None
              else np.asarray(image_grid_thw, dtype=np.int64).reshape(-1, 3))
    iters = {IMAGE: iter(images), VIDEO: iter(videos)}
    position_ids = np.zeros((3, B, L), dtype=np.int64)
    deltas = np.zeros(B, dtype=np.int64)
    for b in range(B):
        row = types[b] if mask is None else types[b][mask[b]]
        groups = []
        for key, grp in itertools.groupby(enumerate(row.tolist()), lambda x: x[1]):
            grp = list(grp)
            groups.append((key, grp[0][0], grp[-1][0] + 1))
        current = 0
        parts = []
        for kind, s, e in groups:
            if kind == TEXT:
                n = e - s
                parts.append(np.broadcast_to(np.arange(n, dtype=np.int64) + current, (3, n)))
                current += n
            elif kind in (IMAGE, VIDEO):
                try:
                    grid = next(iters[kind])
                except StopIteration:
                    raise PositionError(f"sample {b}: no grid left for a type-{kind} segment")
                ids = vision_segment_ids(current, grid, merge)
                if ids.shape[1] != e - s:
                    raise PositionError(f"sample {b}: segment of {e - s} tokens, grid {grid} "
                                        f"has {ids.shape[1]} slots")
                parts.append(ids)
                current += max(int(grid[1]), int(grid[2])) // merge
            else:
                raise PositionError(f"sample {b}: unknown token type {kind}")
        if not parts:
            deltas[b] = 0
            continue
        llm = np.concatenate(parts, axis=1)
        if mask is None:
            position_ids[:, b] = llm
        else:
            position_ids[:, b, mask[b]] = llm
        deltas[b] = int(llm.max()) + 1 - llm.shape[1]
    return position_ids, deltas


def vision_pos_ids(grid_thw, merge: int = 2) -> np.ndarray:
    """[2, N] (row, col) of every patch, images in order, each image's patches
    in merge-block order (block row, block col, row in block, col in block),
    repeated for each of its t frames."""
    grids = np.asarray(grid_thw, dtype=np.int64).reshape(-1, 3)
    out = []
    for t, h, w in grids.tolist():
        if h % merge or w % merge:
            raise PositionError(f"grid {(t, h, w)} is not divisible by merge {merge}")
        mh, mw = h // merge, w // merge
        br = np.arange(mh)[:, None, None, None]
        bc = np.arange(mw)[None, :, None, None]
        ir = np.arange(merge)[None, None, :, None]
        ic = np.arange(merge)[None, None, None, :]
        rows = np.broadcast_to(br * merge + ir, (mh, mw, merge, merge)).reshape(-1)
        cols = np.broadcast_to(bc * merge + ic, (mh, mw, merge, merge)).reshape(-1)
        coords = np.stack([rows, cols], axis=0)
        out.append(np.tile(coords, (1, t)))
    if not out:
        return np.zeros((2, 0), dtype=np.int64)
    return np.concatenate(out, axis=1).astype(np.int64)
