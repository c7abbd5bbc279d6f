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

Plain Python loops over tokens, runs and slots; every result is an exact
integer.

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

import numpy as np

TEXT, IMAGE, VIDEO = 0, 1, 2


class PositionError(ValueError):
    """The inputs describe a sequence the walkthrough cannot build."""


# ---------------------------------------------------------------------------
# Step 1 of the walkthrough: the grid queues
# ---------------------------------------------------------------------------

def grid_queues(image_grid_thw, video_grid_thw):
    """The two grid queues of a batch: images as given, and every video of t
    temporal slices as t single-slice grids (1, h, w) in slice order (the
    walkthrough cuts videos into per-slice segments at their timestamps).
    Returns (images, slices), each a list of (t, h, w) int tuples."""
    images = []
    if image_grid_thw is not None:
        for t, h, w in np.asarray(image_grid_thw, dtype=np.int64).reshape(-1, 3).tolist():
            images.append((t, h, w))
    slices = []
    if video_grid_thw is not None:
        for t, h, w in np.asarray(video_grid_thw, dtype=np.int64).reshape(-1, 3).tolist():
            for _ in range(t):
                slices.append((1, h, w))
    return images, slices


# ---------------------------------------------------------------------------
# Step 2: runs of equal token type in the sequence left after padding
# ---------------------------------------------------------------------------

def type_runs(types):
    """Maximal runs of one token type, as (type, first, end) with end
    exclusive: a new run starts wherever the type differs from the token
    before it (two images separated by a text token are two runs)."""
    runs = []
    for i, ty in enumerate(types):
        if runs and runs[-1][0] == ty:
            runs[-1][2] = i + 1
        else:
            runs.append([ty, i, i + 1])
    return [tuple(r) for r in runs]


# ---------------------------------------------------------------------------
# Steps 3-4: positions of a visual run
# ---------------------------------------------------------------------------

def visual_run_positions(start: int, grid_thw, merge: int) -> np.ndarray:
    """[3, n] positions of the slots of one visual run that begins at rotary
    position ``start``.

    The grid is given before spatial merging: its slots form the
    (t, h // merge, w // merge) grid, taken width first, then height, then
    time.  Slot s is at time index s // (rows * cols), row (s // cols) %
    rows and column s % cols, and gets (start + time, start + row,
    start + column): every axis is offset by the run's start.
    """
    t, h, w = (int(v) for v in grid_thw)
    rows, cols = h // merge, w // merge
    n = t * rows * cols
    out = np.empty((3, n), dtype=np.int64)
    for s in range(n):
        out[0, s] = start + s // (rows * cols)
        out[1, s] = start + (s // cols) % rows
        out[2, s] = start + s % cols
    return out


# ---------------------------------------------------------------------------
# The builder
# ---------------------------------------------------------------------------

def get_rope_index(mm_token_type, image_grid_thw=None, video_grid_thw=None,
                   attention_mask=None, merge: int = 2):
    """3-axis positions [3, B, L] and rope_deltas [B] (int64).

    ``mm_token_type`` is [B, L] with 0 text, 1 image, 2 video.  Grids are
    [n, 3] (t, h, w) before spatial merging.  The walkthrough's steps, in its
    order:

    1. the grid queues (``grid_queues``): one image queue and one video-slice
       queue for the whole batch, taken in sample order, then in order of
       appearance;
    2. per sample, the tokens the mask keeps (all of them without a mask),
       cut into runs of one type (``type_runs``);
    3. a running rotary position, 0 at the sample's first kept token: a text
       run of n tokens takes p, p + 1, ..., p + n - 1 on all three axes and
       moves p on by n; a visual run takes the next grid of its queue, its
       slots take ``visual_run_positions(p, grid)``, and p moves on by the
       longer merged side max(h, w) // merge, not by the slot count;
    4. (the flattening of the slot grid, inside ``visual_run_positions``);
    5. the kept tokens' positions are written back to their slots; slots the
       mask drops keep 0;
    6. rope_delta = largest position + 1 - number of kept tokens.
    """
    types = np.asarray(mm_token_type, dtype=np.int64)
    if types.ndim != 2:
        raise PositionError("mm_token_type must be [B, L]")
    B, L = types.shape
    keep = (np.ones((B, L), dtype=bool) if attention_mask is None
            else np.asarray(attention_mask).astype(bool))
    queues = dict(zip((IMAGE, VIDEO), grid_queues(image_grid_thw, video_grid_thw)))
    taken = {IMAGE: 0, VIDEO: 0}
    position_ids = np.zeros((3, B, L), dtype=np.int64)
    deltas = np.zeros(B, dtype=np.int64)
    for b in range(B):
        slots = np.nonzero(keep[b])[0]               # kept slots, in order
        kept_types = types[b, slots].tolist()
        pos = np.zeros((3, len(slots)), dtype=np.int64)
        p = 0
        for ty, first, end in type_runs(kept_types):
            if ty == TEXT:
                pos[:, first:end] = p + np.arange(end - first, dtype=np.int64)
                p += end - first
            elif ty in (IMAGE, VIDEO):
                if taken[ty] >= len(queues[ty]):
                    raise PositionError(f"sample {b}: no grid left for a type-{ty} run")
                grid = queues[ty][taken[ty]]
                taken[ty] += 1
                ids = visual_run_positions(p, grid, merge)
                if ids.shape[1] != end - first:
                    raise PositionError(f"sample {b}: run of {end - first} tokens, grid {grid} "
                                        f"has {ids.shape[1]} slots")
                pos[:, first:end] = ids
                p += max(grid[1], grid[2]) // merge
            else:
                raise PositionError(f"sample {b}: unknown token type {ty}")
        position_ids[:, b, slots] = pos
        deltas[b] = int(pos.max()) + 1 - len(slots) if len(slots) else 0
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
