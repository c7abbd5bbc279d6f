"""Pins of the position-builder oracle (get_rope_index, rot_pos_emb order).

Checks against the pages' printed single-batch table, closed forms for
text-only and padded batches, the walkthrough's stated rules (video slices,
shared grid iterators, segment splitting), and an independently written
builder (the input generator's segment-list builder); planted mistakes must
fail at least one pin.
"""
import json
import os

import numpy as np
import pytest

from oracle import positions_oracle as P
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _types_of(segments, merge=2):
    """Token types and image grids of a segment list (text n / image (t,h,w))."""
    types, grids = [], []
    for kind, arg in segments:
        if kind == "text":
            types += [P.TEXT] * arg
        else:
            t, h, w = arg
            types += [P.IMAGE] * (t * (h // merge) * (w // merge))
            grids.append(list(arg))
    return np.array(types, dtype=np.int64), np.array(grids, dtype=np.int64).reshape(-1, 3)


def check_printed_table():
    """RoPE post, three-axis position table, single-batch example."""
    g = _golden("position_table.json")
    segs = [(k, tuple(v) if isinstance(v, list) else v) for k, v in g["segments"]]
    types, grids = _types_of(segs, g["merge"])
    pos, delta = P.get_rope_index(types[None], image_grid_thw=grids, merge=g["merge"])
    assert pos[0, 0].tolist() == g["T"]
    assert pos[1, 0].tolist() == g["H"]
    assert pos[2, 0].tolist() == g["W"]
    assert pos[:, 0, g["I12_column"]].tolist() == g["I12_position"]
    # the next rotary position is 7 (advance by the longer merged side, 3),
    # so the delta is 7 - 10
    assert delta.tolist() == [-3]


def check_text_only_and_padding():
    L = 12
    types = np.zeros((1, L), dtype=np.int64)
    pos, delta = P.get_rope_index(types)
    assert np.array_equal(pos, np.broadcast_to(np.arange(L), (3, 1, L)))
    assert delta.tolist() == [0]
    # left padding, right padding and a hole: valid slots get the unpadded
    # table in order, padded slots keep 0, the delta counts valid tokens
    g = _golden("position_table.json")
    segs = [(k, tuple(v) if isinstance(v, list) else v) for k, v in g["segments"]]
    t0, grids = _types_of(segs, g["merge"])
    base, d0 = P.get_rope_index(t0[None], image_grid_thw=grids)
    n = t0.shape[0]
    for mask in ([0] * 3 + [1] * n, [1] * n + [0] * 4, [1] * 4 + [0, 0] + [1] * (n - 4)):
        mask = np.array(mask)
        types = np.zeros(mask.shape[0], dtype=np.int64)
        types[mask.astype(bool)] = t0
        pos, d = P.get_rope_index(types[None], image_grid_thw=grids, attention_mask=mask[None])
        assert np.array_equal(pos[:, 0, mask.astype(bool)], base[:, 0])
        assert np.all(pos[:, 0, ~mask.astype(bool)] == 0)
        assert d.tolist() == d0.tolist()


def check_video_slices_and_shared_iterators():
    # one video of 3 slices, each slice its own segment between timestamp text
    # tokens, equals three single-slice videos
    hw = (4, 6)
    n_slot = (hw[0] // 2) * (hw[1] // 2)
    types = np.array(([0, 0] + [2] * n_slot) * 3 + [0], dtype=np.int64)[None]
    a, da = P.get_rope_index(types, video_grid_thw=[[3, *hw]])
    b, db = P.get_rope_index(types, video_grid_thw=[[1, *hw]] * 3)
    assert np.array_equal(a, b) and da.tolist() == db.tolist()
    # each slice has a constant T, and the next segment starts max(h,w)/2 later
    starts = [2, 2 + n_slot + 2, 2 + 2 * (n_slot + 2)]
    for s in starts:
        assert len(set(a[0, 0, s:s + n_slot].tolist())) == 1
    assert a[0, 0, starts[1]] - a[0, 0, starts[0]] == 3 + 2
    # the image iterator is shared by the batch: sample 1 takes the second grid
    types = np.array([[0, 1, 1, 1, 1, 0, 0, 0, 0, 0, 0, 0],
                      [0] + [1] * 8 + [0, 0, 0]], dtype=np.int64)
    pos, d = P.get_rope_index(types, image_grid_thw=[[1, 4, 4], [1, 4, 8]])
    assert pos[2, 1, 1:9].tolist() == [1, 2, 3, 4, 1, 2, 3, 4]       # 2 x 4 merged grid
    assert pos[1, 1, 1:9].tolist() == [1, 1, 1, 1, 2, 2, 2, 2]
    # sample 0: image advances 2 (merged 2 x 2), text ends at 9 -> 10 - 12;
    # sample 1: image advances 4 (merged 2 x 4), text ends at 7 -> 8 - 12
    assert d.tolist() == [-2, -4]
    # two image groups separated by a text token are two segments
    types = np.array([[1, 1, 1, 1, 0, 1, 1, 1, 1]], dtype=np.int64)
    pos, _ = P.get_rope_index(types, image_grid_thw=[[1, 4, 4], [1, 4, 4]])
    assert pos[:, 0, 4].tolist() == [2, 2, 2] and pos[:, 0, 5].tolist() == [3, 3, 3]


def check_against_segment_builder():
    """The input generator's builder is a separate implementation of the same
    rule over segment lists; both must agree on the workload layouts."""
    for segs in ([("text", 512), ("image", (1, 48, 64)), ("text", 700)],
                 [("text", 1024), ("image", (16, 48, 48)), ("text", 1024)],
                 [("text", 3), ("image", (1, 4, 6)), ("text", 1), ("image", (2, 6, 4)),
                  ("text", 5)]):
        types, grids = _types_of(segs)
        want, wd = W.rope_index(segs)
        got, gd = P.get_rope_index(types[None], image_grid_thw=grids)
        assert np.array_equal(got[:, 0], want) and int(gd[0]) == wd


def check_vision_pos_ids():
    got = P.vision_pos_ids([[1, 4, 4]], merge=2)
    assert got[0].tolist() == [0, 0, 1, 1, 0, 0, 1, 1, 2, 2, 3, 3, 2, 2, 3, 3]
    assert got[1].tolist() == [0, 1, 0, 1, 2, 3, 2, 3, 0, 1, 0, 1, 2, 3, 2, 3]
    two = P.vision_pos_ids([[2, 4, 4]], merge=2)
    assert np.array_equal(two, np.concatenate([got, got], axis=1))
    assert np.array_equal(P.vision_pos_ids([[1, 64, 64]] * 3),
                          W.vision_patch_positions(3, 64, 64))
    # every (row, col) of a frame appears exactly once
    g = P.vision_pos_ids([[1, 6, 10]], merge=2)
    assert len(set(zip(g[0].tolist(), g[1].tolist()))) == 60


def test_printed_table():
    check_printed_table()


def test_text_only_and_padding():
    check_text_only_and_padding()


def test_video_slices_and_shared_iterators():
    check_video_slices_and_shared_iterators()


def test_against_segment_builder():
    check_against_segment_builder()


def test_vision_pos_ids():
    check_vision_pos_ids()


def test_errors():
    with pytest.raises(P.PositionError):
        P.get_rope_index(np.array([[0, 1, 1, 1, 1]]))                      # no grid
    with pytest.raises(P.PositionError):
        P.get_rope_index(np.array([[0, 1, 1, 1]]), image_grid_thw=[[1, 4, 4]])   # 3 != 4
    with pytest.raises(P.PositionError):
        P.get_rope_index(np.array([[0, 3, 3]]))                            # unknown type
    with pytest.raises(P.PositionError):
        P.vision_pos_ids([[1, 5, 4]])
    pos, d = P.get_rope_index(np.zeros((1, 4), dtype=np.int64), attention_mask=np.zeros((1, 4)))
    assert np.all(pos == 0) and d.tolist() == [0]


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

_ORIG_SEG = P.visual_run_positions
_ORIG_GRI = P.get_rope_index


def _mut_height_fastest(start, grid_thw, merge):
    ids = _ORIG_SEG(start, grid_thw, merge)
    t, h, w = (int(v) for v in grid_thw)
    gh, gw = h // merge, w // merge
    perm = np.arange(gh * gw).reshape(gh, gw).T.reshape(-1)
    return ids[:, np.tile(perm, t)] if ids.shape[1] == t * gh * gw else ids


def _mut_advance_by_token_count(mm_token_type, image_grid_thw=None, video_grid_thw=None,
                                attention_mask=None, merge=2):
    # the text after a visual segment resumes at the segment start plus its
    # slot count instead of plus max(h, w) / merge
    types = np.asarray(mm_token_type)
    pos, d = _ORIG_GRI(mm_token_type, image_grid_thw, video_grid_thw, attention_mask, merge)
    out = pos.copy()
    for b in range(types.shape[0]):
        row = types[b]
        shift = 0
        prev = 0
        for l in range(row.shape[0]):
            if prev != 0 and row[l] == 0:
                n = 0
                j = l - 1
                while j >= 0 and row[j] != 0:
                    n += 1
                    j -= 1
                shift += n - (pos[0, b, l] - pos[0, b, j + 1])
            out[:, b, l] += shift
            prev = row[l]
    return out, d


def _mut_iterator_per_sample(mm_token_type, image_grid_thw=None, video_grid_thw=None,
                             attention_mask=None, merge=2):
    types = np.asarray(mm_token_type)
    outs, ds = [], []
    for b in range(types.shape[0]):
        m = None if attention_mask is None else np.asarray(attention_mask)[b:b + 1]
        p, d = _ORIG_GRI(types[b:b + 1], image_grid_thw, video_grid_thw, m, merge)
        outs.append(p)
        ds.append(d)
    return np.concatenate(outs, axis=1), np.concatenate(ds)


def _mut_no_mask_filter(mm_token_type, image_grid_thw=None, video_grid_thw=None,
                        attention_mask=None, merge=2):
    pos, d = _ORIG_GRI(mm_token_type, image_grid_thw, video_grid_thw, None, merge)
    if attention_mask is not None:
        pos = pos * np.asarray(attention_mask)[None].astype(np.int64)
    return pos, d


MUTATIONS = [
    ("visual_run_positions", _mut_height_fastest, check_printed_table),
    ("get_rope_index", _mut_advance_by_token_count, check_printed_table),
    ("get_rope_index", _mut_iterator_per_sample, check_video_slices_and_shared_iterators),
    ("get_rope_index", _mut_no_mask_filter, check_text_only_and_padding),
]


@pytest.mark.parametrize("name,mutant,check", MUTATIONS,
                         ids=[f"{n}:{m.__name__}" for n, m, _ in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, check):
    check()
    monkeypatch.setattr(P, name, mutant)
    with pytest.raises((AssertionError, P.PositionError, StopIteration)):
        check()
