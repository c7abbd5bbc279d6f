"""mrope_rope_index_noalloc (static device workspace) against
mrope_rope_index (caller workspace) through the C ABI: the same 3-axis
positions, rope_deltas and status word, bit for bit, on two calls in a row,
the second with a smaller batch (the static array keeps the first call's
contents); both against the position oracle too.  Sizes whose workspace
exceeds the static array are refused on the host with nothing launched."""
import ctypes

import numpy as np
import pytest

from oracle import positions_oracle as P
import workloads as W
from tests._helpers import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from vlm_multimodal_rotary_amd import _lib
    return _lib.load()


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).cuda()


def _grids(g):
    g = np.asarray(g, dtype=np.int32).reshape(-1, 3)
    return (_i32(g), g.shape[0]) if g.shape[0] else (None, 0)


def _call(lib, types, mask, images, videos, static):
    """One call of either entry point; returns (pos [3,B,L], delta, status)."""
    import torch
    from vlm_multimodal_rotary_amd import _lib
    B, L = types.shape
    td, md = _i32(types), _i32(mask)
    (gi, ni), (gv, nv) = _grids(images), _grids(videos)
    pos = torch.full((3, B * L), -7, dtype=torch.int32, device="cuda")
    delta = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    P_ = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if static:
        rc = lib.mrope_rope_index_noalloc(P_(td), P_(md), B, L, P_(gi), ni, P_(gv), nv, 2,
                                          P_(pos), B * L, P_(delta), P_(status), stream)
    else:
        ws_bytes = lib.mrope_rope_index_workspace_size(B, L, ni, nv)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        rc = lib.mrope_rope_index(P_(td), P_(md), B, L, P_(gi), ni, P_(gv), nv, 2, P_(pos), B * L,
                                  P_(delta), P_(status), P_(ws), ws_bytes, stream)
    _lib.check(rc)
    torch.cuda.synchronize()
    return pos.cpu().numpy().reshape(3, B, L), delta.cpu().numpy(), int(status.item())


def _batches():
    big = W.mm_prompt_batch("mm_prompt_positions")                  # 8 x 8192, two kernels
    rng = np.random.default_rng(91)
    t, m, i, v = W.random_mm_batch(rng, 3, 2500)                     # smaller, many runs
    return [("8x8192 prompts", big), ("3x2500 random", (t, m, i, v))]


def test_static_workspace_matches_caller_workspace_twice(lib):
    for what, (types, mask, images, videos) in _batches():
        note(f"rope_index_noalloc {what}")
        want, wd = P.get_rope_index(types, image_grid_thw=np.asarray(images).reshape(-1, 3),
                                    video_grid_thw=np.asarray(videos).reshape(-1, 3),
                                    attention_mask=mask)
        a_pos, a_delta, a_st = _call(lib, types, mask, images, videos, static=False)
        b_pos, b_delta, b_st = _call(lib, types, mask, images, videos, static=True)
        n_off = int(np.count_nonzero(a_pos != b_pos))
        print(f"[parity] {what}: {a_pos.size} positions, {n_off} differ between the entry "
              f"points", flush=True)
        assert a_st == 0 and b_st == 0
        assert n_off == 0 and np.array_equal(a_delta, b_delta)
        assert np.array_equal(b_pos, want) and np.array_equal(b_delta, wd)


def test_oversize_workspace_is_refused(lib):
    """n_images large enough that the advance tables alone exceed the static
    array: refused before any launch (the call returns an error code)."""
    import torch
    from vlm_multimodal_rotary_amd import _lib
    n_img = _lib.ROPE_INDEX_SCRATCH_BYTES // 8 + 16
    types = _i32(np.zeros((1, 64)))
    grids = _i32(np.ones((n_img, 3)))
    pos = torch.empty((3, 64), dtype=torch.int32, device="cuda")
    delta = torch.empty(1, dtype=torch.int32, device="cuda")
    status = torch.empty(1, dtype=torch.int32, device="cuda")
    assert lib.mrope_rope_index_workspace_size(1, 64, n_img, 0) > _lib.ROPE_INDEX_SCRATCH_BYTES
    P_ = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc = lib.mrope_rope_index_noalloc(P_(types), None, 1, 64, P_(grids), n_img, None, 0, 2,
                                      P_(pos), 64, P_(delta), P_(status), None)
    assert rc == _lib.MROPE_EUNSUPPORTED
    assert "static workspace" in lib.mrope_last_error().decode()
