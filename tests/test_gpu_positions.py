"""GPU parity of the position builders against the position oracle: the
3-axis table and rope_deltas (get_rope_index) and the vision patch
coordinates (rot_pos_emb order).  Integer results: bit-exact."""
import numpy as np
import pytest

from oracle import positions_oracle as P
import workloads as W
from tests._helpers import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import vlm_multimodal_rotary_amd as lib
    lib.load()
    return lib


def _i32(a):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return torch.from_numpy(a).cuda()


def _grid_arg(g):
    return None if g is None or len(g) == 0 else _i32(np.asarray(g).reshape(-1, 3))


def _run(M, types, images, videos, mask, merge=2, check=True):
    import torch
    B, L = types.shape
    pos, delta, status = M.rope_index(_i32(types), _grid_arg(images), _grid_arg(videos),
                                      None if mask is None else _i32(mask), merge=merge,
                                      check=check)
    torch.cuda.synchronize()
    return (pos.cpu().numpy().reshape(3, B, L), delta.cpu().numpy(), int(status.item()))


def _compare(M, types, images, videos, mask, what):
    note(f"rope_index {what} B={types.shape[0]} L={types.shape[1]}")
    want, wd = P.get_rope_index(types, image_grid_thw=images or None,
                                video_grid_thw=videos or None, attention_mask=mask)
    got, gd, st = _run(M, types, images, videos, mask)
    assert st == 0
    n_off = int(np.count_nonzero(got != want))
    print(f"[parity] {what}: {got.size} positions, {n_off} differ; deltas {gd.tolist()[:4]}",
          flush=True)
    assert n_off == 0
    assert np.array_equal(gd, wd)


def test_printed_table(M):
    types = np.array([[0, 0, 1, 1, 1, 1, 1, 1, 0, 0]])
    got, gd, st = _run(M, types, [(1, 4, 6)], None, None)
    assert got[0, 0].tolist() == [0, 1, 2, 2, 2, 2, 2, 2, 5, 6]
    assert got[1, 0].tolist() == [0, 1, 2, 2, 2, 3, 3, 3, 5, 6]
    assert got[2, 0].tolist() == [0, 1, 2, 3, 4, 2, 3, 4, 5, 6]
    assert gd.tolist() == [-3] and st == 0


@pytest.mark.parametrize("seed,B,L", [(0, 1, 300), (1, 3, 1000), (2, 8, 777), (3, 2, 4096),
                                      (4, 2, 4097), (5, 4, 9000), (6, 1, 40000), (7, 16, 257)])
def test_random_batches(M, seed, B, L):
    rng = np.random.default_rng(500 + seed)
    types, mask, images, videos = W.random_mm_batch(rng, B, L)
    _compare(M, types, images, videos, mask, f"random seed {seed}")


def _image_run_batch(n_images, L):
    """One sample: n_images 4x4 images (four merged slots each, advance 2)
    each after a text token, then text to length L."""
    types = np.zeros((1, L), dtype=np.int64)
    for k in range(n_images):
        types[0, 5 * k + 1:5 * k + 5] = 1
    return types, [(1, 4, 4)] * n_images


@pytest.mark.parametrize("case", ["small", "many_grids", "many_chunks", "grids_at_limit",
                                  "grids_past_limit", "chunks_at_limit", "chunks_past_limit"])
def test_pass_forms(M, case):
    """Passes 2 and 3 run as one kernel when the chunk summaries and grids fit
    LDS (up to 1024 chunks, 256 grids of a type), else as two kernels; both
    forms give the oracle's table, on both sides of each limit."""
    rng = np.random.default_rng(900)
    if case in ("grids_at_limit", "grids_past_limit"):
        n = 256 if case == "grids_at_limit" else 257
        types, images = _image_run_batch(n, 3000)
        mask, videos = None, []
        want = "rope_index_fused" if n == 256 else "rope_index_carry+apply"
    elif case in ("chunks_at_limit", "chunks_past_limit"):
        L = 1024 * 1024 + (0 if case == "chunks_at_limit" else 1)
        types, images = _image_run_batch(3, L)
        mask, videos = None, []
        want = "rope_index_fused" if case == "chunks_at_limit" else "rope_index_carry+apply"
    elif case == "small":
        types, mask, images, videos = W.random_mm_batch(rng, 2, 600)
        want = "rope_index_fused"
        assert len(images) <= 256 and len(videos) <= 256
    elif case == "many_grids":
        types, mask, images, videos = W.random_mm_batch(rng, 4, 4000)
        want = "rope_index_carry+apply"
        assert len(images) > 256 or len(videos) > 256
    else:
        L = 600000   # 2 x 586 chunks of 1024 tokens
        types = np.zeros((2, L), dtype=np.int64)
        types[0, 1000:1012] = 1
        types[1, 5000:5006] = 1
        mask = np.ones((2, L), dtype=np.int64)
        mask[1, :3000] = 0
        images, videos = [(1, 6, 8), (1, 4, 6)], []
        want = "rope_index_carry+apply"
    _compare(M, types, images, videos, mask, f"pass form {case}")
    assert M.last_kernel() == want


def test_workload_layouts_and_no_mask(M):
    """The mixed and video workloads' segment lists, without a mask; the GPU
    table equals both the oracle and the workload generator's table."""
    import torch
    for segs in ([("text", 512), ("image", (1, 48, 64)), ("text", 16384 - 512 - 768)],
                 [("text", 1024), ("image", (16, 48, 48)), ("text", 1024)]):
        types, grids = [], []
        for kind, arg in segs:
            if kind == "text":
                types += [0] * arg
            else:
                types += [1] * (arg[0] * (arg[1] // 2) * (arg[2] // 2))
                grids.append(arg)
        types = np.array([types])
        _compare(M, types, grids, None, None, f"segments {len(types[0])}")
        got, gd, _ = _run(M, types, grids, None, None)
        want, wd = W.rope_index(segs)
        assert np.array_equal(got[:, 0], want) and int(gd[0]) == wd


def test_edge_cases(M):
    # all-padding sample between two valid ones; text only; a sample of one token
    types = np.zeros((3, 50), dtype=np.int64)
    mask = np.ones((3, 50), dtype=np.int64)
    mask[1] = 0
    mask[2, 1:] = 0
    _compare(M, types, [], [], mask, "padding edge cases")
    # empty sequences: rope_delta 0 for every sample, nothing else written
    import torch
    pos, delta, status = M.rope_index(torch.zeros((3, 0), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert pos.shape == (3, 0) and delta.cpu().tolist() == [0, 0, 0]
    assert int(status.item()) == 0


def test_status_flags(M):
    """Inputs the walkthrough cannot build are reported in the status word
    (every access stays inside the buffers; positions are then unspecified)."""
    cases = [
        (np.array([[0, 1, 1, 1, 1, 0]]), [], W_FLAG_NO_GRID),
        (np.array([[0, 1, 1, 1, 0, 0]]), [(1, 4, 4)], W_FLAG_LENGTH),     # 3 tokens, 4 slots
        (np.array([[1, 1, 1, 1, 1, 0]]), [(1, 4, 4)], W_FLAG_LENGTH),     # 5 tokens
        (np.array([[0, 0, 1, 1, 1]]), [(1, 4, 4)], W_FLAG_LENGTH),        # short at the end
        (np.array([[0, 3, 0]]), [], W_FLAG_BAD_TYPE),
        (np.array([[0, 1, 1, 0]]), [(1, 1, 4)], W_FLAG_NO_GRID),          # h < merge
    ]
    for types, imgs, flag in cases:
        note(f"status {types.tolist()} {imgs}")
        _, _, st = _run(M, types, imgs, None, None, check=False)
        assert st & flag, (types.tolist(), imgs, st)
    with pytest.raises(M.MropeError):
        _run(M, np.array([[0, 1, 1, 1, 1]]), [], None, None, check=True)


W_FLAG_BAD_TYPE, W_FLAG_NO_GRID, W_FLAG_LENGTH = 1, 2, 4


@pytest.mark.parametrize("grids", [[(1, 4, 4)], [(1, 64, 64)] * 8, [(2, 6, 10), (1, 4, 8), (3, 2, 2)],
                                   [(1, 28, 40)] * 300])
def test_vision_pos_ids(M, grids):
    import torch
    want = P.vision_pos_ids(grids)
    n = want.shape[1]
    note(f"vision_pos_ids {len(grids)} grids, {n} patches")
    pos, status = M.vision_pos_ids(_i32(grids), n)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(pos.cpu().numpy(), want)


def test_vision_pos_ids_flags(M):
    import torch
    pos, status = M.vision_pos_ids(_i32([(1, 4, 4)]), 20, check=False)   # 16 patches, 20 slots
    torch.cuda.synchronize()
    assert int(status.item()) & 16
    assert np.array_equal(pos.cpu().numpy()[:, :16], P.vision_pos_ids([(1, 4, 4)]))
    assert np.all(pos.cpu().numpy()[:, 16:] == 0)
    pos, status = M.vision_pos_ids(_i32([(1, 5, 4)]), 20, check=False)
    torch.cuda.synchronize()
    assert int(status.item()) & 8


def test_positions_feed_the_fused_path(M):
    """GPU-built positions drive the fused kernel to the same result as the
    oracle's positions (the builder's output layout is the rotation's input)."""
    import torch
    from tests._helpers import from_dev, to_dev
    rng = np.random.default_rng(600)
    types, mask, images, videos = W.random_mm_batch(rng, 2, 700)
    pos, _, _ = M.rope_index(_i32(types), _grid_arg(images), _grid_arg(videos), _i32(mask))
    want, _ = P.get_rope_index(types, image_grid_thw=images or None,
                               video_grid_thw=videos or None, attention_mask=mask)
    T = 2 * 700
    q, k = W.random_qk(rng, T, 8, 2, 128, "bf16")
    qd, kd = to_dev(q, "bf16"), to_dev(k, "bf16")
    a, _ = M.rmsnorm_mrope_qk(qd, kd, pos, 128, 1e6, (24, 20, 20), "interleaved")
    b, _ = M.rmsnorm_mrope_qk(qd, kd, _i32(want.reshape(3, T)), 128, 1e6, (24, 20, 20),
                              "interleaved")
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(a), from_dev(b))
