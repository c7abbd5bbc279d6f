"""GPU parity of the vision qkv fusion (packed [n, 3, heads, D] -> rotated q,
k and copied v in per-head planes) against the CPU oracle.

Bars: as for the fused path (bf16 within 1 ulp, fp32 within 1e-5, v and
pass-through dims bit-exact); the kernel is expected to match bit for bit.
"""
import numpy as np
import pytest

from oracle import mrope_oracle as O
import workloads as W
from tests._helpers import assert_close, from_dev, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import vlm_multimodal_rotary_amd as lib
    lib.load()
    return lib


def _dev_qkv(qkv, dtype):
    n, _, H, D = qkv.shape
    return to_dev(qkv.reshape(n, 3 * H * D), dtype).reshape(n, 3, H, D)


def _run(M, qkv, pos, dtype, rd, theta, **kw):
    import torch
    q, k, v = M.vision_qkv(_dev_qkv(qkv, dtype), to_dev(pos, "i32"), rd, theta, **kw)
    torch.cuda.synchronize()
    return from_dev(q), from_dev(k), None if v is None else from_dev(v)


@pytest.mark.parametrize("dtype,n,H,D,rd", [("f32", 777, 16, 72, 72), ("bf16", 777, 16, 72, 72),
                                             ("bf16", 300, 6, 128, 64), ("f32", 129, 5, 80, 80),
                                             ("bf16", 1, 4, 72, 72)])
def test_vision_qkv_planes(M, dtype, n, H, D, rd):
    rng = np.random.default_rng(n + D)
    qkv = W._store(rng.standard_normal((n, 3, H, D)).astype(np.float32), dtype)
    pos = W.vision_patch_positions(1, 64, 64)[:, :n].astype(np.int32)
    note(f"vision_qkv {dtype} n={n} H={H} D={D} rd={rd}")
    gq, gk, gv = _run(M, qkv, pos, dtype, rd, 1e4)
    oq, ok, ov = O.vision_qkv(qkv, pos, rotary_dim=rd, theta=1e4, dtype=dtype)
    assert_close(gq, oq, dtype, "vision q planes")
    assert_close(gk, ok, dtype, "vision k planes")
    assert np.array_equal(gv.view(np.uint8), ov.view(np.uint8))


@pytest.mark.parametrize("precision", ["dtype", "fp32"])
def test_vision_qkv_precisions_bit_exact(M, precision):
    rng = np.random.default_rng(71)
    qkv = W._store(rng.standard_normal((500, 3, 16, 72)).astype(np.float32), "bf16")
    pos = W.vision_patch_positions(1, 64, 64)[:, 1000:1500].astype(np.int32)
    note(f"vision_qkv precision {precision}")
    gq, gk, _ = _run(M, qkv, pos, "bf16", 72, 1e4, precision=precision)
    oq, ok, _ = O.vision_qkv(qkv, pos, rotary_dim=72, theta=1e4, dtype="bf16", precision=precision)
    assert np.array_equal(gq, oq) and np.array_equal(gk, ok)


def test_vision_qkv_token_major_and_without_v(M):
    rng = np.random.default_rng(72)
    qkv = W._store(rng.standard_normal((400, 3, 16, 72)).astype(np.float32), "f32")
    pos = W.vision_patch_positions(1, 64, 64)[:, :400].astype(np.int32)
    note("vision_qkv token-major, no v")
    gq, gk, gv = _run(M, qkv, pos, "f32", 72, 1e4, head_major=False, with_v=False)
    oq, ok, _ = O.vision_qkv(qkv, pos, rotary_dim=72, theta=1e4, dtype="f32")
    assert gv is None
    assert_close(gq, oq.transpose(1, 0, 2), "f32", "token-major q")
    assert_close(gk, ok.transpose(1, 0, 2), "f32", "token-major k")


def test_vision_qkv_equals_the_fused_path(M):
    """The planes hold exactly what rmsnorm_mrope_qk writes for the same q/k
    views of the packed buffer (vision layout), transposed."""
    import torch
    wl = W.VISION_QKV_WORKLOADS["vision_qkv_planes"]
    inp = W.make_vision_qkv_inputs(wl, n=3000)
    qkv = _dev_qkv(inp["qkv"], wl.dtype)
    pos = to_dev(inp["pos"], "i32")
    q, k, v = M.vision_qkv(qkv, pos, wl.rotary_dim, wl.theta)
    fq, fk = M.rmsnorm_mrope_qk(qkv[:, 0], qkv[:, 1], pos, wl.rotary_dim, wl.theta, None,
                                "vision_2d")
    torch.cuda.synchronize()
    assert torch.equal(q, fq.transpose(0, 1)) and torch.equal(k, fk.transpose(0, 1))
    assert torch.equal(v, qkv[:, 2].transpose(0, 1))


def test_vision_qkv_empty(M):
    import torch
    qkv = torch.empty((0, 3, 16, 72), dtype=torch.float32, device="cuda")
    q, k, v = M.vision_qkv(qkv, torch.empty((2, 0), dtype=torch.int32, device="cuda"), 72, 1e4)
    torch.cuda.synchronize()
    assert q.shape == (16, 0, 72)


# Planes of 2048 tokens or more with full rotary take the group kernel (a
# block per few tokens x every plane, chunks in output order); token counts
# leave a ragged last group.  D = 72 (bf16) and D = 36 (fp32) have a chunk
# that straddles the rotary half.
GROUP = [("bf16", 2051, 16, 72), ("f32", 2049, 16, 72), ("bf16", 2050, 8, 128),
         ("f32", 2050, 16, 36), ("bf16", 2053, 24, 256), ("bf16", 2048, 1, 16),
         ("f32", 4099, 21, 72), ("bf16", 2099, 21, 72)]


@pytest.mark.parametrize("dtype,n,H,D", GROUP, ids=[f"{d}-n{n}-H{H}-D{D}" for d, n, H, D in GROUP])
def test_vision_qkv_group_kernel_planes(M, dtype, n, H, D):
    rng = np.random.default_rng(n * 5 + D + H)
    qkv = W._store(rng.standard_normal((n, 3, H, D)).astype(np.float32), dtype)
    pos = rng.integers(-3000, 60000, (2, n)).astype(np.int32)
    note(f"vision_qkv group kernel {dtype} n={n} H={H} D={D}")
    gq, gk, gv = _run(M, qkv, pos, dtype, D, 1e4)
    assert M.last_kernel() == "planes_kernel"
    oq, ok, ov = O.vision_qkv(qkv, pos, rotary_dim=D, theta=1e4, dtype=dtype)
    assert_close(gq, oq, dtype, "group q planes")
    assert_close(gk, ok, dtype, "group k planes")
    assert np.array_equal(gv.view(np.uint8), ov.view(np.uint8))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_vision_qkv_group_kernel_variants(M, dtype):
    """The group kernel without v, with a cos/sin cache that covers part of
    the positions, and in the tensor-op precisions: every element against
    the oracle."""
    rng = np.random.default_rng(77 if dtype == "bf16" else 78)
    n = 2222
    qkv = W._store(rng.standard_normal((n, 3, 16, 72)).astype(np.float32), dtype)
    pos = rng.integers(0, 4096, (2, n)).astype(np.int32)
    note(f"vision_qkv group kernel {dtype}: no v, cache, precisions")
    gq, gk, gv = _run(M, qkv, pos, dtype, 72, 1e4, with_v=False)
    assert M.last_kernel() == "planes_kernel" and gv is None
    oq, ok, _ = O.vision_qkv(qkv, pos, rotary_dim=72, theta=1e4, dtype=dtype)
    assert_close(gq, oq, dtype, "group q without v")
    assert_close(gk, ok, dtype, "group k without v")
    cache = M.mrope_cos_sin_cache(36, 1e4, 1500, device="cuda")   # part of [0, 4096)
    cq, ck, _ = _run(M, qkv, pos, dtype, 72, 1e4, cs_cache=cache)
    assert M.last_kernel() == "planes_kernel"
    assert np.array_equal(cq, gq) and np.array_equal(ck, gk)
    for precision in (["dtype", "fp32"] if dtype == "bf16" else ["fp32"]):
        pq, pk, _ = _run(M, qkv, pos, dtype, 72, 1e4, precision=precision)
        assert M.last_kernel() == "planes_kernel"
        wq, wk, _ = O.vision_qkv(qkv, pos, rotary_dim=72, theta=1e4, dtype=dtype,
                                 precision=precision)
        assert np.array_equal(pq.view(np.uint8), wq.view(np.uint8)), precision
        assert np.array_equal(pk.view(np.uint8), wk.view(np.uint8)), precision


# bfloat16 planes of 2048 tokens or more with partial rotary take the staged
# kernel (rows through LDS a few tokens per block); token counts leave a
# ragged last block.
STAGED = [(2100, 6, 128, 64), (2049, 5, 80, 48), (2053, 3, 16, 8), (2051, 16, 72, 64)]


@pytest.mark.parametrize("n,H,D,rd", STAGED, ids=[f"n{n}-H{H}-D{D}-rd{r}" for n, H, D, r in STAGED])
def test_vision_qkv_staged_planes(M, n, H, D, rd):
    rng = np.random.default_rng(n * 3 + D)
    qkv = W._store(rng.standard_normal((n, 3, H, D)).astype(np.float32), "bf16")
    pos = rng.integers(0, 4096, (2, n)).astype(np.int32)
    note(f"vision_qkv staged bf16 n={n} H={H} D={D} rd={rd}")
    gq, gk, gv = _run(M, qkv, pos, "bf16", rd, 1e4)
    oq, ok, ov = O.vision_qkv(qkv, pos, rotary_dim=rd, theta=1e4, dtype="bf16")
    assert M.last_kernel() == "stage_kernel"
    assert_close(gq, oq, "bf16", "staged q planes")
    assert_close(gk, ok, "bf16", "staged k planes")
    assert np.array_equal(gv.view(np.uint8), ov.view(np.uint8))
    assert np.array_equal(gq[..., rd:], qkv[:, 0, :, rd:].transpose(1, 0, 2))


@pytest.mark.parametrize("precision", ["dtype", "fp32"])
def test_vision_qkv_staged_precisions_bit_exact(M, precision):
    rng = np.random.default_rng(74)
    n = 2500
    qkv = W._store(rng.standard_normal((n, 3, 16, 72)).astype(np.float32), "bf16")
    pos = rng.integers(0, 4096, (2, n)).astype(np.int32)
    note(f"vision_qkv staged precision {precision}")
    gq, gk, _ = _run(M, qkv, pos, "bf16", 64, 1e4, precision=precision)
    assert M.last_kernel() == "stage_kernel"
    oq, ok, _ = O.vision_qkv(qkv, pos, rotary_dim=64, theta=1e4, dtype="bf16", precision=precision)
    assert np.array_equal(gq, oq) and np.array_equal(gk, ok)


def test_vision_qkv_staged_without_v_and_cached(M):
    """Partial rotary on the staged kernel: no v plane (two tensors), and
    cos/sin gathered from a cache that covers only part of the positions
    (the rest computed): same planes as without."""
    import torch
    rng = np.random.default_rng(75)
    n = 2222
    qkv = W._store(rng.standard_normal((n, 3, 16, 72)).astype(np.float32), "bf16")
    pos = rng.integers(0, 4096, (2, n)).astype(np.int32)
    note("vision_qkv staged without v, cos/sin cache of 3000 rows")
    gq, gk, gv = _run(M, qkv, pos, "bf16", 64, 1e4, with_v=False)
    assert M.last_kernel() == "stage_kernel"
    oq, ok, _ = O.vision_qkv(qkv, pos, rotary_dim=64, theta=1e4, dtype="bf16")
    assert gv is None
    assert_close(gq, oq, "bf16", "staged q without v")
    assert_close(gk, ok, "bf16", "staged k without v")
    cache = M.mrope_cos_sin_cache(32, 1e4, 3000, device="cuda")   # vision: dim = rotary_dim / 2
    cq, ck, _ = _run(M, qkv, pos, "bf16", 64, 1e4, cs_cache=cache)
    assert np.array_equal(cq, gq) and np.array_equal(ck, gk)


def test_kernel_choice_by_shape(M):
    """Planes of 2048+ tokens with full rotary take the group kernel; with
    partial rotary, bf16 planes the staged kernel and fp32 planes the flat
    one; token-major vision rows the flat one; short launches the general
    one."""
    import torch
    for dtype, n, head_major, rd, want in [("bf16", 2048, True, 72, "planes_kernel"),
                                           ("f32", 2048, True, 72, "planes_kernel"),
                                           ("bf16", 2048, True, 64, "stage_kernel"),
                                           ("f32", 2048, True, 64, "flat_kernel"),
                                           ("bf16", 2048, False, 72, "flat_kernel"),
                                           ("bf16", 2047, True, 72, "qk_kernel")]:
        qkv = torch.zeros((n, 3, 16, 72), dtype=torch.bfloat16 if dtype == "bf16"
                          else torch.float32, device="cuda")
        pos = torch.zeros((2, n), dtype=torch.int32, device="cuda")
        M.vision_qkv(qkv, pos, rd, 1e4, head_major=head_major)
        torch.cuda.synchronize()
        assert M.last_kernel() == want, (dtype, n, head_major, rd, M.last_kernel())


def test_many_heads_fall_back_to_the_flat_kernel(M):
    """bf16 planes whose rows exceed the group kernel's block and the staged
    kernel's registers (96 heads of 72) take the flat kernel, with the same
    results."""
    rng = np.random.default_rng(76)
    n, H = 2048, 96
    qkv = W._store(rng.standard_normal((n, 3, H, 72)).astype(np.float32), "bf16")
    pos = rng.integers(0, 4096, (2, n)).astype(np.int32)
    note("vision_qkv bf16 96 heads (flat fallback)")
    gq, gk, gv = _run(M, qkv, pos, "bf16", 72, 1e4)
    assert M.last_kernel() == "flat_kernel"
    rows = np.array([0, 1, 777, n - 1])
    oq, ok, ov = O.vision_qkv(qkv[rows], pos[:, rows], rotary_dim=72, theta=1e4, dtype="bf16")
    assert_close(gq[:, rows], oq, "bf16", "fallback q")
    assert_close(gk[:, rows], ok, "bf16", "fallback k")
    assert np.array_equal(gv[:, rows].view(np.uint8), ov.view(np.uint8))
