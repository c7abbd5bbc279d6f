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


# bfloat16 planes of 2048 tokens or more take the staged kernel (rows through
# LDS a few tokens per block); token counts leave a ragged last block.
STAGED = [(2051, 16, 72, 72), (2100, 6, 128, 64), (2049, 5, 80, 48), (2053, 3, 16, 8)]


@pytest.mark.parametrize("n,H,D,rd", STAGED, ids=[f"n{n}-H{H}-D{D}-rd{r}" for n, H, D, r in STAGED])
def test_vision_qkv_staged_planes(M, n, H, D, rd):
    rng = np.random.default_rng(n * 3 + D)
    qkv = W._store(rng.standard_normal((n, 3, H, D)).astype(np.float32), "bf16")
    pos = rng.integers(0, 4096, (2, n)).astype(np.int32)
    note(f"vision_qkv staged bf16 n={n} H={H} D={D} rd={rd}")
    gq, gk, gv = _run(M, qkv, pos, "bf16", rd, 1e4)
    oq, ok, ov = O.vision_qkv(qkv, pos, rotary_dim=rd, theta=1e4, dtype="bf16")
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
    gq, gk, _ = _run(M, qkv, pos, "bf16", 72, 1e4, precision=precision)
    oq, ok, _ = O.vision_qkv(qkv, pos, rotary_dim=72, theta=1e4, dtype="bf16", precision=precision)
    assert np.array_equal(gq, oq) and np.array_equal(gk, ok)


def test_vision_qkv_staged_without_v_and_cached(M):
    """No v plane (two tensors), and cos/sin gathered from a cache that covers
    only part of the positions (the rest computed): same planes as without."""
    import torch
    rng = np.random.default_rng(75)
    n = 2222
    qkv = W._store(rng.standard_normal((n, 3, 16, 72)).astype(np.float32), "bf16")
    pos = rng.integers(0, 4096, (2, n)).astype(np.int32)
    note("vision_qkv staged without v, cos/sin cache of 3000 rows")
    gq, gk, gv = _run(M, qkv, pos, "bf16", 72, 1e4, with_v=False)
    oq, ok, _ = O.vision_qkv(qkv, pos, rotary_dim=72, theta=1e4, dtype="bf16")
    assert gv is None
    assert_close(gq, oq, "bf16", "staged q without v")
    assert_close(gk, ok, "bf16", "staged k without v")
    cache = M.mrope_cos_sin_cache(36, 1e4, 3000, device="cuda")   # vision: dim = rotary_dim / 2
    cq, ck, _ = _run(M, qkv, pos, "bf16", 72, 1e4, cs_cache=cache)
    assert np.array_equal(cq, gq) and np.array_equal(ck, gk)


def test_kernel_choice_by_shape(M):
    """bf16 planes of 2048+ tokens take the staged kernel, fp32 planes and
    token-major vision rows the flat one, short launches the general
    one."""
    import torch
    for dtype, n, head_major, want in [("bf16", 2048, True, "stage_kernel"),
                                       ("f32", 2048, True, "flat_kernel"),
                                       ("bf16", 2048, False, "flat_kernel"),
                                       ("bf16", 2047, True, "qk_kernel")]:
        qkv = torch.zeros((n, 3, 16, 72), dtype=torch.bfloat16 if dtype == "bf16"
                          else torch.float32, device="cuda")
        pos = torch.zeros((2, n), dtype=torch.int32, device="cuda")
        M.vision_qkv(qkv, pos, 72, 1e4, head_major=head_major)
        torch.cuda.synchronize()
        assert M.last_kernel() == want, (dtype, n, head_major, M.last_kernel())


def test_many_heads_fall_back_to_the_flat_kernel(M):
    """bf16 planes whose v rows of one token exceed the staged kernel's
    registers (96 heads of 72) take the flat kernel, with the same results."""
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
