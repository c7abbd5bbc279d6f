"""GPU: the cos/sin cache by position (builder against the oracle, bit-exact)
and the cached fused paths against the computing ones (bit-identical)."""
import numpy as np
import pytest

from oracle import mrope_oracle as O
import workloads as W
from tests._helpers import from_dev, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import vlm_multimodal_rotary_amd as lib
    lib.load()
    return lib


@pytest.mark.parametrize("dim,theta,rows", [(128, 1e6, 40000), (64, 1e7, 3000), (36, 1e4, 128),
                                            (16, 1e4, 1)])
def test_cache_builder_matches_oracle(M, dim, theta, rows):
    import torch
    note(f"cos_sin_cache dim={dim} rows={rows}")
    got = M.mrope_cos_sin_cache(dim, theta, rows)
    torch.cuda.synchronize()
    want = O.cos_sin_cache(dim, theta, rows)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


def _fused(M, wl, inp, cache=None, pos=None):
    import torch
    qd, kd = to_dev(inp["q"], wl.dtype), to_dev(inp["k"], wl.dtype)
    pd = to_dev(inp["pos"] if pos is None else pos, "i32")
    wq = to_dev(inp["wq"], wl.dtype) if wl.norm else None
    wk = to_dev(inp["wk"], wl.dtype) if wl.norm else None
    qo, ko = M.rmsnorm_mrope_qk(qd, kd, pd, wl.rotary_dim, wl.theta, wl.section, wl.layout,
                                wq=wq, wk=wk, eps=wl.eps, cs_cache=cache)
    torch.cuda.synchronize()
    return from_dev(qo), from_dev(ko)


def _cache_for(M, wl, rows):
    dim = wl.rotary_dim // 2 if wl.layout == "vision_2d" else wl.rotary_dim
    return M.mrope_cos_sin_cache(dim, wl.theta, rows)


@pytest.mark.parametrize("name,T", [("tiny_mrope", None), ("omni_text_prefill", 2000),
                                    ("qwen35_partial_mixed", 1400), ("chunked_video", 700),
                                    ("vision_2d", 4500)])
def test_cached_fused_equals_computed(M, name, T):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, T=T)
    rows = int(inp["pos"].max()) + 1
    note(f"cached fused {name} rows={rows}")
    a = _fused(M, wl, inp)
    b = _fused(M, wl, inp, cache=_cache_for(M, wl, rows))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # a cache that covers only part of the positions: the rest are computed
    c = _fused(M, wl, inp, cache=_cache_for(M, wl, max(1, rows // 3)))
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


@pytest.mark.parametrize("name,T", [("omni_text_prefill", 2048), ("qwen35_partial_mixed", 2100),
                                    ("chunked_video", 2500)])
def test_cached_pipelined_kernel_partial_cache(M, name, T):
    # 2048 tokens or more take the pipelined kernel; a cache that covers part
    # of the positions sends some lanes of a wavefront to the cache and the
    # rest to the sincos (image and video segments: the axes differ).
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, T=T)
    rows = int(inp["pos"].max()) + 1
    note(f"cached pipelined {name} T={T} rows={rows}")
    a = _fused(M, wl, inp)
    assert M.last_kernel() == "qk_pipe_kernel"
    for r in (rows, max(1, rows // 3), max(1, (2 * rows) // 3)):
        b = _fused(M, wl, inp, cache=_cache_for(M, wl, r))
        assert M.last_kernel() == "qk_pipe_kernel"
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), r
    qo, ko = O.rmsnorm_mrope_qk(inp["q"], inp["k"], inp["pos"], rotary_dim=wl.rotary_dim,
                                theta=wl.theta, section=wl.section, layout=wl.layout,
                                wq=inp["wq"], wk=inp["wk"], eps=wl.eps, dtype=wl.dtype)
    assert np.array_equal(b[0], qo) and np.array_equal(b[1], ko)


def test_cached_fused_negative_and_large_positions(M):
    wl = W.WORKLOADS["omni_text_prefill"]
    inp = W.make_inputs(wl, T=512)
    rng = np.random.default_rng(80)
    pos = rng.integers(-5000, 200000, (3, 512)).astype(np.int32)
    note("cached fused, positions outside the cache")
    a = _fused(M, wl, inp, pos=pos)
    b = _fused(M, wl, inp, cache=_cache_for(M, wl, 100000), pos=pos)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    qo, ko = O.rmsnorm_mrope_qk(inp["q"], inp["k"], pos, rotary_dim=wl.rotary_dim, theta=wl.theta,
                                section=wl.section, layout=wl.layout, wq=inp["wq"], wk=inp["wk"],
                                eps=wl.eps, dtype=wl.dtype)
    assert np.array_equal(b[0], qo) and np.array_equal(b[1], ko)


def test_cached_full_size_headline(M):
    wl = W.WORKLOADS["omni_text_prefill"]
    inp = W.make_inputs(wl)
    note("cached fused full omni")
    a = _fused(M, wl, inp)
    b = _fused(M, wl, inp, cache=_cache_for(M, wl, wl.T))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_cached_vision_qkv(M):
    import torch
    wl = W.VISION_QKV_WORKLOADS["vision_qkv_planes_bf16"]
    inp = W.make_vision_qkv_inputs(wl, n=5000)
    n = inp["T"]
    qkv = to_dev(inp["qkv"].reshape(n, -1), wl.dtype).reshape(n, 3, wl.heads, wl.D)
    pos = to_dev(inp["pos"], "i32")
    cache = M.mrope_cos_sin_cache(wl.rotary_dim // 2, wl.theta, 64)
    note("cached vision qkv")
    a = M.vision_qkv(qkv, pos, wl.rotary_dim, wl.theta)
    b = M.vision_qkv(qkv, pos, wl.rotary_dim, wl.theta, cs_cache=cache)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
