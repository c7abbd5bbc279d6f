"""The Python binding checks every tensor before a pointer reaches the C ABI.

The C ABI sizes each buffer from the sizes passed to it (T, heads and D of q,
the element size of q's dtype), so a k, an output, a weight, a cache or a
cos/sin table that does not match them would be read or written out of
bounds on the GPU.  These CPU tests hand the binding "meta" tensors (shapes,
dtypes and strides without storage) in place of GPU tensors and a stand-in
library whose every entry point fails the test if it is reached: each
mismatch must raise MropeError(EINVAL) first, and a matching set of
arguments must get through to the library.
"""
import pytest
import torch

import vlm_multimodal_rotary_amd as M
from vlm_multimodal_rotary_amd import _lib


class Launched(Exception):
    pass


class FakeLib:
    """Every entry point raises Launched; the workspace size query answers."""

    def __getattr__(self, name):
        if name == "mrope_rope_index_workspace_size":
            return lambda *a: 4096
        if name == "mrope_last_error":
            return lambda: b""

        def entry(*args):
            raise Launched(name)
        return entry


@pytest.fixture
def meta(monkeypatch):
    monkeypatch.setattr(M, "_GPU_DEVICE_TYPES", ("meta",))
    monkeypatch.setattr(_lib, "_LIB", FakeLib())
    monkeypatch.setattr(M, "_stream", lambda t: None)
    monkeypatch.setattr(M, "_ptr", lambda t: None)

    def t(*shape, dtype=torch.bfloat16):
        return torch.empty(shape, dtype=dtype, device="meta")
    return t


T, HQ, HK, D = 8, 4, 2, 16
BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def fused_args(t):
    return dict(q=t(T, HQ, D), k=t(T, HK, D), pos=t(3, T, dtype=I32), wq=t(D), wk=t(D))


def call_fused(a, **over):
    a = dict(a, **over)
    return M.rmsnorm_mrope_qk(a.pop("q"), a.pop("k"), a.pop("pos"), D, 1e6, (4, 2, 2),
                              "interleaved", **a)


def expect_einval(fn):
    with pytest.raises(M.MropeError) as e:
        fn()
    assert e.value.code == _lib.MROPE_EINVAL


def test_fused_valid_arguments_reach_the_library(meta):
    with pytest.raises(Launched):
        call_fused(fused_args(meta))
    with pytest.raises(Launched):
        call_fused(fused_args(meta), wq=None, wk=None, q_out=meta(T, HQ, D), k_out=meta(T, HK, D))


@pytest.mark.parametrize("case", [
    "k_dtype", "k_tokens", "k_dim", "q_out_dtype", "q_out_shape", "k_out_tokens", "wq_dtype",
    "wq_length", "wq_strided", "only_wq", "pos_int64", "pos_tokens", "pos_axes", "pos_strided",
    "cache_freqs", "cache_dtype", "cache_pairs", "q_on_cpu", "k_on_cpu", "pos_on_cpu", "q_2d",
])
def test_fused_mismatch_raises_before_launch(meta, case):
    a = fused_args(meta)
    wide = meta(T, 2 * D)
    over = {
        "k_dtype": dict(k=meta(T, HK, D, dtype=F32)),
        "k_tokens": dict(k=meta(T - 1, HK, D)),
        "k_dim": dict(k=meta(T, HK, D + 2)),
        "q_out_dtype": dict(q_out=meta(T, HQ, D, dtype=F32)),
        "q_out_shape": dict(q_out=meta(T, HQ - 1, D)),
        "k_out_tokens": dict(k_out=meta(T - 1, HK, D)),
        "wq_dtype": dict(wq=meta(D, dtype=F32)),
        "wq_length": dict(wq=meta(D - 2)),
        "wq_strided": dict(wq=wide[0, ::2]),
        "only_wq": dict(wk=None),
        "pos_int64": dict(pos=meta(3, T, dtype=torch.int64)),
        "pos_tokens": dict(pos=meta(3, T - 1, dtype=I32)),
        "pos_axes": dict(pos=meta(2, T, dtype=I32)),
        "pos_strided": dict(pos=meta(3, 2 * T, dtype=I32)[:, ::2]),
        "cache_freqs": dict(cs_cache=meta(100, 7, 2, dtype=F32)),
        "cache_dtype": dict(cs_cache=meta(100, 8, 2)),
        "cache_pairs": dict(cs_cache=meta(100, 8, 3, dtype=F32)),
        "q_on_cpu": dict(q=torch.empty(T, HQ, D, dtype=BF)),
        "k_on_cpu": dict(k=torch.empty(T, HK, D, dtype=BF)),
        "pos_on_cpu": dict(pos=torch.empty(3, T, dtype=I32)),
        "q_2d": dict(q=meta(T, HQ * D)),
    }[case]
    expect_einval(lambda: call_fused(a, **over))


def test_apply_rotary_checks(meta):
    q, k = meta(T, HQ, D), meta(T, HK, D)
    c, s = meta(T, D, dtype=F32), meta(T, D, dtype=F32)
    with pytest.raises(Launched):
        M.apply_rotary_qk(q, k, c, s, D)
    expect_einval(lambda: M.apply_rotary_qk(q, k, meta(T, D), s, D))             # bf16 table
    expect_einval(lambda: M.apply_rotary_qk(q, k, meta(T, D - 2, dtype=F32), s, D))
    expect_einval(lambda: M.apply_rotary_qk(q, k, meta(D, T, dtype=F32).t(), s, D))
    expect_einval(lambda: M.apply_rotary_qk(q, k, c, meta(T, 2 * D, dtype=F32), D))  # strides
    expect_einval(lambda: M.apply_rotary_qk(q, k, meta(T + 1, D, dtype=F32), s, D))
    expect_einval(lambda: M.apply_rotary_qk(q, meta(T, HK, D, dtype=F32), c, s, D))


def test_decode_checks(meta):
    B, cap = 4, 32
    q, k = meta(B, HQ, D, dtype=F32), meta(B, HK, D, dtype=F32)
    cl, rd = meta(B, dtype=I32), meta(B, dtype=I32)
    cache = meta(B, cap, HK, D, dtype=F32)

    def call(**over):
        a = dict(q=q, k=k, cache_len=cl, rope_delta=rd, k_cache=cache)
        a.update(over)
        return M.mrope_decode_qk(a["q"], a["k"], a["cache_len"], a["rope_delta"], 1, D, 1e6,
                                 a["k_cache"])
    with pytest.raises(Launched):
        call()
    expect_einval(lambda: call(k_cache=meta(B, cap, HK, D)))              # bf16 cache, f32 q
    expect_einval(lambda: call(k_cache=meta(B, cap, HK + 1, D, dtype=F32)))
    expect_einval(lambda: call(k_cache=meta(B - 1, cap, HK, D, dtype=F32)))
    expect_einval(lambda: call(cache_len=meta(B, dtype=torch.int64)))
    expect_einval(lambda: call(rope_delta=meta(B - 1, dtype=I32)))
    expect_einval(lambda: call(cache_len=meta(B + 1, dtype=I32)))         # rows != batch
    expect_einval(lambda: call(k=meta(B, HK, D)))                         # k bf16


def test_vision_qkv_checks(meta):
    n, H, Dv = 16, 2, 8
    qkv = meta(n, 3, H, Dv, dtype=F32)
    pos = meta(2, n, dtype=I32)
    with pytest.raises(Launched):
        M.vision_qkv(qkv, pos, Dv, 1e4)
    expect_einval(lambda: M.vision_qkv(qkv, pos, Dv, 1e4, q_out=meta(H, n, Dv)))
    expect_einval(lambda: M.vision_qkv(qkv, pos, Dv, 1e4, v_out=meta(H, n - 1, Dv, dtype=F32)))
    expect_einval(lambda: M.vision_qkv(qkv, meta(3, n, dtype=I32), Dv, 1e4))
    expect_einval(lambda: M.vision_qkv(qkv, pos, Dv, 1e4, cs_cache=meta(50, 3, 2, dtype=F32)))


def test_rms_norm_checks(meta):
    x = meta(T, HQ, D)
    with pytest.raises(Launched):
        M.rms_norm(x, meta(D), 1e-6)
    expect_einval(lambda: M.rms_norm(x, meta(D, dtype=F32), 1e-6))
    expect_einval(lambda: M.rms_norm(x, meta(D), 1e-6, out=meta(T, HQ, D - 2)))


def test_rope_index_and_copy_checks(meta):
    B, L = 2, 32
    types, mask = meta(B, L, dtype=I32), meta(B, L, dtype=I32)
    grid = meta(1, 3, dtype=I32)
    pos, delta, status = meta(3, B * L, dtype=I32), meta(B, dtype=I32), meta(1, dtype=I32)
    ws = meta(4096, dtype=torch.uint8)
    with pytest.raises(Launched):
        M.rope_index_into(types, mask, grid, None, 2, pos, delta, status, ws)
    expect_einval(lambda: M.rope_index_into(types, mask, grid, None, 2, meta(3, L, dtype=I32),
                                            delta, status, ws))
    expect_einval(lambda: M.rope_index_into(types, meta(B, L - 1, dtype=I32), grid, None, 2, pos,
                                            delta, status, ws))
    expect_einval(lambda: M.rope_index_into(types, mask, meta(1, 2, dtype=I32), None, 2, pos,
                                            delta, status, ws))
    expect_einval(lambda: M.rope_index_into(types, mask, grid, None, 2, pos, delta, status,
                                            meta(1024, dtype=I32)))
    src = meta(64, dtype=torch.uint8)
    with pytest.raises(Launched):
        M.stream_copy(src, meta(64, dtype=torch.uint8))
    expect_einval(lambda: M.stream_copy(src, meta(32, dtype=torch.uint8)))
