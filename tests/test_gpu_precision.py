"""GPU parity of the tensor-operation rotation precisions ("dtype": cos/sin
cast to the tensor dtype and every operation rounded to it; "fp32": binary32
operations and one cast at the end) against the CPU oracle.

These modes exist for bit-compatibility with a framework's tensor arithmetic,
so the bar is bit-identical outputs, not a tolerance.
"""
import numpy as np
import pytest

from oracle import mrope_oracle as O
import workloads as W
from tests._helpers import from_dev, note, to_dev

pytestmark = pytest.mark.gpu

MODES = ("dtype", "fp32")


@pytest.fixture(scope="module")
def M():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import vlm_multimodal_rotary_amd as lib
    lib.load()
    return lib


def _assert_bits(got, want, what):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    g = got.view(np.uint16 if got.dtype == np.uint16 else np.uint32)
    w = want.view(np.uint16 if want.dtype == np.uint16 else np.uint32)
    n_off = int(np.count_nonzero(g != w))
    print(f"[parity] {what}: {g.size} values, {n_off} not bit-equal", flush=True)
    assert n_off == 0, f"{what}: {n_off} values differ"


def _fused_dev(M, inp, wl, precision, rows=None):
    import torch
    q, k, pos = inp["q"], inp["k"], inp["pos"]
    qd, kd = to_dev(q, wl.dtype), to_dev(k, wl.dtype)
    pd = to_dev(pos, "i32")
    wq = to_dev(inp["wq"], wl.dtype) if wl.norm else None
    wk = to_dev(inp["wk"], wl.dtype) if wl.norm else None
    qo, ko = M.rmsnorm_mrope_qk(qd, kd, pd, wl.rotary_dim, wl.theta, wl.section, wl.layout,
                                wq=wq, wk=wk, eps=wl.eps, precision=precision)
    torch.cuda.synchronize()
    return from_dev(qo), from_dev(ko)


def _fused_oracle(inp, wl, precision, rows=None):
    q, k, pos = inp["q"], inp["k"], inp["pos"]
    if rows is not None:
        q, k, pos = q[rows], k[rows], pos[:, rows]
    return O.rmsnorm_mrope_qk(q, k, pos, rotary_dim=wl.rotary_dim, theta=wl.theta,
                              section=wl.section, layout=wl.layout,
                              wq=inp["wq"] if wl.norm else None,
                              wk=inp["wk"] if wl.norm else None, eps=wl.eps, dtype=wl.dtype,
                              precision=precision)


WINDOWS = [("tiny_mrope", None), ("omni_text_prefill", 777), ("qwen35_partial_mixed", 1400),
           ("chunked_video", 700), ("vision_2d", 4500)]


@pytest.mark.parametrize("precision", MODES)
@pytest.mark.parametrize("name,T", WINDOWS, ids=[n for n, _ in WINDOWS])
def test_fused_windows_bit_exact(M, name, T, precision):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, T=T)
    note(f"fused {name} T={inp['T']} precision={precision}")
    gq, gk = _fused_dev(M, inp, wl, precision)
    oq, ok = _fused_oracle(inp, wl, precision)
    _assert_bits(gq, oq, f"{name} q {precision}")
    _assert_bits(gk, ok, f"{name} k {precision}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("precision", MODES)
def test_apply_rotary_tables_bit_exact(M, dtype, precision):
    """Caller cos/sin tables, partial rotary with pass-through lanes."""
    import torch
    rng = np.random.default_rng(310)
    T, hq, hk, D, rd = 257, 6, 2, 96, 64
    q, k = W.random_qk(rng, T, hq, hk, D, dtype)
    pos = rng.integers(0, 300000, (3, T)).astype(np.int32)
    cos, sin = O.mrope_cos_sin(pos, O.inv_freq(rd, 1e6), (16, 8, 8), "interleaved", rd)
    note(f"apply_rotary {dtype} {precision}")
    qd, kd = to_dev(q, dtype), to_dev(k, dtype)
    cd, sd = to_dev(cos, "f32"), to_dev(sin, "f32")
    gq, gk = M.apply_rotary_qk(qd, kd, cd, sd, rd, precision=precision)
    torch.cuda.synchronize()
    oq, ok = O.apply_rotary_qk(q, k, cos, sin, rd, dtype, precision)
    _assert_bits(from_dev(gq), oq, f"apply_rotary q {dtype} {precision}")
    _assert_bits(from_dev(gk), ok, f"apply_rotary k {dtype} {precision}")


def test_fused_equals_composition_in_every_precision(M):
    import torch
    for name in ("omni_text_prefill", "qwen35_partial_mixed", "vision_2d"):
        wl = W.WORKLOADS[name]
        inp = W.make_inputs(wl, T=500)
        qd, kd = to_dev(inp["q"], wl.dtype), to_dev(inp["k"], wl.dtype)
        pd = to_dev(inp["pos"], "i32")
        wq = to_dev(inp["wq"], wl.dtype) if wl.norm else None
        wk = to_dev(inp["wk"], wl.dtype) if wl.norm else None
        nq = M.rms_norm(qd, wq, wl.eps) if wl.norm else qd
        nk = M.rms_norm(kd, wk, wl.eps) if wl.norm else kd
        half = wl.rotary_dim // 2
        inv = M.mrope_inv_freq(half if wl.layout == "vision_2d" else wl.rotary_dim, wl.theta)
        c, s = M.mrope_cos_sin(pd, inv, wl.section, wl.layout, wl.rotary_dim)
        for precision in MODES:
            note(f"fused vs composition {name} {precision}")
            fq, fk = M.rmsnorm_mrope_qk(qd, kd, pd, wl.rotary_dim, wl.theta, wl.section,
                                        wl.layout, wq=wq, wk=wk, eps=wl.eps, precision=precision)
            cq, ck = M.apply_rotary_qk(nq, nk, c, s, wl.rotary_dim, precision=precision)
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(fq), from_dev(cq)), (name, precision)
            assert np.array_equal(from_dev(fk), from_dev(ck)), (name, precision)


def test_modes_differ_on_the_gpu_as_in_the_oracle(M):
    """The three precisions are distinct computations for bf16 (the check has
    teeth), and "dtype" and "fp32" coincide for binary32."""
    wl = W.WORKLOADS["omni_text_prefill"]
    inp = W.make_inputs(wl, T=2048)
    outs = {p: _fused_dev(M, inp, wl, p)[0] for p in O.PRECISIONS}
    assert np.count_nonzero(outs["exact"] != outs["dtype"]) > 0
    assert np.count_nonzero(outs["dtype"] != outs["fp32"]) > 0
    wl32 = W.WORKLOADS["vision_2d"]
    inp32 = W.make_inputs(wl32, T=300)
    a = _fused_dev(M, inp32, wl32, "dtype")[0]
    b = _fused_dev(M, inp32, wl32, "fp32")[0]
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("precision", MODES)
def test_decode_bit_exact(M, precision):
    import torch
    dw = W.DECODE_WORKLOADS["omni_decode"]
    inp = W.make_decode_inputs(dw, batch=24, new_tokens=2, capacity=40, seed=320)
    note(f"decode batch=24 n=2 precision={precision}")
    qd, kd = to_dev(inp["q"], dw.dtype), to_dev(inp["k"], dw.dtype)
    cl, rdl = to_dev(inp["cache_len"], "i32"), to_dev(inp["rope_delta"], "i32")
    kc = to_dev(inp["k_cache"], dw.dtype)
    wq, wk = to_dev(inp["wq"], dw.dtype), to_dev(inp["wk"], dw.dtype)
    qo = M.mrope_decode_qk(qd, kd, cl, rdl, 2, dw.rotary_dim, dw.theta, kc, wq=wq, wk=wk,
                           eps=dw.eps, precision=precision)
    torch.cuda.synchronize()
    oq, oc = O.mrope_decode_qk(inp["q"], inp["k"], inp["cache_len"], 2, inp["rope_delta"],
                               inp["k_cache"], rotary_dim=dw.rotary_dim, theta=dw.theta,
                               wq=inp["wq"], wk=inp["wk"], eps=dw.eps, dtype=dw.dtype,
                               precision=precision)
    _assert_bits(from_dev(qo), oq, f"decode q {precision}")
    _assert_bits(from_dev(kc), oc, f"decode cache {precision}")
