"""GPU parity at full size: every output element of every workload, in the
launch configuration the benchmark times, against the oracle.

The M01 drill page's acceptance list asks for the RMSNorm, the cos/sin
(image grids included) and the rotated q/k to equal the reference; here all
T * (hq + hk) * D values of configs 2-5 are compared, plus the vision
tower's per-head planes (fp32 and bf16) and the headline prefill in the two
tensor-operation precisions.  The oracle runs over 1024-token chunks in
worker processes (tests/_oracle_pool.py), each worker comparing its chunk.

Bars: bf16 within 1 bf16 ulp of the oracle, binary32 within 1e-5 absolute;
the tensor-operation precisions bit-exact; pass-through dims and the copied
v bit-exact.
"""
import numpy as np
import pytest

import workloads as W
from tests import _oracle_pool as OP
from tests._helpers import from_dev, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import vlm_multimodal_rotary_amd as lib
    lib.load()
    return lib


@pytest.fixture(scope="module")
def pool():
    ex = OP.make_pool()
    yield ex
    ex.shutdown()


def _report(what, res, dtype):
    n, off, worst = res
    unit = "ulp" if dtype == "bf16" else "abs"
    print(f"[parity] {what}: {n} values compared, {off} differ, max {worst:g} {unit}", flush=True)
    return n, off, worst


def _fused_full(M, pool, name, precision):
    import torch
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl)
    note(f"fused full size {name} T={wl.T} precision={precision}")
    wq = to_dev(inp["wq"], wl.dtype) if wl.norm else None
    wk = to_dev(inp["wk"], wl.dtype) if wl.norm else None
    qo, ko = M.rmsnorm_mrope_qk(to_dev(inp["q"], wl.dtype), to_dev(inp["k"], wl.dtype),
                                to_dev(inp["pos"], "i32"), wl.rotary_dim, wl.theta, wl.section,
                                wl.layout, wq=wq, wk=wk, eps=wl.eps, precision=precision)
    torch.cuda.synchronize()
    kernel = M.last_kernel()
    gq, gk = from_dev(qo), from_dev(ko)
    kw = dict(rotary_dim=wl.rotary_dim, theta=wl.theta, section=wl.section, layout=wl.layout,
              eps=wl.eps, dtype=wl.dtype)
    jobs = []
    for a in range(0, wl.T, OP.CHUNK):
        sl = slice(a, min(wl.T, a + OP.CHUNK))
        jobs.append((kw, inp["q"][sl], inp["k"][sl], inp["pos"][:, sl],
                     inp["wq"] if wl.norm else None, inp["wk"] if wl.norm else None, precision,
                     gq[sl], gk[sl]))
    res = list(pool.map(OP.fused_chunk, jobs))
    rq = _report(f"{name} q full ({kernel}, {precision})", OP.merge([r[0] for r in res]),
                 wl.dtype)
    rk = _report(f"{name} k full ({kernel}, {precision})", OP.merge([r[1] for r in res]),
                 wl.dtype)
    assert rq[0] == wl.T * wl.hq * wl.D and rk[0] == wl.T * wl.hk * wl.D
    if wl.rotary_dim < wl.D and not wl.norm:
        assert np.array_equal(gq[..., wl.rotary_dim:], inp["q"][..., wl.rotary_dim:])
    return wl, rq, rk


@pytest.mark.parametrize("name", ["omni_text_prefill", "qwen35_partial_mixed", "chunked_video",
                                  "vision_2d"])
def test_fused_full_size_every_element(M, pool, name):
    wl, rq, rk = _fused_full(M, pool, name, "exact")
    bar = 1 if wl.dtype == "bf16" else 1e-5
    assert rq[2] <= bar and rk[2] <= bar


@pytest.mark.parametrize("precision", ["dtype", "fp32"])
def test_headline_tensor_op_precisions_full_size_bit_exact(M, pool, precision):
    wl, rq, rk = _fused_full(M, pool, "omni_text_prefill", precision)
    assert rq[1] == 0 and rk[1] == 0


@pytest.mark.parametrize("name", list(W.VISION_QKV_WORKLOADS))
def test_vision_qkv_planes_full_size_every_element(M, pool, name):
    import torch
    wl = W.VISION_QKV_WORKLOADS[name]
    inp = W.make_vision_qkv_inputs(wl)
    note(f"vision_qkv full size {name} n={wl.T}")
    flat = inp["qkv"]
    qkv = to_dev(flat.reshape(wl.T, -1), wl.dtype).reshape(wl.T, 3, wl.heads, wl.D)
    q, k, v = M.vision_qkv(qkv, to_dev(inp["pos"], "i32"), wl.rotary_dim, wl.theta)
    torch.cuda.synchronize()
    kernel = M.last_kernel()
    gq, gk, gv = from_dev(q), from_dev(k), from_dev(v)
    kw = dict(rotary_dim=wl.rotary_dim, theta=wl.theta, dtype=wl.dtype)
    jobs = []
    for a in range(0, wl.T, OP.CHUNK):
        sl = slice(a, min(wl.T, a + OP.CHUNK))
        jobs.append((kw, flat[sl], inp["pos"][:, sl], np.ascontiguousarray(gq[:, sl]),
                     np.ascontiguousarray(gk[:, sl]), np.ascontiguousarray(gv[:, sl])))
    res = list(pool.map(OP.vision_chunk, jobs))
    rq = _report(f"{name} q planes full ({kernel})", OP.merge([r[0] for r in res]), wl.dtype)
    rk = _report(f"{name} k planes full ({kernel})", OP.merge([r[1] for r in res]), wl.dtype)
    rv = OP.merge([r[2] for r in res])
    print(f"[parity] {name} v planes full: {rv[0]} values, {rv[1]} differ", flush=True)
    bar = 1 if wl.dtype == "bf16" else 1e-5
    assert rq[0] == rk[0] == rv[0] == wl.T * wl.heads * wl.D
    assert rq[2] <= bar and rk[2] <= bar and rv[1] == 0
