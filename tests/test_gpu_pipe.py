"""The pipelined q/k kernel (one token per wavefront, row-steps streamed with
the next steps' loads in flight): the launch-size boundary of the kernel
choice, in place, a packed qkv whose third tensor is copied, and capture in a
HIP graph.  Bars: bf16 within 1 bf16 ulp of the oracle (the GPU matches it
bit for bit), binary32 within 1e-5; same-kernel comparisons bit-identical."""
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


def _fused(M, inp, wl, **kw):
    import torch
    wq = to_dev(inp["wq"], wl.dtype) if wl.norm else None
    wk = to_dev(inp["wk"], wl.dtype) if wl.norm else None
    qo, ko = M.rmsnorm_mrope_qk(to_dev(inp["q"], wl.dtype), to_dev(inp["k"], wl.dtype),
                                to_dev(inp["pos"], "i32"), wl.rotary_dim, wl.theta, wl.section,
                                wl.layout, wq=wq, wk=wk, eps=wl.eps, **kw)
    torch.cuda.synchronize()
    return from_dev(qo), from_dev(ko), M.last_kernel()


@pytest.mark.parametrize("name", ["omni_text_prefill", "qwen35_partial_mixed", "chunked_video"])
@pytest.mark.parametrize("T", [2047, 2048, 2049])
def test_kernel_choice_boundary(M, name, T):
    """2048 tokens and more take the pipelined kernel, fewer the general one;
    both match the oracle on every element."""
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, T=T, pos_offset=300)
    note(f"pipe boundary {name} T={T}")
    gq, gk, kernel = _fused(M, inp, wl)
    assert kernel == ("qk_pipe_kernel" if T >= 2048 else "qk_kernel"), kernel
    oq, ok = O.rmsnorm_mrope_qk(inp["q"], inp["k"], inp["pos"], rotary_dim=wl.rotary_dim,
                                theta=wl.theta, section=wl.section, layout=wl.layout,
                                wq=inp["wq"] if wl.norm else None,
                                wk=inp["wk"] if wl.norm else None, eps=wl.eps, dtype=wl.dtype)
    assert_close(gq, oq, wl.dtype, f"{name} T={T} q ({kernel})")
    assert_close(gk, ok, wl.dtype, f"{name} T={T} k ({kernel})")


@pytest.mark.parametrize("name", ["omni_text_prefill", "qwen35_partial_mixed"])
def test_in_place_equals_out_of_place(M, name):
    import torch
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, T=3000)
    note(f"pipe in place {name}")
    q, k = to_dev(inp["q"], wl.dtype), to_dev(inp["k"], wl.dtype)
    pos = to_dev(inp["pos"], "i32")
    wq, wk = to_dev(inp["wq"], wl.dtype), to_dev(inp["wk"], wl.dtype)
    qo, ko = M.rmsnorm_mrope_qk(q, k, pos, wl.rotary_dim, wl.theta, wl.section, wl.layout,
                                wq=wq, wk=wk, eps=wl.eps)
    assert M.last_kernel() == "qk_pipe_kernel"
    qi, ki = q.clone(), k.clone()
    M.rmsnorm_mrope_qk(qi, ki, pos, wl.rotary_dim, wl.theta, wl.section, wl.layout, wq=wq,
                       wk=wk, eps=wl.eps, q_out=qi, k_out=ki)
    torch.cuda.synchronize()
    assert torch.equal(qi.view(torch.int16), qo.view(torch.int16))
    assert torch.equal(ki.view(torch.int16), ko.view(torch.int16))


@pytest.mark.parametrize("head_major", [False, True])
def test_packed_qkv_with_copied_v(M, head_major):
    """A packed qkv [n, 3, heads, 128] bf16 through mrope_vision_qkv: q and k
    rotated (vision 2-D layout), v copied; token-major rows of 256 bytes take
    the pipelined kernel with three tensors."""
    rng = np.random.default_rng(41)
    n, H, D = 2304, 6, 128
    qkv = W._store(rng.standard_normal((n, 3, H, D)).astype(np.float32), "bf16")
    pos = W.vision_patch_positions(1, 48, 48)[:, :n].astype(np.int32)
    note(f"pipe packed qkv head_major={head_major}")
    dev = to_dev(qkv.reshape(n, -1), "bf16").reshape(n, 3, H, D)
    q, k, v = M.vision_qkv(dev, to_dev(pos, "i32"), D, 1e4, head_major=head_major)
    import torch
    torch.cuda.synchronize()
    kernel = M.last_kernel()
    if not head_major:
        assert kernel == "qk_pipe_kernel", kernel
    oq, ok, ov = O.vision_qkv(qkv, pos, rotary_dim=D, theta=1e4, dtype="bf16")
    gq, gk, gv = from_dev(q), from_dev(k), from_dev(v)
    if not head_major:
        gq, gk, gv = (x.transpose(1, 0, 2) for x in (gq, gk, gv))
    assert_close(np.ascontiguousarray(gq), oq, "bf16", f"packed q ({kernel})")
    assert_close(np.ascontiguousarray(gk), ok, "bf16", f"packed k ({kernel})")
    assert np.array_equal(np.ascontiguousarray(gv), ov)


def test_replays_in_a_hip_graph(M):
    """The pipelined kernel captured in a graph (headline shape, 4096 tokens,
    and qwen35's shape): several replays with the outputs cleared and eager
    work between them, each equal to the eager result."""
    import torch
    cases = []
    for name in ("omni_text_prefill", "qwen35_partial_mixed"):
        wl = W.WORKLOADS[name]
        inp = W.make_inputs(wl, T=4096, pos_offset=100)
        d = dict(q=to_dev(inp["q"], wl.dtype), k=to_dev(inp["k"], wl.dtype),
                 pos=to_dev(inp["pos"], "i32"), wq=to_dev(inp["wq"], wl.dtype),
                 wk=to_dev(inp["wk"], wl.dtype))
        eq, ek = M.rmsnorm_mrope_qk(d["q"], d["k"], d["pos"], wl.rotary_dim, wl.theta,
                                    wl.section, wl.layout, wq=d["wq"], wk=d["wk"], eps=wl.eps)
        assert M.last_kernel() == "qk_pipe_kernel"
        d.update(eq=eq, ek=ek, gq=torch.empty_like(eq), gk=torch.empty_like(ek), wl=wl)
        cases.append(d)
    torch.cuda.synchronize()

    def launch_all():
        for d in cases:
            wl = d["wl"]
            M.rmsnorm_mrope_qk(d["q"], d["k"], d["pos"], wl.rotary_dim, wl.theta, wl.section,
                               wl.layout, wq=d["wq"], wk=d["wk"], eps=wl.eps, q_out=d["gq"],
                               k_out=d["gk"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch_all()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch_all()
    for rep in range(4):
        for d in cases:
            d["gq"].zero_()
            d["gk"].zero_()
        torch.cuda.synchronize()
        note(f"pipe graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for d in cases:
            assert torch.equal(d["gq"].view(torch.int16), d["eq"].view(torch.int16)), rep
            assert torch.equal(d["gk"].view(torch.int16), d["ek"].view(torch.int16)), rep


# (head dim, rotary dim, q heads, k heads): the contiguous-halves layout (one
# chunk of each half of the row per lane, rotary partners exchanged between
# lanes) at 2, 4 and 8 rotary chunks per half, and with 8 lanes per row.
HALVES_SHAPES = [(256, 64, 24, 4), (256, 32, 8, 2), (256, 128, 8, 2), (128, 64, 16, 2)]


@pytest.mark.parametrize("D,rd,hq,hk", HALVES_SHAPES)
@pytest.mark.parametrize("precision", ["exact", "dtype", "fp32"])
def test_contiguous_halves_layout(M, D, rd, hq, hk, precision):
    """Partial rotary over at most half the row in the pipelined kernel, in
    every precision: bit-exact against the oracle."""
    import torch
    rng = np.random.default_rng(D * 1000 + rd)
    T = 2304
    q, k = W.random_qk(rng, T, hq, hk, D, "bf16")
    wq, wk = W.random_weight(rng, D, "bf16"), W.random_weight(rng, D, "bf16")
    half = rd // 2
    sec = (half - 2 * (half // 3), half // 3, half // 3)
    pos = np.stack([np.arange(T) + 17, (np.arange(T) * 7) % 501, (np.arange(T) * 3) % 97])
    pos = pos.astype(np.int32)
    note(f"contiguous halves D={D} rd={rd} {precision}")
    qo, ko = M.rmsnorm_mrope_qk(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(pos, "i32"), rd,
                                1e6, sec, "interleaved", wq=to_dev(wq, "bf16"),
                                wk=to_dev(wk, "bf16"), eps=1e-6, precision=precision)
    torch.cuda.synchronize()
    assert M.last_kernel() == "qk_pipe_kernel"
    oq, ok = O.rmsnorm_mrope_qk(q, k, pos, rotary_dim=rd, theta=1e6, section=sec,
                                layout="interleaved", wq=wq, wk=wk, eps=1e-6, dtype="bf16",
                                precision=precision)
    gq, gk = from_dev(qo), from_dev(ko)
    assert np.array_equal(gq.view(np.uint16), np.asarray(oq).view(np.uint16)), "q"
    assert np.array_equal(gk.view(np.uint16), np.asarray(ok).view(np.uint16)), "k"
