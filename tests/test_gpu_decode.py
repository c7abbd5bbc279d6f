"""GPU parity of the decode step (mrope_decode_qk) against the CPU oracle."""
import numpy as np
import pytest

from oracle import mrope_oracle as O
import workloads as W
from tests._helpers import assert_bf16_close, assert_close, from_dev, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import vlm_multimodal_rotary_amd as lib
    lib.load()
    return lib


def _run(M, inp, wl, use_delta=True, in_place=False):
    import torch
    dt = wl.dtype
    q, k = to_dev(inp["q"], dt), to_dev(inp["k"], dt)
    cache = to_dev(inp["k_cache"], dt)
    cl = to_dev(inp["cache_len"], "i32")
    rd = to_dev(inp["rope_delta"], "i32") if use_delta else None
    wq = to_dev(inp["wq"], dt) if wl.norm else None
    wk = to_dev(inp["wk"], dt) if wl.norm else None
    qo = M.mrope_decode_qk(q, k, cl, rd, inp["new_tokens"], wl.rotary_dim, wl.theta, cache,
                           wq=wq, wk=wk, eps=wl.eps, q_out=q if in_place else None)
    torch.cuda.synchronize()
    return from_dev(qo), from_dev(cache)


def _oracle(inp, wl, use_delta=True):
    return O.mrope_decode_qk(inp["q"], inp["k"], inp["cache_len"], inp["new_tokens"],
                             inp["rope_delta"] if use_delta else None, inp["k_cache"],
                             rotary_dim=wl.rotary_dim, theta=wl.theta,
                             wq=inp["wq"] if wl.norm else None,
                             wk=inp["wk"] if wl.norm else None, eps=wl.eps, dtype=wl.dtype)


@pytest.mark.parametrize("batch,new_tokens,capacity,use_delta", [
    (7, 1, 64, True), (5, 3, 40, True), (9, 2, 300, False), (1, 1, 1, True)])
def test_decode_matches_oracle(M, batch, new_tokens, capacity, use_delta):
    wl = W.DECODE_WORKLOADS["omni_decode"]
    inp = W.make_decode_inputs(wl, batch=batch, new_tokens=new_tokens, capacity=capacity)
    note(f"decode B={batch} n={new_tokens} cap={capacity} delta={use_delta}")
    gq, gc = _run(M, inp, wl, use_delta)
    oq, oc = _oracle(inp, wl, use_delta)
    assert_bf16_close(gq, oq, 1, "decode q")
    assert_bf16_close(gc, oc, 1, "decode k cache")
    # rows other than the appended ones are untouched, bit for bit
    touched = np.zeros((batch, capacity), bool)
    for b in range(batch):
        for i in range(new_tokens):
            if inp["cache_len"][b] + i < capacity:
                touched[b, inp["cache_len"][b] + i] = True
    assert np.array_equal(gc[~touched], inp["k_cache"][~touched])


def test_decode_rows_past_capacity_are_not_written(M):
    wl = W.DECODE_WORKLOADS["omni_decode"]
    inp = W.make_decode_inputs(wl, batch=4, new_tokens=4, capacity=10)
    inp["cache_len"] = np.array([0, 7, 9, 12], dtype=np.int32)   # 7..10, 9..12, 12..15 overflow
    note("decode capacity overflow")
    gq, gc = _run(M, inp, wl)
    oq, oc = _oracle(inp, wl)
    assert_bf16_close(gq, oq, 1, "decode q")
    assert_bf16_close(gc, oc, 1, "decode cache")
    assert np.array_equal(gc[3], inp["k_cache"][3])


def test_decode_in_place_q_and_full_size(M):
    wl = W.DECODE_WORKLOADS["omni_decode"]
    inp = W.make_decode_inputs(wl, batch=64, capacity=256)
    note("decode in place")
    gq, gc = _run(M, inp, wl, in_place=True)
    oq, oc = _oracle(inp, wl)
    assert_bf16_close(gq, oq, 1, "decode q in place")
    assert_bf16_close(gc, oc, 1, "decode cache")
    # the benchmark's configuration, every sequence and every cache row
    inp = W.make_decode_inputs(wl)
    note(f"decode full B={inp['batch']} cap={inp['capacity']}")
    gq, gc = _run(M, inp, wl)
    oq, oc = _oracle(inp, wl)
    assert_bf16_close(gq, oq, 1, "decode q full")
    assert_bf16_close(gc, oc, 1, "decode cache full")


def test_decode_and_prefill_replay_in_a_hip_graph(M):
    """Captured launches replay correctly: several replays with eager work and
    synchronisations between them, each checked against the eager result."""
    import torch
    wl = W.DECODE_WORKLOADS["omni_decode"]
    inp = W.make_decode_inputs(wl, batch=32, capacity=128)
    dt = wl.dtype
    q, k = to_dev(inp["q"], dt), to_dev(inp["k"], dt)
    cl, rd = to_dev(inp["cache_len"], "i32"), to_dev(inp["rope_delta"], "i32")
    wq, wk = to_dev(inp["wq"], dt), to_dev(inp["wk"], dt)
    cache_eager = to_dev(inp["k_cache"], dt)
    q_eager = M.mrope_decode_qk(q, k, cl, rd, 1, wl.rotary_dim, wl.theta, cache_eager,
                                wq=wq, wk=wk, eps=wl.eps)
    pw = W.WORKLOADS["omni_text_prefill"]
    pinp = W.make_inputs(pw, T=100)
    pq, pk, pos = to_dev(pinp["q"], "bf16"), to_dev(pinp["k"], "bf16"), to_dev(pinp["pos"], "i32")
    pwq, pwk = to_dev(pinp["wq"], "bf16"), to_dev(pinp["wk"], "bf16")
    pq_eager, pk_eager = M.rmsnorm_mrope_qk(pq, pk, pos, 128, pw.theta, pw.section, pw.layout,
                                            wq=pwq, wk=pwk, eps=pw.eps)
    torch.cuda.synchronize()

    cache_g = to_dev(inp["k_cache"], dt)
    q_g = torch.empty_like(q)
    pq_g, pk_g = torch.empty_like(pq), torch.empty_like(pk)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.mrope_decode_qk(q, k, cl, rd, 1, wl.rotary_dim, wl.theta, cache_g, wq=wq, wk=wk,
                          eps=wl.eps, q_out=q_g)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.mrope_decode_qk(q, k, cl, rd, 1, wl.rotary_dim, wl.theta, cache_g, wq=wq, wk=wk,
                          eps=wl.eps, q_out=q_g)
        M.rmsnorm_mrope_qk(pq, pk, pos, 128, pw.theta, pw.section, pw.layout, wq=pwq, wk=pwk,
                           eps=pw.eps, q_out=pq_g, k_out=pk_g)
    for rep in range(4):
        q_g.zero_()
        pq_g.zero_()
        pk_g.zero_()
        cache_g.copy_(to_dev(inp["k_cache"], dt))
        torch.cuda.synchronize()
        note(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(q_g.view(torch.int16), q_eager.view(torch.int16)), rep
        assert torch.equal(cache_g.view(torch.int16), cache_eager.view(torch.int16)), rep
        assert torch.equal(pq_g.view(torch.int16), pq_eager.view(torch.int16)), rep
        assert torch.equal(pk_g.view(torch.int16), pk_eager.view(torch.int16)), rep


def test_position_builder_and_vision_fusion_replay_in_a_hip_graph(M):
    """The position builder (both forms of passes 2 and 3) and the vision
    fusion (staged bf16 planes, flat fp32 planes and fp32 token-major rows)
    captured in one graph: every replay, with the outputs cleared and eager
    work between replays, equals the eager result."""
    import torch
    rng = np.random.default_rng(31)
    batches = [W.random_mm_batch(rng, 2, 600), W.random_mm_batch(rng, 4, 4000)]
    assert len(batches[1][2]) > 256            # the second one takes the two-kernel form
    dev_batches = []
    for types, mask, images, videos in batches:
        g = lambda x: None if not x else to_dev(np.asarray(x, dtype=np.int32).reshape(-1, 3), "i32")
        dev_batches.append((to_dev(types.astype(np.int32), "i32"), g(images), g(videos),
                            to_dev(mask.astype(np.int32), "i32")))
    eager_pos = [M.rope_index(t, i, v, m)[:2] for t, i, v, m in dev_batches]
    vis = []
    for name, head_major in (("vision_qkv_planes_bf16", True), ("vision_qkv_planes", True),
                             ("vision_qkv_planes", False)):
        wl = W.VISION_QKV_WORKLOADS[name]
        inp = W.make_vision_qkv_inputs(wl, n=4096)
        qkv = to_dev(inp["qkv"].reshape(4096, -1), wl.dtype).reshape(4096, 3, wl.heads, wl.D)
        pos = to_dev(inp["pos"], "i32")
        outs = M.vision_qkv(qkv, pos, wl.rotary_dim, wl.theta, head_major=head_major)
        vis.append((qkv, pos, wl, head_major, [o.clone() for o in outs]))
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):            # warm the allocator outside the capture
        for t, i, v, m in dev_batches:
            M.rope_index(t, i, v, m, check=False)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        g_pos = [M.rope_index(t, i, v, m, check=False)[:2] for t, i, v, m in dev_batches]
        g_vis = [M.vision_qkv(qkv, pos, wl.rotary_dim, wl.theta, head_major=hm)
                 for qkv, pos, wl, hm, _ in vis]
    for rep in range(3):
        for pair in g_pos:
            for x in pair:
                x.zero_()
        for outs in g_vis:
            for x in outs:
                x.zero_()
        torch.cuda.synchronize()
        note(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for (gp, gd), (ep, ed) in zip(g_pos, eager_pos):
            assert torch.equal(gp, ep) and torch.equal(gd, ed), rep
        for outs, (_, _, _, _, want) in zip(g_vis, vis):
            for a, b in zip(outs, want):
                assert torch.equal(a.view(torch.int8), b.view(torch.int8)), rep
