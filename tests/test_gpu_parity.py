"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars (written here): bf16 outputs within 1 bf16 ulp of the oracle, fp32
outputs within 1e-5 absolute, pass-through dims and integer tables bit-exact,
the fused call bit-identical to rms_norm -> mrope_cos_sin -> apply_rotary_qk.
"""
import numpy as np
import pytest

from oracle import mrope_oracle as O
import workloads as W
from tests._helpers import (assert_bf16_close, assert_close, assert_f32_close, from_dev, note,
                            to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import vlm_multimodal_rotary_amd as lib
    lib.load()
    return lib


def _run_fused(M, inp, wl, q=None, k=None, pos=None):
    qd = to_dev(inp["q"] if q is None else q, wl.dtype)
    kd = to_dev(inp["k"] if k is None else k, wl.dtype)
    pd = to_dev(inp["pos"] if pos is None else pos, "i32")
    wq = to_dev(inp["wq"], wl.dtype) if wl.norm else None
    wk = to_dev(inp["wk"], wl.dtype) if wl.norm else None
    qo, ko = M.rmsnorm_mrope_qk(qd, kd, pd, wl.rotary_dim, wl.theta, wl.section, wl.layout,
                                wq=wq, wk=wk, eps=wl.eps)
    import torch
    torch.cuda.synchronize()
    return from_dev(qo), from_dev(ko)


def _oracle_fused(inp, wl, rows=None):
    q, k, pos = inp["q"], inp["k"], inp["pos"]
    if rows is not None:
        q, k, pos = q[rows], k[rows], pos[:, rows]
    return O.rmsnorm_mrope_qk(q, k, pos, rotary_dim=wl.rotary_dim, theta=wl.theta,
                              section=wl.section, layout=wl.layout,
                              wq=inp["wq"] if wl.norm else None,
                              wk=inp["wk"] if wl.norm else None, eps=wl.eps, dtype=wl.dtype)


# Small windows of every workload: several tiles, a ragged tail, and the
# segment boundaries of the mixed and video position tables.
SMALL = [
    ("tiny_mrope", None, 0),
    ("omni_text_prefill", 777, 0),
    ("qwen35_partial_mixed", 1400, 0),
    ("chunked_video", 700, 900),
    ("chunked_video", 600, 10664),
    ("vision_2d", 4500, 0),
]


@pytest.mark.parametrize("name,T,off", SMALL, ids=[f"{n}-T{t}-off{o}" for n, t, o in SMALL])
def test_fused_small_windows(M, name, T, off):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, T=T, pos_offset=off)
    note(f"fused {name} T={inp['T']} off={off}")
    gq, gk = _run_fused(M, inp, wl)
    oq, ok = _oracle_fused(inp, wl)
    assert_close(gq, oq, wl.dtype, f"{name} q")
    assert_close(gk, ok, wl.dtype, f"{name} k")
    if wl.rotary_dim < wl.D and not wl.norm:
        assert np.array_equal(gq[..., wl.rotary_dim:], inp["q"][..., wl.rotary_dim:])


def test_fused_equals_unfused_composition_bitwise(M):
    import torch
    for name in ("omni_text_prefill", "qwen35_partial_mixed", "vision_2d", "chunked_video"):
        wl = W.WORKLOADS[name]
        inp = W.make_inputs(wl, T=600, pos_offset=400 if name != "vision_2d" else 0)
        note(f"fused vs composition {name}")
        qd, kd = to_dev(inp["q"], wl.dtype), to_dev(inp["k"], wl.dtype)
        pd = to_dev(inp["pos"], "i32")
        wq = to_dev(inp["wq"], wl.dtype) if wl.norm else None
        wk = to_dev(inp["wk"], wl.dtype) if wl.norm else None
        fq, fk = M.rmsnorm_mrope_qk(qd, kd, pd, wl.rotary_dim, wl.theta, wl.section, wl.layout,
                                    wq=wq, wk=wk, eps=wl.eps)
        nq = M.rms_norm(qd, wq, wl.eps) if wl.norm else qd
        nk = M.rms_norm(kd, wk, wl.eps) if wl.norm else kd
        half = wl.rotary_dim // 2
        if wl.layout == "vision_2d":
            inv = M.mrope_inv_freq(half, wl.theta)
        else:
            inv = M.mrope_inv_freq(wl.rotary_dim, wl.theta)
        c, s = M.mrope_cos_sin(pd, inv, wl.section, wl.layout, wl.rotary_dim)
        cq, ck = M.apply_rotary_qk(nq, nk, c, s, wl.rotary_dim)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(fq), from_dev(cq)), name
        assert np.array_equal(from_dev(fk), from_dev(ck)), name


def test_cos_sin_matches_oracle(M):
    for name in W.WORKLOADS:
        wl = W.WORKLOADS[name]
        inp = W.make_inputs(wl, T=min(wl.T, 3000))
        half = wl.rotary_dim // 2
        inv = O.inv_freq(half if wl.layout == "vision_2d" else wl.rotary_dim, wl.theta)
        note(f"cos_sin {name}")
        c, s = M.mrope_cos_sin(to_dev(inp["pos"], "i32"), inv, wl.section, wl.layout,
                               wl.rotary_dim)
        oc, os_ = O.mrope_cos_sin(inp["pos"], inv, wl.section, wl.layout, wl.rotary_dim)
        gc, gs = from_dev(c), from_dev(s)
        # one binary32 ulp at most (both round a double cos/sin of the same angle)
        for g, o in ((gc, oc), (gs, os_)):
            d = np.abs(g.view(np.int32).astype(np.int64) - o.view(np.int32).astype(np.int64))
            d = np.where(np.sign(g) == np.sign(o), d, 0)
            assert d.max() <= 1 and np.mean(d == 0) > 0.9999, (name, d.max(), np.mean(d == 0))
            assert_f32_close(g, o, 1e-6, f"{name} cos/sin")


def test_acos_probe_on_gpu(M, golden):
    g = golden("acos_probe.json")
    letters = {"T": 1, "H": 2, "W": 3}
    import torch
    pos = torch.tensor([[1], [2], [3]], dtype=torch.int32, device="cuda")
    for case in g["cases"]:
        note(f"acos probe {case}")
        half = case["half"]
        c, _ = M.mrope_cos_sin(pos, np.ones(half, np.float32), case["section"], case["layout"],
                               2 * half)
        got = [int(round(float(np.arccos(v)))) for v in from_dev(c)[0]]
        want = ([int(ch) for ch in case["digits"]] if "digits" in case
                else [letters[ch] for ch in case["letters"]])
        assert got == want + want, (case, got)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 256), ("bf16", 72), ("f32", 72),
                                     ("f32", 256), ("bf16", 16), ("f32", 2), ("bf16", 1024)])
def test_rms_norm_matches_oracle(M, dtype, D):
    rng = np.random.default_rng(D + (1 if dtype == "bf16" else 0))
    T, H = 203, 3
    x, _ = W.random_qk(rng, T, H, 1, D, dtype, scale=float(rng.uniform(0.01, 30)))
    w = W.random_weight(rng, D, dtype)
    note(f"rms_norm {dtype} D={D}")
    out = M.rms_norm(to_dev(x, dtype), to_dev(w, dtype), 1e-6)
    got = from_dev(out)
    want = O.rms_norm(x, w, 1e-6, dtype)
    assert_close(got, want, dtype, f"rms_norm {dtype} D={D}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_apply_rotary_with_general_tables(M, dtype):
    """cos/sin tables whose halves differ: the elementwise definition
    x*cos + rotate_half(x)*sin over [T, rotary_dim], partial rotary."""
    rng = np.random.default_rng(31)
    T, hq, hk, D, rd = 97, 5, 2, 96, 48
    q, k = W.random_qk(rng, T, hq, hk, D, dtype)
    cos = rng.uniform(-1, 1, (T, rd)).astype(np.float32)
    sin = rng.uniform(-1, 1, (T, rd)).astype(np.float32)
    note(f"apply_rotary general {dtype}")
    qo, ko = M.apply_rotary_qk(to_dev(q, dtype), to_dev(k, dtype), to_dev(cos, "f32"),
                               to_dev(sin, "f32"), rd)
    oq, ok = O.apply_rotary_qk(q, k, cos, sin, rd, dtype)
    assert_close(from_dev(qo), oq, dtype, "apply_rotary q")
    assert_close(from_dev(ko), ok, dtype, "apply_rotary k")
    assert np.array_equal(from_dev(qo)[..., rd:], q[..., rd:])


def test_text_only_layouts_agree_bitwise_on_gpu(M):
    import torch
    rng = np.random.default_rng(32)
    T, hq, hk, D = 300, 4, 2, 128
    q, k = W.random_qk(rng, T, hq, hk, D, "bf16")
    p = np.arange(5000, 5000 + T, dtype=np.int32)
    qd, kd = to_dev(q, "bf16"), to_dev(k, "bf16")
    note("text-only layouts")
    outs = []
    for layout, sec, pos in [("interleaved", (24, 20, 20), np.stack([p, p, p])),
                             ("chunked", (16, 24, 24), np.stack([p, p, p])),
                             ("chunked", (64,), p.reshape(1, -1))]:
        qo, ko = M.rmsnorm_mrope_qk(qd, kd, to_dev(pos, "i32"), D, 1e6, sec, layout)
        outs.append((from_dev(qo), from_dev(ko)))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0]) and np.array_equal(o[1], outs[0][1])


def test_edge_cases(M):
    import torch
    rng = np.random.default_rng(33)
    wl = W.WORKLOADS["omni_text_prefill"]
    # T = 0 and T = 1
    for T in (0, 1):
        inp = W.make_inputs(wl, T=T)
        note(f"edge T={T}")
        gq, gk = _run_fused(M, inp, wl)
        if T:
            oq, ok = _oracle_fused(inp, wl)
            assert_bf16_close(gq, oq, 1, "T=1 q")
            assert_bf16_close(gk, ok, 1, "T=1 k")
    # no k heads
    inp = W.make_inputs(wl, T=50)
    note("edge hk=0")
    qd = to_dev(inp["q"], "bf16")
    kd = torch.empty((50, 0, 128), dtype=torch.bfloat16, device="cuda")
    qo, ko = M.rmsnorm_mrope_qk(qd, kd, to_dev(inp["pos"], "i32"), 128, wl.theta, wl.section,
                                wl.layout, wq=to_dev(inp["wq"], "bf16"),
                                wk=to_dev(inp["wk"], "bf16"), eps=wl.eps)
    oq, _ = _oracle_fused(inp, wl)
    assert_bf16_close(from_dev(qo), oq, 1, "hk=0 q")
    # in place
    note("edge in place")
    qd, kd = to_dev(inp["q"], "bf16"), to_dev(inp["k"], "bf16")
    M.rmsnorm_mrope_qk(qd, kd, to_dev(inp["pos"], "i32"), 128, wl.theta, wl.section, wl.layout,
                       wq=to_dev(inp["wq"], "bf16"), wk=to_dev(inp["wk"], "bf16"), eps=wl.eps,
                       q_out=qd, k_out=kd)
    oq, ok = _oracle_fused(inp, wl)
    assert_bf16_close(from_dev(qd), oq, 1, "in-place q")
    assert_bf16_close(from_dev(kd), ok, 1, "in-place k")


def test_packed_qkv_views_and_strided_positions(M):
    """q and k as views into a packed [T, 3, H, D] buffer (token stride
    3*H*D), positions as a row-slice of a wider table, 1-D positions
    broadcast to three axes with axis stride 0."""
    import torch
    rng = np.random.default_rng(34)
    T, H, D, rd = 333, 6, 64, 64
    qkv = (rng.standard_normal((T, 3, H, D))).astype(np.float32)
    qkv_bits = W.to_bf16_bits(qkv)
    dev = to_dev(qkv_bits, "bf16")
    q, k = dev[:, 0], dev[:, 1]
    assert q.stride(0) == 3 * H * D
    wide = rng.integers(0, 9000, (3, T + 17)).astype(np.int32)
    pos_dev = to_dev(wide, "i32")[:, 5:5 + T]
    note("packed qkv views")
    qo, ko = M.rmsnorm_mrope_qk(q, k, pos_dev, rd, 1e6, (12, 10, 10), "interleaved")
    torch.cuda.synchronize()
    oq, ok = O.rmsnorm_mrope_qk(qkv_bits[:, 0], qkv_bits[:, 1], wide[:, 5:5 + T], rotary_dim=rd,
                                theta=1e6, section=(12, 10, 10), layout="interleaved",
                                dtype="bf16")
    assert_bf16_close(from_dev(qo), oq, 1, "packed q")
    assert_bf16_close(from_dev(ko), ok, 1, "packed k")
    # untouched v plane
    assert np.array_equal(from_dev(dev[:, 2]), qkv_bits[:, 2])
    # 1-D positions broadcast (axis stride 0) == explicit three equal rows
    p1 = np.arange(T, dtype=np.int32) * 7
    from vlm_multimodal_rotary_amd import _lib
    import ctypes
    lib = _lib.load()
    qd = to_dev(qkv_bits[:, 0], "bf16")
    kd = to_dev(qkv_bits[:, 1], "bf16")
    qo1, ko1 = torch.empty_like(qd), torch.empty_like(kd)
    p1d = to_dev(p1, "i32")
    sec = _lib.int_array([12, 10, 10])
    note("broadcast positions stride 0")
    rc = lib.rmsnorm_mrope_qk(qd.data_ptr(), H * D, H, kd.data_ptr(), H * D, H, T, D, rd,
                              p1d.data_ptr(), 0, 3, sec, 3, _lib.LAYOUT_INTERLEAVED, 1e6, None,
                              None, 1e-6, _lib.DTYPE_BF16, _lib.PRECISION_EXACT, qo1.data_ptr(),
                              H * D, ko1.data_ptr(),
                              H * D, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(rc)
    qo3, _ = M.rmsnorm_mrope_qk(qd, kd, to_dev(np.stack([p1, p1, p1]), "i32"), rd, 1e6,
                                (12, 10, 10), "interleaved")
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(qo1), from_dev(qo3))


@pytest.mark.parametrize("dtype,D,rd,norm", [
    ("bf16", 72, 72, True),     # 9 lanes per row: non-power-of-two reduction
    ("f32", 72, 72, True),
    ("f32", 256, 128, True),    # 32 lanes per row
    ("bf16", 512, 512, True),   # largest rotary_dim, 32 lanes per row
    ("bf16", 2, 2, True),       # one lane per row
    ("f32", 16, 8, False),
    ("bf16", 48, 16, True),     # partial rotary with two-chunk pass-through lanes
])
def test_geometries(M, dtype, D, rd, norm):
    rng = np.random.default_rng(D * 3 + rd)
    T, hq, hk = 131, 5, 3
    q, k = W.random_qk(rng, T, hq, hk, D, dtype)
    wq = W.random_weight(rng, D, dtype) if norm else None
    wk = W.random_weight(rng, D, dtype) if norm else None
    half = rd // 2
    layout = "vision_2d" if half % 2 == 0 and D == 72 else "interleaved"
    if layout == "interleaved":
        if half >= 3:
            sh = sw = half // 3
            section = (half - sh - sw, sh, sw)
            while True:
                try:
                    O.axis_table(half, section, "interleaved")
                    break
                except AssertionError:
                    sh -= 1
                    sw -= 1
                    section = (half - sh - sw, sh, sw)
        else:
            section = (half, 0, 0)
        pos = rng.integers(-50, 20000, (3, T)).astype(np.int32)
    else:
        section = None
        pos = rng.integers(0, 64, (2, T)).astype(np.int32)
    note(f"geometry {dtype} D={D} rd={rd} norm={norm} {layout} {section}")
    qo, ko = M.rmsnorm_mrope_qk(to_dev(q, dtype), to_dev(k, dtype), to_dev(pos, "i32"), rd, 1e5,
                                section, layout, wq=to_dev(wq, dtype), wk=to_dev(wk, dtype),
                                eps=1e-6)
    oq, ok = O.rmsnorm_mrope_qk(q, k, pos, rotary_dim=rd, theta=1e5, section=section,
                                layout=layout, wq=wq, wk=wk, eps=1e-6, dtype=dtype)
    assert_close(from_dev(qo), oq, dtype, f"D={D} q")
    assert_close(from_dev(ko), ok, dtype, f"D={D} k")


def test_unaligned_buffer_takes_narrow_chunks(M):
    """A bf16 view starting 2 bytes into an allocation forces 1-element chunks."""
    import torch
    rng = np.random.default_rng(35)
    T, H, D = 70, 3, 32
    q, k = W.random_qk(rng, T, H, H, D, "bf16")
    big = torch.zeros(T * H * D + 1, dtype=torch.bfloat16, device="cuda")
    qv = big[1:].view(T, H, D)
    qv.copy_(to_dev(q, "bf16"))
    kd = to_dev(k, "bf16")
    pos = rng.integers(0, 1000, (3, T)).astype(np.int32)
    note("unaligned q view")
    qo, ko = M.rmsnorm_mrope_qk(qv, kd, to_dev(pos, "i32"), D, 1e4, (6, 5, 5), "interleaved")
    oq, ok = O.rmsnorm_mrope_qk(q, k, pos, rotary_dim=D, theta=1e4, section=(6, 5, 5),
                                layout="interleaved", dtype="bf16")
    assert_bf16_close(from_dev(qo), oq, 1, "unaligned q")
    assert_bf16_close(from_dev(ko), ok, 1, "unaligned k")


def test_extreme_positions(M):
    """Positions up to 2^24 - 1 (the largest exact in float32) and negative."""
    rng = np.random.default_rng(36)
    T, H, D = 64, 2, 64
    q, k = W.random_qk(rng, T, H, H, D, "f32")
    pos = rng.integers(-(2 ** 24) + 1, 2 ** 24, (3, T)).astype(np.int32)
    pos[:, 0] = 2 ** 24 - 1
    note("extreme positions")
    qo, ko = M.rmsnorm_mrope_qk(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(pos, "i32"), D, 1e4,
                                (12, 10, 10), "interleaved")
    oq, ok = O.rmsnorm_mrope_qk(q, k, pos, rotary_dim=D, theta=1e4, section=(12, 10, 10),
                                layout="interleaved", dtype="f32")
    assert_f32_close(from_dev(qo), oq, 1e-5, "extreme q")
    assert_f32_close(from_dev(ko), ok, 1e-5, "extreme k")


# Geometries that take the flat kernel (positions path, no norm, at least
# 2048 tokens, rows that are not a whole number of 256-byte lines pairs).
FLAT = [("f32", 72, 72, (16, 16), "vision_2d", None),
        ("bf16", 72, 72, (16, 16), "vision_2d", None),
        ("f32", 80, 48, (5, 3), "interleaved", (12, 6, 6)),
        ("bf16", 96, 32, (12, 2), "chunked", (8, 4, 4)),
        ("bf16", 160, 160, (9, 1), "interleaved", (40, 20, 20)),
        ("f32", 48, 48, (7, 0), "vision_2d", None)]


@pytest.mark.parametrize("dtype,D,rd,heads,layout,section", FLAT,
                         ids=[f"{d}-D{D}-rd{r}-{l}" for d, D, r, _, l, _ in FLAT])
def test_flat_kernel_geometries(M, dtype, D, rd, heads, layout, section):
    import torch
    T = 2100
    rng = np.random.default_rng(D * 7 + rd)
    q, k = W.random_qk(rng, T, heads[0], heads[1], D, dtype)
    n_axes = 2 if layout == "vision_2d" else 3
    pos = rng.integers(0, 5000, (n_axes, T)).astype(np.int32)
    note(f"flat {dtype} D={D} rd={rd} heads={heads} {layout}")
    qo, ko = M.rmsnorm_mrope_qk(to_dev(q, dtype), to_dev(k, dtype), to_dev(pos, "i32"), rd, 1e4,
                                section, layout)
    torch.cuda.synchronize()
    oq, ok = O.rmsnorm_mrope_qk(q, k, pos, rotary_dim=rd, theta=1e4, section=section,
                                layout=layout, dtype=dtype)
    assert_close(from_dev(qo), oq, dtype, "flat q")
    if heads[1]:
        assert_close(from_dev(ko), ok, dtype, "flat k")
    if rd < D:
        assert np.array_equal(from_dev(qo)[..., rd:], q[..., rd:])


@pytest.mark.parametrize("heads", [(16, 16), (32, 8)], ids=["one-batch", "rows-across-batches"])
def test_in_place_long_launch_matches_out_of_place(M, heads):
    """In place on 2048+ tokens of 72-wide fp32 rows (the flat kernel's
    shapes): bit-identical to the out-of-place call, also where a token's
    rows span more than one of the flat kernel's load batches."""
    import torch
    T = 2100
    rng = np.random.default_rng(91)
    q, k = W.random_qk(rng, T, heads[0], heads[1], 72, "f32")
    pos = rng.integers(0, 5000, (2, T)).astype(np.int32)
    note(f"in place, long launch, heads {heads}")
    qd, kd, pd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(pos, "i32")
    qo, ko = M.rmsnorm_mrope_qk(qd, kd, pd, 72, 1e4, None, "vision_2d")
    qi, ki = qd.clone(), kd.clone()
    M.rmsnorm_mrope_qk(qi, ki, pd, 72, 1e4, None, "vision_2d", q_out=qi, k_out=ki)
    torch.cuda.synchronize()
    assert torch.equal(qi, qo) and torch.equal(ki, ko)
    oq, ok = O.rmsnorm_mrope_qk(q[:64], k[:64], pos[:, :64], rotary_dim=72, theta=1e4,
                                section=None, layout="vision_2d", dtype="f32")
    assert_close(from_dev(qi)[:64], oq, "f32", "in place q")
    assert_close(from_dev(ki)[:64], ok, "f32", "in place k")
