"""Seeded random sweeps of the fused path's geometry against the oracle:
head dims from 2 to 512, partial rotary, every layout with a random valid
section, token strides wider than the rows (so the chunk width drops below
16 bytes when the stride is not a multiple of it), with and without the
norm, all three precisions, in place and out of place, wide position
ranges; eight of them at 2048-4096 tokens with the norm.  A second sweep runs 2048+ tokens without the norm (the flat and
staged kernels), token-major and as the vision tower's per-head planes,
checked on sampled tokens.

Bars: as for the fused path (bf16 within 1 ulp, fp32 within 1e-5) in exact
precision; bit-exact for the tensor-op precisions.
"""
import numpy as np
import pytest

from oracle import mrope_oracle as O
import workloads as W
from tests._helpers import assert_close, from_dev, note, to_dev

pytestmark = pytest.mark.gpu

DIMS = [2, 4, 6, 8, 12, 16, 24, 32, 40, 48, 64, 72, 80, 96, 128, 160, 192, 256, 320, 384, 512]


def _random_case(rng):
    while True:
        dtype = ["bf16", "f32"][rng.integers(2)]
        D = int(rng.choice(DIMS))
        rd = 2 * int(rng.integers(1, D // 2 + 1))
        half = rd // 2
        layout = ["interleaved", "chunked", "vision_2d"][rng.integers(3)]
        if layout == "vision_2d":
            if half % 2:
                continue
            section = None
        elif layout == "chunked":
            n = int(rng.integers(1, 4))
            cuts = np.sort(rng.integers(0, half + 1, n - 1))
            section = tuple(int(x) for x in np.diff(np.concatenate([[0], cuts, [half]])))
        else:
            sh = int(rng.integers(0, half // 3 + 1))
            sw = int(rng.integers(0, half // 3 + 1))
            section = (half - sh - sw, sh, sw)
            try:
                O.axis_table(half, section, layout)
            except AssertionError:
                continue
        return dict(dtype=dtype, D=D, rd=rd, layout=layout, section=section,
                    hq=int(rng.integers(1, 41)), hk=int(rng.integers(0, 9)),
                    T=int(rng.integers(1, 301)), pad=int(rng.choice([0, 1, 2, 8, 24])),
                    norm=bool(rng.integers(2)),
                    precision=["exact", "dtype", "fp32"][rng.integers(3)],
                    inplace=bool(rng.integers(2)), seed=int(rng.integers(1 << 30)))


def _random_large_norm_case(rng):
    """2048-4096 tokens with the norm: one part per tile, tiles of one or two
    tokens, and the row-steps preloaded ahead of the cos/sin prologue."""
    c = _random_case(rng)
    c["T"] = int(rng.integers(2048, 4097))
    c["norm"] = True
    cap = 6_000_000 // (c["T"] * c["D"])
    if c["hq"] + c["hk"] > cap:
        c["hk"] = min(c["hk"], max(cap - 1, 0))
        c["hq"] = max(1, cap - c["hk"])
    return c


_RNG = np.random.default_rng(2024)
CASES = [_random_case(_RNG) for _ in range(48)]
_NRNG = np.random.default_rng(4096)
CASES += [_random_large_norm_case(_NRNG) for _ in range(8)]


@pytest.fixture(scope="module")
def M():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import vlm_multimodal_rotary_amd as lib
    lib.load()
    return lib


def _vector_width(es, D, rd, strides):
    """The chunk width the library can use (the host's rule; 0 = none)."""
    half = rd // 2
    v = 16 // es
    while v >= 1:
        if (D % (2 * v) == 0 and half % v == 0 and (D - rd) % (2 * v) == 0
                and D // (2 * v) <= 64 and all(x % v == 0 for x in strides)):
            return v
        v //= 2
    return 0


def _strided(buf, T, H, D, stride):
    return buf.as_strided((T, H, D), (stride, D, 1))


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_random_geometry(M, case):
    import torch
    c = case
    rng = np.random.default_rng(c["seed"])
    T, D, rd, dtype = c["T"], c["D"], c["rd"], c["dtype"]
    hq, hk = c["hq"], c["hk"]
    q, k = W.random_qk(rng, T, hq, hk, D, dtype, scale=float(2.0 ** rng.integers(-4, 5)))
    n_axes = 2 if c["layout"] == "vision_2d" else (len(c["section"]) if c["layout"] == "chunked"
                                                   else 3)
    pos = rng.integers(-1000, 100000, (n_axes, T)).astype(np.int32)
    wq = W.random_weight(rng, D, dtype) if c["norm"] else None
    wk = W.random_weight(rng, D, dtype) if c["norm"] else None
    note(f"random {c}")
    qs, ks = hq * D + c["pad"], hk * D + c["pad"]
    qbuf = torch.zeros((T * qs + D,), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                       device="cuda")
    kbuf = torch.zeros((T * max(ks, 1) + D,), dtype=qbuf.dtype, device="cuda")
    qv, kv = _strided(qbuf, T, hq, D, qs), _strided(kbuf, T, hk, D, max(ks, 1))
    qv.copy_(to_dev(q, dtype))
    if hk:
        kv.copy_(to_dev(k, dtype))
    qo, ko = (qv, kv) if c["inplace"] else (None, None)
    es = 2 if dtype == "bf16" else 4
    strides = [qs] + ([max(ks, 1)] if hk else [])
    if not c["inplace"]:
        strides += [hq * D] + ([hk * D] if hk else [])
    if _vector_width(es, D, rd, strides) == 0:
        # no chunk width fits the strides: the call is refused before any work
        with pytest.raises(M.MropeError) as err:
            M.rmsnorm_mrope_qk(qv, kv, to_dev(pos, "i32"), rd, 1e4, c["section"], c["layout"],
                               wq=to_dev(wq, dtype), wk=to_dev(wk, dtype), q_out=qo, k_out=ko)
        assert err.value.code == -2
        return
    gq, gk = M.rmsnorm_mrope_qk(qv, kv, to_dev(pos, "i32"), rd, 1e4, c["section"], c["layout"],
                                wq=to_dev(wq, dtype), wk=to_dev(wk, dtype), eps=1e-6,
                                q_out=qo, k_out=ko, precision=c["precision"])
    torch.cuda.synchronize()
    oq, ok = O.rmsnorm_mrope_qk(q, k, pos, rotary_dim=rd, theta=1e4, section=c["section"],
                                layout=c["layout"], wq=wq, wk=wk, eps=1e-6, dtype=dtype,
                                precision=c["precision"])
    got_q = from_dev(gq.contiguous())
    got_k = from_dev(gk.contiguous()) if hk else ok
    if c["precision"] == "exact":
        assert_close(got_q, oq, dtype, "random q")
        if hk:
            assert_close(got_k, ok, dtype, "random k")
    else:
        assert np.array_equal(got_q.view(np.uint8), oq.view(np.uint8))
        assert np.array_equal(got_k.view(np.uint8), ok.view(np.uint8))
    # rows of the padding stay untouched
    if c["pad"] and T > 1:
        tail = from_dev(qbuf[hq * D:qs].contiguous())
        assert np.all(tail.view(np.uint8) == 0)


# Long launches (2048+ tokens) without RMSNorm take the flat or the staged
# kernel; random shapes, strides, precisions and output orders, checked on
# sampled tokens.
LONG_DIMS = [8, 16, 24, 40, 48, 64, 72, 80, 96, 128, 160, 256]


def _random_long_case(rng, planes=False):
    while True:
        dtype = ["bf16", "f32"][rng.integers(2)]
        D = int(rng.choice(LONG_DIMS))
        rd = 2 * int(rng.integers(1, D // 2 + 1))
        if rd % 4 and rng.integers(2):
            continue                       # mostly even halves (the staged kernel's rule)
        layout = "vision_2d" if planes else ["interleaved", "vision_2d"][rng.integers(2)]
        if layout == "vision_2d" and (rd // 2) % 2:
            continue
        section = None
        if layout == "interleaved":
            half = rd // 2
            sh = int(rng.integers(0, half // 3 + 1))
            sw = int(rng.integers(0, half // 3 + 1))
            section = (half - sh - sw, sh, sw)
            try:
                O.axis_table(half, section, layout)
            except AssertionError:
                continue
        return dict(dtype=dtype, D=D, rd=rd, layout=layout, section=section,
                    hq=int(rng.integers(1, 25)), hk=int(rng.integers(0, 9)),
                    T=int(rng.integers(2048, 2600)), pad=int(rng.choice([0, 8, 16, 3])),
                    precision=["exact", "dtype", "fp32"][rng.integers(3)],
                    inplace=bool(rng.integers(2)), planes=planes,
                    seed=int(rng.integers(1 << 30)))


_LRNG = np.random.default_rng(2025)
LONG_CASES = ([_random_long_case(_LRNG) for _ in range(16)] +
              [_random_long_case(_LRNG, planes=True) for _ in range(8)])


@pytest.mark.parametrize("case", LONG_CASES, ids=[f"L{i}" for i in range(len(LONG_CASES))])
def test_random_long_launch(M, case):
    import torch
    c = case
    rng = np.random.default_rng(c["seed"])
    T, D, rd, dtype, hq, hk = c["T"], c["D"], c["rd"], c["dtype"], c["hq"], c["hk"]
    q, k = W.random_qk(rng, T, hq, hk, D, dtype)
    n_axes = 2 if c["layout"] == "vision_2d" else 3
    pos = rng.integers(-1000, 100000, (n_axes, T)).astype(np.int32)
    note(f"random long {c}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 64, replace=False)]))
    oq, ok = O.rmsnorm_mrope_qk(q[rows], k[rows], pos[:, rows], rotary_dim=rd, theta=1e4,
                                section=c["section"], layout=c["layout"], dtype=dtype,
                                precision=c["precision"])
    if c["planes"]:
        # the vision tower's packed qkv into per-head planes (q, k, v of hq heads)
        H = hq
        k2 = W.random_qk(rng, T, H, 0, D, dtype)[0]
        v2 = W.random_qk(rng, T, H, 0, D, dtype)[0]
        qkv_np = np.stack([q, k2, v2], axis=1)
        qkv = to_dev(qkv_np.reshape(T, 3 * H * D), dtype).reshape(T, 3, H, D)
        gq, gk, gv = M.vision_qkv(qkv, to_dev(pos, "i32"), rd, 1e4, precision=c["precision"])
        torch.cuda.synchronize()
        ok2, _ = O.rmsnorm_mrope_qk(k2[rows], k2[rows][:, :0], pos[:, rows], rotary_dim=rd,
                                    theta=1e4, section=None, layout="vision_2d", dtype=dtype,
                                    precision=c["precision"])
        assert np.array_equal(from_dev(gv).transpose(1, 0, 2)[rows].view(np.uint8),
                              v2[rows].view(np.uint8))
        for got, want, what in ((from_dev(gq)[:, rows].transpose(1, 0, 2), oq, "q"),
                                (from_dev(gk)[:, rows].transpose(1, 0, 2), ok2, "k")):
            if c["precision"] == "exact":
                assert_close(got, want, dtype, f"random long planes {what}")
            else:
                assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
        return
    qs, ks = hq * D + c["pad"], hk * D + c["pad"]
    qbuf = torch.zeros((T * qs + D,), dtype=tdt, device="cuda")
    kbuf = torch.zeros((T * max(ks, 1) + D,), dtype=tdt, device="cuda")
    qv, kv = _strided(qbuf, T, hq, D, qs), _strided(kbuf, T, hk, D, max(ks, 1))
    qv.copy_(to_dev(q, dtype))
    if hk:
        kv.copy_(to_dev(k, dtype))
    qo, ko = (qv, kv) if c["inplace"] else (None, None)
    es = 2 if dtype == "bf16" else 4
    strides = [qs] + ([max(ks, 1)] if hk else [])
    if not c["inplace"]:
        strides += [hq * D] + ([hk * D] if hk else [])
    if _vector_width(es, D, rd, strides) == 0:
        # no chunk width fits the strides: the call is refused before any work
        with pytest.raises(M.MropeError) as err:
            M.rmsnorm_mrope_qk(qv, kv, to_dev(pos, "i32"), rd, 1e4, c["section"], c["layout"],
                               q_out=qo, k_out=ko, precision=c["precision"])
        assert err.value.code == -2
        return
    gq, gk = M.rmsnorm_mrope_qk(qv, kv, to_dev(pos, "i32"), rd, 1e4, c["section"], c["layout"],
                                q_out=qo, k_out=ko, precision=c["precision"])
    torch.cuda.synchronize()
    got_q = from_dev(gq.contiguous())[rows]
    got_k = from_dev(gk.contiguous())[rows] if hk else ok
    if c["precision"] == "exact":
        assert_close(got_q, oq, dtype, "random long q")
        if hk:
            assert_close(got_k, ok, dtype, "random long k")
    else:
        assert np.array_equal(got_q.view(np.uint8), oq.view(np.uint8))
        assert np.array_equal(got_k.view(np.uint8), ok.view(np.uint8))
