"""Pins of the CPU oracle to facts the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: values
printed on the pages (tests/golden/*.json, each with its citation), closed
forms, high-precision evaluation, library routines for the special cases that
reduce to them, brute force on tiny inputs, and invariants of the rotation.
The mutation tests at the end plant plausible mistakes in the oracle (on the
CPU) and show that at least one pin fails for each.
"""
import json
import math
import os
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import mrope_oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _nearest_f32_of_decimal(v: Decimal) -> np.float32:
    """The binary32 nearest to a high-precision decimal (ties to even)."""
    f = np.float32(float(v))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        d = abs(Decimal(float(c)) - v)
        key = (d, int(np.array(c, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


# ---------------------------------------------------------------------------
# Rounding primitives
# ---------------------------------------------------------------------------

def check_fl32():
    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000),
                           [1 / 3, 2 / 3, 1e-40, 3.4028235e38, 0.1]])
    for v in vals:
        ref = struct.unpack("<f", struct.pack("<f", float(v)))[0]
        assert float(O.fl32(v)) == ref


def check_bf16_rounding():
    import torch
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(200000) * 10.0 ** rng.integers(-5, 5, 200000)).astype(np.float32)
    # exact ties (low 16 bits == 0x8000) with odd and even kept parts
    ties = (rng.integers(0, 2 ** 15, 2000, dtype=np.uint32) << 17 | 0x8000 |
            (rng.integers(0, 2, 2000, dtype=np.uint32) << 16)).astype(np.uint32)
    ties &= np.uint32(0x7F7FFFFF)
    x = np.concatenate([x, ties.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(x), ref)
    # brute force: the result is the nearer of the two bf16 neighbours, ties even
    bits = O.f32_to_bf16_bits(x[:5000])
    for xi, b in zip(x[:5000].astype(np.float64), bits):
        lo = int(np.array(xi, dtype=np.float32).view(np.uint32)) >> 16
        cand = []
        for kb in (lo, lo + 1):
            v = float(np.array(kb << 16, dtype=np.uint32).view(np.float32)) if kb < 0x10000 else None
            if v is not None:
                cand.append((abs(Fraction(v) - Fraction(float(xi))), kb & 1, kb))
        cand.sort()
        assert int(b) == cand[0][2]


def test_fl32_is_binary32_rounding():
    check_fl32()


def test_bf16_rounding_nearest_even():
    check_bf16_rounding()


# ---------------------------------------------------------------------------
# inv_freq
# ---------------------------------------------------------------------------

def check_inv_freq_printed():
    g = _golden("inv_freq_printed.json")
    for case in g["cases"]:
        got = O.inv_freq(case["dim"], case["theta"])
        assert got.shape == (len(case["values"]),)
        assert np.all(np.abs(got.astype(np.float64) - case["values"]) < 0.5 * 10 ** -g["digits"] + 1e-12)


def check_inv_freq_exact():
    getcontext().prec = 60
    tables = [(128, 1e6), (64, 1e7), (16, 1e4), (36, 1e4), (8, 1e4), (6, 100.0), (256, 1e4)]
    for dim, theta in tables:
        got = O.inv_freq(dim, theta)
        for i in range(dim // 2):
            exact = Decimal(theta) ** (Decimal(-2 * i) / Decimal(dim))
            assert got[i] == _nearest_f32_of_decimal(exact), (dim, theta, i)


def test_inv_freq_printed():
    check_inv_freq_printed()


def test_inv_freq_closed_form():
    # theta = 1e4, dim = 8: 10^-i exactly, rounded once to binary32
    assert [float(v) for v in O.inv_freq(8, 1e4)] == [float(np.float32(10.0 ** -i)) for i in range(4)]
    # theta = 1e6, dim = 6: 10^(-2i)
    assert [float(v) for v in O.inv_freq(6, 1e6)] == [float(np.float32(10.0 ** (-2 * i))) for i in range(3)]
    # the first frequency is always exactly 1
    for dim, theta in [(128, 1e6), (64, 1e7), (36, 1e4)]:
        assert O.inv_freq(dim, theta)[0] == 1.0


def test_inv_freq_nearest_binary32_of_exact_value():
    check_inv_freq_exact()


def test_partial_rotary_frequencies_use_rotary_dim():
    # RoPE post: frequencies are computed over the 64 rotated dims, not cut
    # from a 256-dim table: inv[1] = 1e7^(-2/64), not 1e7^(-2/256).
    inv = O.column_inv(32, 1e7, "interleaved", 64)
    assert inv.shape == (32,)
    assert inv[1] == np.float32(1e7 ** (-2 / 64))
    assert inv[1] != np.float32(1e7 ** (-2 / 256))


# ---------------------------------------------------------------------------
# Axis tables
# ---------------------------------------------------------------------------

def _probe_digits(half, section, layout):
    """acos(cos) probe with inv = ones and positions t=1, h=2, w=3."""
    pos = np.array([[1], [2], [3]], dtype=np.int32)
    inv = np.ones(half, dtype=np.float32)
    c, _ = O.mrope_cos_sin(pos, inv, section, layout, 2 * half)
    return [int(round(math.acos(float(v)))) for v in c[0]]


def check_acos_probe():
    g = _golden("acos_probe.json")
    letters = {"T": 1, "H": 2, "W": 3}
    for case in g["cases"]:
        got = _probe_digits(case["half"], case["section"], case["layout"])
        if "digits" in case:
            want = [int(ch) for ch in case["digits"]]
        else:
            want = [letters[ch] for ch in case["letters"]]
        assert got == want + want, (case, got)
    for case in g["j7"]["cases"]:
        axis = O.axis_table(case["half"], case["section"], "interleaved")
        assert "THW"[axis[7]] == case["axis"]
    q = g["qwen35"]
    axis = O.axis_table(q["half"], q["section"], "interleaved")
    for a, name in enumerate("THW"):
        assert [j for j in range(q["half"]) if axis[j] == a] == q[name]


def test_acos_probe_axis_tables():
    check_acos_probe()


def test_vision_axis_and_frequencies():
    half = 36
    axis = O.axis_table(half, None, "vision_2d")
    assert list(axis) == [0] * 18 + [1] * 18
    invc = O.column_inv(half, 1e4, "vision_2d", 72)
    getcontext().prec = 60
    for i in range(18):
        # qwen3vis.rs rope_angles: 1 / 10000^(2i/36), shared by row and column
        exact = 1 / Decimal(10000) ** (Decimal(2 * i) / Decimal(36))
        assert invc[i] == _nearest_f32_of_decimal(exact)
        assert invc[i + 18] == invc[i]


def test_interleaved_rejects_sections_the_rule_cannot_place():
    # [2,4,2] over half = 8: H can only take j = 1, 4, 7 (three columns, not four)
    with pytest.raises(AssertionError):
        O.axis_table(8, (2, 4, 2), "interleaved")
    with pytest.raises(AssertionError):
        O.axis_table(8, (4, 2, 1), "interleaved")     # sum != half


# ---------------------------------------------------------------------------
# Positions (input builder) and angles
# ---------------------------------------------------------------------------

def test_position_table_worked_example():
    g = _golden("position_table.json")
    segs = [(k, tuple(v) if isinstance(v, list) else v) for k, v in g["segments"]]
    pos, delta = W.rope_index(segs, merge=g["merge"])
    assert pos.tolist() == [g["T"], g["H"], g["W"]]
    assert pos[:, g["I12_column"]].tolist() == g["I12_position"]
    assert delta == 7 - 10


def check_i12_angles():
    g = _golden("i12_angles.json")
    rd = g["rotary_dim"]
    half = rd // 2
    axis = O.axis_table(half, g["section"], "interleaved")
    # position factors: inv = ones makes the angle equal the chosen coordinate
    pos = np.array(g["I12"], dtype=np.int32).reshape(3, 1)
    a = O.angles(pos, axis, np.ones(half, dtype=np.float32))[0]
    assert [int(v) for v in a] == [[2, 3, 4][j % 3] for j in range(half)]
    c, s = O.mrope_cos_sin(pos, np.ones(half, dtype=np.float32), g["section"], "interleaved", rd)
    for j, jp, coord in g["pairs"]:
        assert c[0, j] == c[0, jp] and s[0, j] == s[0, jp]
        ang = math.atan2(float(s[0, j]), float(c[0, j])) % (2 * math.pi)
        assert int(round(ang)) == coord
    # with the real frequencies each angle is fl32(coordinate * inv[j])
    inv = O.inv_freq(rd, 1e7)
    a = O.angles(pos, axis, inv)[0]
    for j in range(half):
        assert a[j] == np.float32(np.float32([2, 3, 4][j % 3]) * inv[j])
    text = np.array(g["text"], dtype=np.int32).reshape(3, 1)
    a = O.angles(text, axis, inv)[0]
    assert np.array_equal(a, (np.float32(6) * inv).astype(np.float32))


def test_i12_angles():
    check_i12_angles()


# ---------------------------------------------------------------------------
# cos / sin
# ---------------------------------------------------------------------------

def check_cos_sin_printed():
    g = _golden("rotary_printed.json")
    pos = np.full((3, 1), g["position"], dtype=np.int32)
    c, s = O.mrope_cos_sin(pos, np.array(g["inv_freq"], dtype=np.float32), g["section"],
                           g["layout"], g["D"])
    tol = 0.5 * 10 ** -g["digits"] + 1e-9
    assert np.all(np.abs(c[0].astype(np.float64) - g["cos"]) <= tol)
    assert np.all(np.abs(s[0].astype(np.float64) - g["sin"]) <= tol)


def test_cos_sin_printed():
    check_cos_sin_printed()


def test_cos_sin_is_nearest_binary32_of_exact_trig():
    import mpmath
    mpmath.mp.dps = 50
    rng = np.random.default_rng(13)
    # angles as the workloads make them: up to ~3.3e4 rad
    a = np.concatenate([rng.uniform(0, 33000, 300), rng.uniform(-4, 4, 100)]).astype(np.float32)
    axis = np.zeros(1, dtype=np.uint8)
    for v in a:
        c, s = O.cos_sin_half(np.array([[1]], dtype=np.int32), axis, np.array([v], dtype=np.float32))
        ec = Decimal(mpmath.nstr(mpmath.cos(mpmath.mpf(float(v))), 45))
        es = Decimal(mpmath.nstr(mpmath.sin(mpmath.mpf(float(v))), 45))
        assert c[0, 0] == _nearest_f32_of_decimal(ec)
        assert s[0, 0] == _nearest_f32_of_decimal(es)


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

def check_rmsnorm_printed():
    g = _golden("rmsnorm_printed.json")
    x = np.array(g["x"], dtype=np.float32)
    w = np.array(g["w"], dtype=np.float32)
    y = O.rms_norm(x, w, g["eps"], "f32").astype(np.float64)
    assert np.all(np.abs(y - np.array(g["y"])) <= 0.5 * 10 ** -g["digits"] + 1e-9)


def check_rmsnorm_bf16_order():
    g = _golden("rmsnorm_bf16_order.json")
    x = np.array(g["x_bf16_bits"], dtype=np.uint16)
    w = np.array(g["w_bf16_bits"], dtype=np.uint16)
    y = O.bf16_bits_to_f64(O.rms_norm(x, w, g["eps"], "bf16"))
    assert y[g["element"]] == g["correct"]


def check_rms_scale_exact():
    getcontext().prec = 60
    rng = np.random.default_rng(14)
    for D, scale in [(128, 1.0), (256, 3.0), (72, 0.01), (16, 100.0)]:
        for _ in range(40):
            x = O.bf16_bits_to_f64(O.f32_to_bf16_bits((scale * rng.standard_normal(D)).astype(np.float32)))
            eps = 1e-6
            ssq = sum(Fraction(float(v)) ** 2 for v in x)
            m = Decimal(ssq.numerator) / Decimal(ssq.denominator) / Decimal(D) + Decimal(float(np.float32(eps)))
            exact = 1 / m.sqrt()
            assert np.float32(O.rms_scale(x, eps)) == _nearest_f32_of_decimal(exact)


def test_rmsnorm_printed():
    check_rmsnorm_printed()


def test_rmsnorm_bf16_cast_before_weight():
    check_rmsnorm_bf16_order()


def test_rms_scale_is_nearest_binary32():
    check_rms_scale_exact()


def test_rmsnorm_fp32_is_plain_definition_within_rounding():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((7, 3, 40)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(40)).astype(np.float32)
    y = O.rms_norm(x, w, 1e-6, "f32").astype(np.float64)
    xd = x.astype(np.float64)
    ref = xd / np.sqrt(np.mean(xd ** 2, axis=-1, keepdims=True) + np.float32(1e-6)) * w
    assert np.max(np.abs(y - ref) / np.abs(ref)) < 2 ** -22


# ---------------------------------------------------------------------------
# Rotation
# ---------------------------------------------------------------------------

def check_rotary_printed():
    g = _golden("rotary_printed.json")
    assert O.rotate_half(np.array(g["rotate_half"]["x"])).tolist() == g["rotate_half"]["y"]
    pos = np.full((3, 1), g["position"], dtype=np.int32)
    c, s = O.mrope_cos_sin(pos, np.array(g["inv_freq"], dtype=np.float32), g["section"],
                           g["layout"], g["D"])
    tol = 0.5 * 10 ** -g["digits"] + 1e-9
    for case in g["apply"]:
        x = np.array(case["x"], dtype=np.float32).reshape(1, 1, g["D"])
        qo, ko = O.apply_rotary_qk(x, x, c, s, g["D"], "f32")
        assert np.all(np.abs(qo.reshape(-1).astype(np.float64) - case["y"]) <= tol), qo
        assert np.array_equal(qo, ko)


def check_rotation_bruteforce():
    """Explicit D x D matrices: a 2x2 rotation block on each pair (j, j+h), the
    identity on pass-through dims (RoPE post: block-orthogonal map up to a
    fixed channel permutation)."""
    rng = np.random.default_rng(16)
    for D, rd in [(8, 8), (12, 4), (16, 16), (10, 6)]:
        h = rd // 2
        T, H = 5, 3
        y = rng.standard_normal((T, H, D)).astype(np.float32)
        c = rng.uniform(-1, 1, (T, h)).astype(np.float32)
        s = rng.uniform(-1, 1, (T, h)).astype(np.float32)
        cos = np.concatenate([c, c], 1)
        sin = np.concatenate([s, s], 1)
        got = O.apply_rotary_values(y.astype(np.float64), cos, sin, rd)
        for t in range(T):
            M = np.eye(D)
            for j in range(h):
                cj, sj = float(c[t, j]), float(s[t, j])
                M[j, j], M[j, j + h] = cj, -sj
                M[j + h, j], M[j + h, j + h] = sj, cj
            for hh in range(H):
                want = M @ y[t, hh].astype(np.float64)
                assert np.max(np.abs(got[t, hh] - want)) <= 1e-15 * np.max(np.abs(want) + 1)


def test_rotary_printed():
    check_rotary_printed()


def test_rotation_bruteforce_matrices():
    check_rotation_bruteforce()


def test_rotation_direction():
    # pair (a, b) = (1, 0) rotated by +pi/2 must land on (0, 1): out = (a c - b s, b c + a s)
    y = np.zeros((1, 1, 2))
    y[0, 0, 0] = 1.0
    out = O.apply_rotary_values(y, np.array([[0.0, 0.0]]), np.array([[1.0, 1.0]]), 2)
    assert out[0, 0].tolist() == [0.0, 1.0]


def test_pair_norm_preserved():
    rng = np.random.default_rng(17)
    T, H, D = 16, 4, 32
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    pos = rng.integers(0, 5000, (3, T)).astype(np.int32)
    qo, _ = O.rmsnorm_mrope_qk(q, q, pos, rotary_dim=D, theta=1e6, section=(6, 5, 5),
                               layout="interleaved", dtype="f32")
    h = D // 2
    n_in = q[..., :h].astype(np.float64) ** 2 + q[..., h:].astype(np.float64) ** 2
    n_out = qo[..., :h].astype(np.float64) ** 2 + qo[..., h:].astype(np.float64) ** 2
    assert np.max(np.abs(n_in - n_out) / n_in) < 1e-6


def _dot_after_rotation(q, k, pq, pk, section, layout, rd, theta):
    qo, _ = O.rmsnorm_mrope_qk(q, q, pq, rotary_dim=rd, theta=theta, section=section,
                               layout=layout, dtype="f32")
    ko, _ = O.rmsnorm_mrope_qk(k, k, pk, rotary_dim=rd, theta=theta, section=section,
                               layout=layout, dtype="f32")
    return float(np.dot(qo.reshape(-1).astype(np.float64), ko.reshape(-1).astype(np.float64)))


def test_relative_position_mrope_and_vision():
    rng = np.random.default_rng(18)
    for layout, section, rd, n_axes in [("interleaved", (4, 2, 2), 16, 3), ("chunked", (4, 2, 2), 16, 3),
                                        ("vision_2d", None, 16, 2)]:
        q = rng.standard_normal((1, 1, rd)).astype(np.float32)
        k = rng.standard_normal((1, 1, rd)).astype(np.float32)
        pq = rng.integers(0, 40, (n_axes, 1)).astype(np.int32)
        pk = rng.integers(0, 40, (n_axes, 1)).astype(np.int32)
        base = _dot_after_rotation(q, k, pq, pk, section, layout, rd, 1e4)
        for _ in range(4):
            shift = rng.integers(0, 60, (n_axes, 1)).astype(np.int32)   # one shift per axis
            moved = _dot_after_rotation(q, k, pq + shift, pk + shift, section, layout, rd, 1e4)
            assert abs(moved - base) < 1e-4 * (1 + abs(base))
        # a shift of the query alone changes the score (the check has teeth)
        other = _dot_after_rotation(q, k, pq + 1, pk, section, layout, rd, 1e4)
        assert abs(other - base) > 1e-3


def test_text_only_collapses_to_1d_rope_bitwise():
    rng = np.random.default_rng(19)
    T, H, D = 40, 3, 16
    q = O.f32_to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
    p = np.arange(100, 100 + T, dtype=np.int32)
    pos3 = np.stack([p, p, p])
    outs = [O.rmsnorm_mrope_qk(q, q, pos3, rotary_dim=D, theta=1e6, section=(4, 2, 2),
                               layout="interleaved", dtype="bf16")[0],
            O.rmsnorm_mrope_qk(q, q, pos3, rotary_dim=D, theta=1e6, section=(4, 2, 2),
                               layout="chunked", dtype="bf16")[0],
            O.rmsnorm_mrope_qk(q, q, p.reshape(1, -1), rotary_dim=D, theta=1e6, section=(8,),
                               layout="chunked", dtype="bf16")[0]]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_partial_rotary_pass_through_is_copied_and_pairs_are_j_j_plus_rd_half():
    rng = np.random.default_rng(20)
    T, H, D, rd = 3, 2, 24, 8
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    pos = rng.integers(0, 100, (3, T)).astype(np.int32)
    qo, _ = O.rmsnorm_mrope_qk(q, q, pos, rotary_dim=rd, theta=1e4, section=(2, 1, 1),
                               layout="interleaved", dtype="f32")
    assert np.array_equal(qo[..., rd:], q[..., rd:])
    # pair (0, rd/2) keeps its norm; pair (0, D/2) would not be a rotation pair
    n_in = q[..., 0].astype(np.float64) ** 2 + q[..., rd // 2].astype(np.float64) ** 2
    n_out = qo[..., 0].astype(np.float64) ** 2 + qo[..., rd // 2].astype(np.float64) ** 2
    assert np.max(np.abs(n_in - n_out) / n_in) < 1e-6


def test_fused_equals_composition_of_the_parts():
    rng = np.random.default_rng(21)
    T, hq, hk, D, rd = 9, 3, 2, 32, 16
    q, k = W.random_qk(rng, T, hq, hk, D, "bf16")
    wq, wk = W.random_weight(rng, D, "bf16"), W.random_weight(rng, D, "bf16")
    pos = rng.integers(0, 1000, (3, T)).astype(np.int32)
    fq, fk = O.rmsnorm_mrope_qk(q, k, pos, rotary_dim=rd, theta=1e6, section=(4, 2, 2),
                                layout="interleaved", wq=wq, wk=wk, eps=1e-6, dtype="bf16")
    nq, nk = O.rms_norm(q, wq, 1e-6, "bf16"), O.rms_norm(k, wk, 1e-6, "bf16")
    c, s = O.mrope_cos_sin(pos, O.inv_freq(rd, 1e6), (4, 2, 2), "interleaved", rd)
    cq, ck = O.apply_rotary_qk(nq, nk, c, s, rd, "bf16")
    assert np.array_equal(fq, cq) and np.array_equal(fk, ck)


# ---------------------------------------------------------------------------
# Rotation precisions written as tensor operations
# ---------------------------------------------------------------------------

def _torch_tensor_rotation(x_stored, cos, sin, rd, dtype, precision):
    """``x*cos + rotate_half(x)*sin`` evaluated by PyTorch CPU tensor ops, one
    op at a time, in the dtypes the two readings name: cos/sin cast to the
    tensor's dtype ("dtype", M01 drill), or everything upcast to float32 and
    one cast at the end ("fp32", Qwen3-VL vision rotary).  PyTorch's own
    kernels do the rounding, so this is an implementation independent of the
    oracle's float64-plus-explicit-rounding arithmetic."""
    import torch
    if dtype == "bf16":
        x = torch.from_numpy(np.ascontiguousarray(x_stored).view(np.int16)).view(torch.bfloat16)
    else:
        x = torch.from_numpy(np.ascontiguousarray(x_stored))
    c = torch.from_numpy(np.ascontiguousarray(cos))[:, None, :]
    s = torch.from_numpy(np.ascontiguousarray(sin))[:, None, :]
    xr = x[..., :rd]
    if precision == "dtype":
        c, s = c.to(x.dtype), s.to(x.dtype)
    else:
        xr = xr.float()
    h = rd // 2
    rh = torch.cat((-xr[..., h:], xr[..., :h]), dim=-1)
    out = (xr * c + rh * s).to(x.dtype)
    out = torch.cat((out, x[..., rd:]), dim=-1)
    if dtype == "bf16":
        return out.view(torch.int16).numpy().view(np.uint16)
    return out.numpy()


def check_tensor_op_precisions():
    rng = np.random.default_rng(41)
    for dtype in ("bf16", "f32"):
        # 2^20 elements: binary32 arithmetic then one bf16 cast differs from
        # the single rounding on about one element in 40000
        for T, H, D, rd in ((2048, 8, 64, 64), (96, 3, 48, 16)):
            v = rng.standard_normal((T, H, D)) * 2.0 ** rng.integers(-12, 12, (T, H, 1))
            x = O.encode(v, dtype)
            pos = rng.integers(0, 200000, (3, T)).astype(np.int32)
            cos, sin = O.mrope_cos_sin(pos, O.inv_freq(rd, 1e6), (rd // 4, rd // 8, rd // 8),
                                       "interleaved", rd)
            exact = O.apply_rotary_qk(x, x, cos, sin, rd, dtype)[0]
            for precision in ("dtype", "fp32"):
                got = O.apply_rotary_qk(x, x, cos, sin, rd, dtype, precision)[0]
                want = _torch_tensor_rotation(x, cos, sin, rd, dtype, precision)
                assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (dtype, precision)
                # the rounding points matter: each reading differs from one rounding
                if rd == D:
                    assert np.count_nonzero(got != exact) > 0, (dtype, precision)


def test_tensor_op_precisions_match_pytorch_tensor_arithmetic():
    check_tensor_op_precisions()


def test_tensor_op_precisions_differ_where_the_readings_differ():
    """For bf16 the two readings give different results on some elements
    (cos/sin rounded to 8 bits and three roundings, against binary32
    arithmetic and one cast); for binary32 they are the same arithmetic."""
    rng = np.random.default_rng(42)
    T, H, D = 64, 4, 32
    pos = rng.integers(0, 100000, (3, T)).astype(np.int32)
    cos, sin = O.mrope_cos_sin(pos, O.inv_freq(D, 1e6), (8, 4, 4), "interleaved", D)
    xb = O.encode(rng.standard_normal((T, H, D)), "bf16")
    a = O.apply_rotary_qk(xb, xb, cos, sin, D, "bf16", "dtype")[0]
    b = O.apply_rotary_qk(xb, xb, cos, sin, D, "bf16", "fp32")[0]
    assert np.count_nonzero(a != b) > 0
    xf = O.encode(rng.standard_normal((T, H, D)), "f32")
    a = O.apply_rotary_qk(xf, xf, cos, sin, D, "f32", "dtype")[0]
    b = O.apply_rotary_qk(xf, xf, cos, sin, D, "f32", "fp32")[0]
    assert np.array_equal(a, b)


def test_every_precision_is_the_identity_at_position_zero():
    rng = np.random.default_rng(43)
    T, H, D = 5, 2, 16
    pos = np.zeros((3, T), dtype=np.int32)
    for dtype in ("bf16", "f32"):
        x = O.encode(rng.standard_normal((T, H, D)), dtype)
        for precision in O.PRECISIONS:
            out, _ = O.rmsnorm_mrope_qk(x, x, pos, rotary_dim=D, theta=1e6, section=(4, 2, 2),
                                        layout="interleaved", dtype=dtype, precision=precision)
            assert np.array_equal(np.abs(out.astype(np.float64) if dtype == "f32" else
                                         O.decode(out, dtype)),
                                  np.abs(O.decode(x, dtype))), (dtype, precision)


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _mut_rotate_half_wrong_sign(x):
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    return np.concatenate([x[..., h:], -x[..., :h]], axis=-1)


def _mut_axis_slice_end_section(half, section, layout):
    lay = O.layout_id(layout)
    if lay != O.LAYOUT_INTERLEAVED:
        return _ORIG_AXIS(half, section, layout)
    axis = np.zeros(half, dtype=np.uint8)
    for j in range(half):
        if j % 3 == 1 and j < section[1]:
            axis[j] = 1
        elif j % 3 == 2 and j < section[2]:
            axis[j] = 2
    return axis


def _mut_axis_chunked_from_zero(half, section, layout):
    lay = O.layout_id(layout)
    if lay != O.LAYOUT_CHUNKED:
        return _ORIG_AXIS(half, section, layout)
    # the pitfall: every axis' chunk taken from column 0 of its own table is
    # the same table shape; model it as the T table everywhere
    return np.zeros(half, dtype=np.uint8)


def _mut_inv_freq_head_dim(dim, theta):
    return np.array([np.float32(float(theta) ** (-(2.0 * i) / (2 * dim))) for i in range(dim // 2)],
                    dtype=np.float32)


def _mut_rms_eps_outside(row, eps):
    row = np.asarray(row, dtype=np.float64)
    ssq = math.fsum(row * row)
    return float(np.float32(1.0 / (math.sqrt(ssq / row.shape[0]) + float(np.float32(eps)))))


def _mut_rms_sum_not_mean(row, eps):
    row = np.asarray(row, dtype=np.float64)
    return float(np.float32(1.0 / math.sqrt(math.fsum(row * row) + float(np.float32(eps)))))


def _mut_norm_values_multiply_first(x, w, eps, dtype):
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    D = x.shape[-1]
    rows = x.reshape(-1, D)
    out = np.empty_like(rows)
    for i in range(rows.shape[0]):
        n = O.fl32(rows[i] * O.rms_scale(rows[i], eps)).astype(np.float64)
        out[i] = O.bf(n * w) if dtype == "bf16" else O.fl32(n * w)
    return out.reshape(x.shape)


def _mut_gptj_pairs(y, cos, sin, rotary_dim):
    # adjacent-pair (repeat_interleave) convention, which the pages call incompatible
    y = np.asarray(y, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float64)[:, None, :]
    out = y.copy()
    h = rotary_dim // 2
    for j in range(h):
        a, b = y[..., 2 * j], y[..., 2 * j + 1]
        out[..., 2 * j] = a * c[..., j] - b * s[..., j]
        out[..., 2 * j + 1] = b * c[..., j] + a * s[..., j]
    return out


def _mut_cos_sin_swapped(pos, axis, invc):
    c, s = _ORIG_CS(pos, axis, invc)
    return s, c


def _mut_tensor_ops_cos_not_cast(y, cos, sin, rotary_dim, dtype, precision):
    # the cast of cos/sin to the tensor dtype forgotten: binary32 arithmetic
    return _ORIG_TENSOR_OPS(y, cos, sin, rotary_dim, dtype, "fp32")


def _mut_tensor_ops_products_unrounded(y, cos, sin, rotary_dim, dtype, precision):
    # the products kept exact: only the cast at the end rounds
    return O.apply_rotary_values(y, cos, sin, rotary_dim)


_ORIG_AXIS = O.axis_table
_ORIG_CS = O.cos_sin_half
_ORIG_TENSOR_OPS = O.apply_rotary_tensor_ops

MUTATIONS = [
    ("rotate_half", _mut_rotate_half_wrong_sign, check_rotary_printed),
    ("axis_table", _mut_axis_slice_end_section, check_acos_probe),
    ("axis_table", _mut_axis_chunked_from_zero, check_acos_probe),
    ("inv_freq", _mut_inv_freq_head_dim, check_inv_freq_printed),
    ("rms_scale", _mut_rms_eps_outside, check_rms_scale_exact),
    ("rms_scale", _mut_rms_sum_not_mean, check_rmsnorm_printed),
    ("rms_norm_values", _mut_norm_values_multiply_first, check_rmsnorm_bf16_order),
    ("apply_rotary_values", _mut_gptj_pairs, check_rotation_bruteforce),
    ("cos_sin_half", _mut_cos_sin_swapped, check_cos_sin_printed),
    ("apply_rotary_tensor_ops", _mut_tensor_ops_cos_not_cast, check_tensor_op_precisions),
    ("apply_rotary_tensor_ops", _mut_tensor_ops_products_unrounded, check_tensor_op_precisions),
]


@pytest.mark.parametrize("name,mutant,check", MUTATIONS,
                         ids=[f"{n}:{m.__name__}" for n, m, _ in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, check):
    check()                                   # passes on the real oracle
    monkeypatch.setattr(O, name, mutant)
    with pytest.raises(AssertionError):
        check()


# ---------------------------------------------------------------------------
# Decode positions
# ---------------------------------------------------------------------------

def test_decode_position_continues_the_prefill():
    """rope_deltas is the next rotary position minus the valid length (RoPE
    post, get_rope_index), so the first decode token after a prefill sits at
    the prefill's largest position + 1 on every axis; text-only prompts have
    delta 0 and decode continues at the cache length."""
    g = _golden("position_table.json")
    segs = [(k, tuple(v) if isinstance(v, list) else v) for k, v in g["segments"]]
    pos, delta = W.rope_index(segs, merge=g["merge"])
    L = pos.shape[1]
    p = O.decode_positions([L], 3, [delta])
    assert p.tolist() == [int(pos.max()) + 1 + i for i in range(3)]     # 7, 8, 9
    text, d0 = W.rope_index([("text", 5)])
    assert d0 == 0
    assert O.decode_positions([5, 9], 2).tolist() == [5, 6, 9, 10]


def test_decode_equals_prefill_on_the_same_positions():
    """A decode step is the fused path on text positions plus a cache write."""
    rng = np.random.default_rng(40)
    B, n, hq, hk, D, cap = 3, 2, 4, 2, 32, 12
    q, k = W.random_qk(rng, B * n, hq, hk, D, "bf16")
    wq, wk = W.random_weight(rng, D, "bf16"), W.random_weight(rng, D, "bf16")
    cache_len = np.array([0, 5, 11])
    delta = np.array([0, -3, 2])
    cache = W.random_qk(rng, B * cap, hk, 1, D, "bf16")[0].reshape(B, cap, hk, D)
    qo, newc = O.mrope_decode_qk(q, k, cache_len, n, delta, cache, rotary_dim=D, theta=1e6,
                                 wq=wq, wk=wk, eps=1e-6, dtype="bf16")
    pos = O.decode_positions(cache_len, n, delta)
    for layout, sec in [("interleaved", (6, 5, 5)), ("chunked", (6, 5, 5))]:
        fq, fk = O.rmsnorm_mrope_qk(q, k, np.stack([pos, pos, pos]), rotary_dim=D, theta=1e6,
                                    section=sec, layout=layout, wq=wq, wk=wk, eps=1e-6,
                                    dtype="bf16")
        assert np.array_equal(fq, qo)
    assert np.array_equal(newc[0, 0:2], fk[0:2]) and np.array_equal(newc[1, 5:7], fk[2:4])
    assert np.array_equal(newc[2, 11], fk[4])            # slot 12 is past the capacity
    untouched = np.ones((B, cap), bool)
    untouched[0, 0:2] = untouched[1, 5:7] = untouched[2, 11] = False
    assert np.array_equal(newc[untouched], cache[untouched])


# ---------------------------------------------------------------------------
# Vision tower: packed qkv to per-head planes
# ---------------------------------------------------------------------------

def _vision_case(dtype="f32", n=40, H=3, D=16, seed=44):
    rng = np.random.default_rng(seed)
    qkv = O.encode(rng.standard_normal((n, 3, H, D)), dtype)
    pos = np.stack([rng.integers(0, 30, n), rng.integers(0, 30, n)]).astype(np.int32)
    return qkv, pos


def test_vision_qkv_planes_are_the_rotated_heads_and_a_copied_v():
    qkv, pos = _vision_case()
    n, _, H, D = qkv.shape
    q, k, v = O.vision_qkv(qkv, pos, rotary_dim=D, theta=1e4)
    assert q.shape == k.shape == v.shape == (H, n, D)
    # v: the plane of head h is the v slot of head h, bit for bit
    assert np.array_equal(v, qkv[:, 2].transpose(1, 0, 2))
    # q, k: each plane row is a rotation of its own head's slot: pair norms
    # (j, j + D/2) are kept, and slot 0 / slot 1 are not mixed up
    for plane, slot in ((q, 0), (k, 1)):
        src = qkv[:, slot].transpose(1, 0, 2).astype(np.float64)
        out = plane.astype(np.float64)
        h = D // 2
        n_in = src[..., :h] ** 2 + src[..., h:] ** 2
        n_out = out[..., :h] ** 2 + out[..., h:] ** 2
        assert np.max(np.abs(n_in - n_out) / (n_in + 1e-30)) < 1e-6
    # a patch at (0, 0) is not rotated
    pos0 = pos.copy()
    pos0[:, 0] = 0
    q0, _, _ = O.vision_qkv(qkv, pos0, rotary_dim=D, theta=1e4)
    assert np.array_equal(q0[:, 0], qkv[0, 0])


def test_vision_qkv_relative_positions_per_head():
    """Per head, q.k after rotation depends only on the 2-D offset between
    the two patches (the vision rotary is a relative encoding on both axes)."""
    rng = np.random.default_rng(45)
    H, D = 2, 16
    qkv = rng.standard_normal((2, 3, H, D)).astype(np.float32)
    def score(pa, pb):
        q, _, _ = O.vision_qkv(qkv[:1], np.array(pa, dtype=np.int32).reshape(2, 1),
                               rotary_dim=D, theta=1e4)
        _, k, _ = O.vision_qkv(qkv[1:], np.array(pb, dtype=np.int32).reshape(2, 1),
                               rotary_dim=D, theta=1e4)
        return (q[:, 0].astype(np.float64) * k[:, 0].astype(np.float64)).sum(-1)
    base = score((3, 5), (7, 2))
    moved = score((3 + 4, 5 + 9), (7 + 4, 2 + 9))
    assert np.max(np.abs(moved - base)) < 1e-4 * (1 + np.max(np.abs(base)))
    assert np.max(np.abs(score((4, 5), (7, 2)) - base)) > 1e-3


def test_cos_sin_cache_gathered_by_position_is_the_per_token_table():
    """Method 2 (a table by position value, gathered) gives the per-token
    cos/sin of method 1 bit for bit, for every layout's column-to-axis map."""
    rng = np.random.default_rng(46)
    for layout, section, rd, n_axes, dim in [("interleaved", (24, 20, 20), 128, 3, 128),
                                             ("chunked", (16, 24, 24), 128, 3, 128),
                                             ("vision_2d", None, 72, 2, 36)]:
        pos = rng.integers(0, 300, (n_axes, 50)).astype(np.int32)
        cache = O.cos_sin_cache(dim, 1e4, 300)
        half = rd // 2
        axis = O.axis_table(half, section, layout)
        fidx = np.arange(half) % (half // 2) if layout == "vision_2d" else np.arange(half)
        c, s = O.mrope_cos_sin(pos, O.inv_freq(dim, 1e4), section, layout, rd)
        p_col = pos[axis, :].T                           # [T, half] position per column
        gathered = cache[p_col, fidx[None, :]]           # [T, half, 2]
        assert np.array_equal(gathered[..., 0], c[:, :half])
        assert np.array_equal(gathered[..., 1], s[:, :half])
    # and the table itself is cos/sin of the binary32 product, rounded once
    cache = O.cos_sin_cache(8, 100.0, 5)
    inv = O.inv_freq(8, 100.0)
    for p_ in range(5):
        for i in range(4):
            a = float(np.float32(np.float32(p_) * inv[i]))
            assert cache[p_, i, 0] == np.float32(math.cos(a))
            assert cache[p_, i, 1] == np.float32(math.sin(a))
