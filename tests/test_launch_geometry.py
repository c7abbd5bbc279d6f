"""CPU model of the q/k kernel's launch geometry and lane mapping.

Mirrors the host plan (chunk width, lanes per row, tokens per tile, grid) and
the kernel's per-lane indexing, then checks for each geometry that every
output element is written exactly once, every read stays inside its buffer,
and every cos/sin LDS index stays inside the wavefront's slice.
"""
import numpy as np
import pytest

import workloads as W

WAVE = 64
WPB = 4


def pick_vec(es, D, rd, aligned_bytes=16, strides=()):
    half = rd // 2
    v = 16 // es
    while v >= 1:
        if (D % (2 * v) == 0 and half % v == 0 and (D - rd) % (2 * v) == 0
                and D // (2 * v) <= WAVE and aligned_bytes % (v * es) == 0
                and all(s % v == 0 for s in strides)):
            return v
        v //= 2
    return 0


def plan(T, D, rd, es, cus=256, fused=True):
    v = pick_vec(es, D, rd)
    assert v, (D, rd, es)
    half = rd // 2
    lpr = D // (2 * v)
    rpw = WAVE // lpr
    lrot = half // v
    target = cus * 16
    nt = (T + target - 1) // target
    nt_max = max(1, min(64, 1024 // half)) if half else 64
    nt = max(1, min(nt, nt_max))
    ntiles = (T + nt - 1) // nt
    grid = min((ntiles + WPB - 1) // WPB, 1048576)
    lds_floats_per_wave = 2 * nt * half if fused else 0
    return dict(v=v, half=half, lpr=lpr, rpw=rpw, lrot=lrot, nt=nt, ntiles=ntiles, grid=grid,
                lds_floats=lds_floats_per_wave)


def simulate(T, heads, D, rd, es, fused=True, U=4):
    """Returns per-slot write counts of q/k outputs; asserts read bounds."""
    p = plan(T, D, rd, es, fused=fused)
    v, half, lpr, rpw, lrot, nt = p["v"], p["half"], p["lpr"], p["rpw"], p["lrot"], p["nt"]
    writes = [np.zeros((T, H, D), dtype=np.int32) for H in heads]
    lanes = np.arange(WAVE)
    grp = lanes // lpr
    l = lanes - grp * lpr
    lane_on = grp < rpw
    col_a = np.where(l < lrot, l * v, rd + (l - lrot) * v)
    col_b = np.where(l < lrot, half + l * v, rd + (lpr - lrot + (l - lrot)) * v)
    assert np.all(col_a + v <= D) and np.all(col_b + v <= D)
    wstride = p["grid"] * WPB
    for wave0 in range(min(wstride, p["ntiles"])):
        for tile in range(wave0, p["ntiles"], wstride):
            t0 = tile * nt
            ntok = min(nt, T - t0)
            if fused:
                n = ntok * half
                assert n <= p["lds_floats"] // 2
            for s, H in enumerate(heads):
                if H == 0:
                    continue
                nrows = ntok * H
                tl = grp // H
                h = grp - tl * H
                dq, dr = rpw // H, rpw % H
                for r0 in range(0, nrows, U * rpw):
                    for u in range(U):
                        r = r0 + u * rpw + grp
                        ok = lane_on & (r < nrows)
                        # the incremental (token, head) equals the division
                        assert np.all(tl[ok] == r[ok] // H) and np.all(h[ok] == r[ok] % H)
                        tok = t0 + tl
                        assert np.all(tok[ok] < T) and np.all(h[ok] < H)
                        tlr = np.where(ok, tl, 0)
                        if fused:
                            rot = l < lrot
                            o = tlr * half + col_a
                            assert np.all(o[rot] + v <= nt * half)
                        for i in np.nonzero(ok)[0]:
                            writes[s][tok[i], h[i], col_a[i]:col_a[i] + v] += 1
                            writes[s][tok[i], h[i], col_b[i]:col_b[i] + v] += 1
                        h = h + dr
                        tl = tl + dq
                        wrap = h >= H
                        h = np.where(wrap, h - H, h)
                        tl = np.where(wrap, tl + 1, tl)
    return writes, p


GEOMS = [
    # (T, (hq, hk), D, rd, elem_bytes)
    (16, (2, 1), 16, 16, 4),        # tiny_mrope
    (777, (32, 4), 128, 128, 2),    # omni text prefill window
    (1400, (24, 4), 256, 64, 2),    # qwen3.5 partial rotary window
    (700, (28, 4), 128, 128, 2),    # chunked video window
    (4500, (16, 16), 72, 72, 4),    # vision window
    (131, (5, 3), 72, 72, 2),
    (131, (5, 3), 256, 128, 4),
    (131, (5, 3), 512, 512, 2),
    (131, (5, 3), 2, 2, 2),
    (131, (5, 3), 16, 8, 4),
    (131, (5, 3), 48, 16, 2),
    (1, (32, 4), 128, 128, 2),
    (50, (32, 0), 128, 128, 2),
    (333, (6, 6), 64, 64, 2),
]


@pytest.mark.parametrize("T,heads,D,rd,es", GEOMS)
def test_every_output_written_once_and_reads_in_bounds(T, heads, D, rd, es):
    writes, p = simulate(T, heads, D, rd, es)
    for s, H in enumerate(heads):
        if H:
            assert np.all(writes[s] == 1), (s, np.unique(writes[s]))
    assert p["lds_floats"] * WPB * 4 <= 32 * 1024


def test_rms_norm_only_geometry():
    writes, p = simulate(203, (3, 0), 1024, 0, 2, fused=False)
    assert np.all(writes[0] == 1)
    writes, p = simulate(203, (3, 0), 72, 0, 4, fused=False)
    assert np.all(writes[0] == 1)


def test_full_size_plans():
    for name, wl in W.WORKLOADS.items():
        p = plan(wl.T, wl.D, wl.rotary_dim, wl.elem_bytes)
        assert p["ntiles"] * p["nt"] >= wl.T > (p["ntiles"] - 1) * p["nt"]
        assert p["lds_floats"] * WPB * 4 <= 32 * 1024
