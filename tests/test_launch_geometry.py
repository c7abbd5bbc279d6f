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


WAVE_TOKENS = 1   # tokens per wavefront without RMSNorm (the host takes 1, 2 or 4 with it)
OUT_OF_RANGE = 0x80000000


MIN_WAVES = 2048  # wavefronts a launch aims for before splitting tiles (MROPE_MIN_WAVES)


def plan(T, D, rd, es, fused=True, wave_tokens=WAVE_TOKENS, heads=(1, 1), min_waves=MIN_WAVES):
    v = pick_vec(es, D, rd)
    assert v, (D, rd, es)
    half = rd // 2
    lpr = D // (2 * v)
    rpw = WAVE // lpr
    lrot = half // v
    nt_cap = max(1, min(16, 512 // half)) if half else 16
    nt = max(1, min(nt_cap, wave_tokens))
    tiles = -(-T // nt)
    tile_steps = sum(-(-nt * H // rpw) for H in heads)
    parts = max(1, min(tile_steps, -(-min_waves // tiles)))
    return dict(v=v, half=half, lpr=lpr, rpw=rpw, lrot=lrot, nt=nt, nwaves=tiles * parts,
                parts=parts, lds_doubles=2 * nt * half if fused else 0)


def first_row_split(r, H):
    """The kernel's r / H through a binary32 reciprocal, corrected once."""
    tl = int(np.float32(np.float32(r) * np.float32(np.float32(1.0) / np.float32(H))))
    if tl * H > r:
        tl -= 1
    if (tl + 1) * H <= r:
        tl += 1
    return tl, r - tl * H


def first_row_split_lanes(r, H):
    """first_row_split over an array of rows (the same binary32 arithmetic)."""
    r = np.asarray(r, dtype=np.int64)
    inv = np.float32(np.float32(1.0) / np.float32(H))
    tl = (r.astype(np.float32) * inv).astype(np.float32).astype(np.int64)
    tl = np.where(tl * H > r, tl - 1, tl)
    tl = np.where((tl + 1) * H <= r, tl + 1, tl)
    return tl, r - tl * H


def simulate(T, heads, D, rd, es, fused=True, U=2, wave_tokens=WAVE_TOKENS, min_waves=MIN_WAVES,
             head_major=False, pre_steps=0):
    """Returns per-slot write counts of the outputs (q, k and, with three
    head counts, the copied v of a packed qkv); asserts read and write
    bounds.  head_major puts the outputs in per-head planes.  pre_steps
    row-steps are issued ahead of the rest (the decode and RMSNorm forms
    preload 1 and 2).  U (steps per batch of loads) orders the steps within a
    run but not which rows they cover, so the model takes them one by one."""
    p = plan(T, D, rd, es, fused=fused, wave_tokens=wave_tokens, heads=heads,
             min_waves=min_waves)
    v, half, lpr, rpw, lrot, nt = p["v"], p["half"], p["lpr"], p["rpw"], p["lrot"], p["nt"]
    parts = p["parts"]
    writes = [np.zeros((T, H, D), dtype=np.int32) for H in heads]
    lanes = np.arange(WAVE)
    grp = lanes // lpr
    l = lanes - grp * lpr
    lane_on = grp < rpw
    col_a = np.where(l < lrot, l * v, rd + (l - lrot) * v)
    col_b = np.where(l < lrot, half + l * v, rd + (lpr - lrot + (l - lrot)) * v)
    assert np.all(col_a + v <= D) and np.all(col_b + v <= D)
    xts = [H * D + 8 * v for H in heads]          # a token stride wider than the rows
    if head_major:
        yts = [D for H in heads]
        yhs = [T * D + 4 * v for H in heads]       # planes with a gap between them
    else:
        yts = [H * D + 4 * v for H in heads]
        yhs = [D for H in heads]
    for w in range(p["nwaves"]):
        tile, part = divmod(w, parts)
        t0 = tile * nt
        assert t0 < T
        ntok = min(nt, T - t0)
        if fused:
            assert ntok * half <= p["lds_doubles"] // 2
        pre = [0]
        for H in heads:
            pre.append(pre[-1] + -(-ntok * H // rpw))
        steps_all = pre[-1]
        sb, se = steps_all * part // parts, steps_all * (part + 1) // parts
        def run(s, lo, enabled):
            """Row-steps lo, lo + 1, ... of tensor s, one per entry of
            `enabled` (False: the step is issued with every lane masked)."""
            H = heads[s]
            extent = ((ntok - 1) * xts[s] + H * D) * es   # tile buffer size in bytes
            out_extent = ((ntok - 1) * yts[s] + (H - 1) * yhs[s] + D) * es
            assert extent < OUT_OF_RANGE and out_extent < OUT_OF_RANGE
            nrows = ntok * H
            tl, h = first_row_split_lanes(lo * rpw + grp, H)
            dq, dr = rpw // H, rpw % H
            xo = (tl * xts[s] + h * D) * es
            xinc = (dq * xts[s] + dr * D) * es
            xwrap = (xts[s] - H * D) * es
            yo = (tl * yts[s] + h * yhs[s]) * es
            yinc = (dq * yts[s] + dr * yhs[s]) * es
            ywrap = (yts[s] - H * yhs[s]) * es
            r0 = lo * rpw
            for on in enabled:
                r = r0 + grp
                ok = lane_on & (r < nrows) & on
                if on:
                    assert np.all(tl[ok] == r[ok] // H) and np.all(h[ok] == r[ok] % H)
                off = np.where(ok, xo, OUT_OF_RANGE)
                # live rows stay inside the tile buffer, masked ones outside it
                assert np.all(off[ok] + col_b[ok] * es + v * es <= extent)
                assert np.all(off[~ok] >= extent)
                yoff = np.where(ok, yo, OUT_OF_RANGE)
                assert np.all(yoff[ok] + col_b[ok] * es + v * es <= out_extent)
                assert np.all(yoff[ok] >= 0)
                assert np.all(yoff[~ok] >= out_extent)
                # the store address is the element (t, h, col) of the view
                assert np.all(yoff[ok] == (tl[ok] * yts[s] + h[ok] * yhs[s]) * es)
                tlr = np.where(ok, tl, 0)
                if fused:
                    o = tlr * half + col_a
                    assert np.all(o[l < lrot] + v <= nt * half)
                tok = (t0 + tl[ok])[:, None]
                hh = h[ok][:, None]
                span_v = np.arange(v)[None, :]
                np.add.at(writes[s], (tok, hh, col_a[ok][:, None] + span_v), 1)
                np.add.at(writes[s], (tok, hh, col_b[ok][:, None] + span_v), 1)
                xo = xo + xinc
                yo = yo + yinc
                h = h + dr
                tl = tl + dq
                wrap = h >= H
                h = np.where(wrap, h - H, h)
                tl = np.where(wrap, tl + 1, tl)
                xo = np.where(wrap, xo + xwrap, xo)
                yo = np.where(wrap, yo + ywrap, yo)
                r0 += rpw

        def span(s):
            return max(sb, pre[s]) - pre[s], min(se, pre[s + 1]) - pre[s]

        # the first pre_steps row-steps of the part's first q or k work,
        # issued before the cos/sin prologue (masked past the available ones)
        s_pre, n_pre = None, 0
        if pre_steps:
            for s in (0, 1):
                if s < len(heads) and heads[s] > 0 and span(s)[0] < span(s)[1]:
                    s_pre = s
                    break
            if s_pre is not None:
                lo, hi = span(s_pre)
                n_pre = min(pre_steps, hi - lo)
                run(s_pre, lo, [u < n_pre for u in range(pre_steps)])
        for s, H in enumerate(heads):
            if H == 0:
                continue
            lo, hi = span(s)
            if s == s_pre:
                lo += n_pre
            if lo >= hi:
                continue
            run(s, lo, [True] * (hi - lo))
    return writes, p


def test_first_row_split_exact():
    for H in range(1, 4097):
        for g in range(64):
            assert first_row_split(g, H) == (g // H, g % H), (g, H)
    rng = np.random.default_rng(1)
    for H in list(range(1, 200)) + [int(x) for x in rng.integers(1, 100000, 200)]:
        r = rng.integers(0, 2 ** 23, 64)
        tl, h = first_row_split_lanes(r, H)
        assert np.array_equal(tl, r // H) and np.array_equal(h, r % H)
        assert [first_row_split(int(x), H) for x in r] == list(zip(tl.tolist(), h.tolist()))
    rng = np.random.default_rng(0)
    for _ in range(20000):
        H = int(rng.integers(1, 100000))
        r = int(rng.integers(0, 2 ** 23))
        assert first_row_split(r, H) == (r // H, r % H), (r, H)


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


@pytest.mark.parametrize("U,wave_tokens,min_waves,pre_steps", [
    (1, 1, 1, 0), (2, 1, 2048, 0), (4, 2, 2048, 0), (2, 16, 64, 0), (2, 1, 1 << 20, 0),
    (2, 1, 2048, 1),                                                 # decode's preload
    (1, 1, 1, 2), (2, 1, 2048, 2), (4, 2, 2048, 2), (2, 16, 64, 2), (2, 1, 1 << 20, 2),
])
@pytest.mark.parametrize("T,heads,D,rd,es", GEOMS)
def test_every_output_written_once_and_reads_in_bounds(T, heads, D, rd, es, U, wave_tokens,
                                                         min_waves, pre_steps):
    writes, p = simulate(T, heads, D, rd, es, U=U, wave_tokens=wave_tokens, min_waves=min_waves,
                         pre_steps=pre_steps)
    for s, H in enumerate(heads):
        if H:
            assert np.all(writes[s] == 1), (s, np.unique(writes[s]))
    assert p["lds_doubles"] * WPB * 8 <= 32 * 1024


def test_rms_norm_only_geometry():
    writes, p = simulate(203, (3, 0), 1024, 0, 2, fused=False)
    assert np.all(writes[0] == 1)
    writes, p = simulate(203, (3, 0), 72, 0, 4, fused=False)
    assert np.all(writes[0] == 1)


def test_decode_sized_launch_splits_tiles():
    p = plan(512, 128, 128, 2, heads=(32, 4))
    assert p["parts"] == 4 and p["nwaves"] == 2048
    for pre_steps in (0, 1):
        writes, p = simulate(512, (32, 4), 128, 128, 2, pre_steps=pre_steps)
        assert np.all(writes[0] == 1) and np.all(writes[1] == 1)


def test_full_size_plans():
    for name, wl in W.WORKLOADS.items():
        p = plan(wl.T, wl.D, wl.rotary_dim, wl.elem_bytes, heads=(wl.hq, wl.hk))
        tiles = p["nwaves"] // p["parts"]
        assert tiles * p["nt"] >= wl.T > (tiles - 1) * p["nt"]
        assert p["lds_doubles"] * WPB * 8 <= 32 * 1024
        if wl.T >= MIN_WAVES:
            assert p["parts"] == 1


@pytest.mark.parametrize("head_major", [False, True])
@pytest.mark.parametrize("T,heads,D,rd,es,min_waves", [
    (777, (16, 16, 16), 72, 72, 4, 2048),    # vision packed qkv, fp32
    (777, (16, 16, 16), 72, 72, 2, 2048),    # bf16
    (300, (6, 6, 6), 128, 64, 2, 2048),
    (129, (5, 5, 5), 80, 80, 4, 1),
    (1, (4, 4, 4), 72, 72, 2, 2048),
    (50, (16, 16, 0), 72, 72, 4, 2048),      # without v
])
def test_three_slot_packed_qkv(T, heads, D, rd, es, min_waves, head_major):
    writes, p = simulate(T, heads, D, rd, es, min_waves=min_waves, head_major=head_major,
                         pre_steps=2)
    for s, H in enumerate(heads):
        if H:
            assert np.all(writes[s] == 1), (s, np.unique(writes[s]))


# ---------------------------------------------------------------------------
# The flat kernel: chunks of the token's block lane after lane, with the
# rotary partner loaded by the same lane.
# ---------------------------------------------------------------------------

FLAT_STEPS = 6


def f32(x):
    return np.float32(x)


def simulate_flat(T, heads, D, rd, es, v, head_major=False):
    half = rd // 2
    cpr, hc, rc = D // v, half // v, rd // v
    cb = v * es
    inv_cpr = f32(f32(1.0) / f32(cpr))
    writes = [np.zeros((T, H, D), dtype=np.int32) for H in heads]
    lanes = np.arange(WAVE)
    for t in range(T):
        for s, H in enumerate(heads):
            if H == 0:
                continue
            rotate = s < 2
            nch = H * cpr
            in_extent = nch * cb
            yhs = T * D + 4 * v if head_major else D
            yts = D if head_major else H * D + 4 * v
            out_extent = ((H - 1) * yhs + D) * es
            assert in_extent < OUT_OF_RANGE and out_extent < OUT_OF_RANGE
            for base in range(0, nch, WAVE * FLAT_STEPS):
                for u in range(FLAT_STEPS):
                    f = base + u * WAVE + lanes
                    ok = f < nch
                    row = (f.astype(np.float32) * inv_cpr).astype(np.int64)
                    row = np.where(row * cpr > f, row - 1, row)
                    row = np.where((row + 1) * cpr <= f, row + 1, row)
                    assert np.all(row == f // cpr)
                    c = f - row * cpr
                    k = np.where(~rotate | (c >= rc), 2, np.where(c < hc, 0, 1))
                    fp = np.where(k == 2, f, np.where(k == 0, f + hc, f - hc))
                    col = np.where(ok & (k < 2), np.where(k == 1, c - hc, c) * v, 0)
                    assert np.all(col + v <= half) or half == 0
                    xo = np.where(ok, f * cb, OUT_OF_RANGE)
                    xp = np.where(ok & (k < 2), fp * cb, OUT_OF_RANGE)
                    assert np.all(xo[ok] + cb <= in_extent) and np.all(xp[ok & (k < 2)] + cb <= in_extent)
                    assert np.all(fp[ok] // cpr == row[ok])          # partner in the same row
                    yoff = np.where(ok, (row * yhs + c * v) * es, OUT_OF_RANGE)
                    assert np.all(yoff[ok] + cb <= out_extent)
                    for i in np.nonzero(ok)[0]:
                        writes[s][t, row[i], c[i] * v:c[i] * v + v] += 1
    return writes


@pytest.mark.parametrize("T,heads,D,rd,es,v", [
    (3, (16, 16, 0), 72, 72, 4, 4),       # vision_2d fp32
    (3, (16, 16, 16), 72, 72, 4, 4),      # vision qkv fp32
    (3, (16, 16, 16), 72, 72, 2, 4),      # vision qkv bf16 (8-byte chunks)
    (2, (28, 4, 0), 128, 128, 2, 8),
    (2, (24, 4, 0), 256, 64, 2, 8),       # partial rotary: pass-through chunks
    (2, (5, 3, 2), 80, 48, 4, 4),
    (2, (40, 8, 0), 384, 384, 4, 4),      # several batches per tensor
    (2, (3, 1, 0), 2, 2, 2, 1),
])
@pytest.mark.parametrize("head_major", [False, True])
def test_flat_every_output_written_once(T, heads, D, rd, es, v, head_major):
    writes = simulate_flat(T, heads, D, rd, es, v, head_major=head_major)
    for s, H in enumerate(heads):
        if H:
            assert np.all(writes[s] == 1), (s, np.unique(writes[s]))


BLOCK = WAVE * WPB
STAGE_LDS_MAX = 64 * 1024   # LDS bytes a staged block may take (kStageLdsMax)
STAGE_V = 3                 # v chunks per lane in registers (kStageV)


def stage_slot_bytes(G, H, D, es):
    chunks = G * H * D * es // 16
    return -(-chunks // WAVE) * WAVE * 16


def div_small(n, d, inv):
    """The staged kernel's quotient through a binary32 reciprocal."""
    q = (n.astype(np.float32) * inv).astype(np.int64)
    q = np.where(q * d > n, q - 1, q)
    q = np.where((q + 1) * d <= n, q + 1, q)
    return q


def simulate_stage(T, heads, D, rd, es, G, head_major, x_pad=0):
    """Model of the staged kernel: per block, the LDS transfers of phase 1,
    the cos/sin indices of phase 2 and the reads and stores of phase 3."""
    half = rd // 2
    ec = 16 // es
    cpr = D * es // 16
    f32 = np.float32
    inv_cpr = f32(f32(1.0) / f32(cpr))
    inv_half = f32(f32(1.0) / f32(half))
    writes = [np.zeros((T, H, D), dtype=np.int32) for H in heads]
    offs, off = [], 0
    for H in heads[:2]:                 # q and k go through LDS, v through registers
        offs.append(off)
        if H:
            off += stage_slot_bytes(G, H, D, es)
    cs_bytes = G * half * 8
    assert off % 16 == 0 and off + cs_bytes <= STAGE_LDS_MAX
    assert G * heads[2] * cpr <= STAGE_V * BLOCK
    lanes = np.arange(WAVE)
    tid = np.arange(BLOCK)
    for blk in range(-(-T // G)):
        t0 = blk * G
        nvalid = min(G, T - t0)
        # phase 1 (q and k to LDS)
        for s, H in enumerate(heads[:2]):
            if H == 0:
                continue
            rcs = H * cpr
            nch = G * rcs
            x_ts = H * D + x_pad
            tsb = x_ts * es
            extent = (nvalid - 1) * tsb + rcs * 16
            inv = f32(f32(1.0) / f32(rcs))
            landed = np.zeros(nch, dtype=np.int32)
            for wib in range(BLOCK // WAVE):
                for kb in range(wib * WAVE, nch, BLOCK):
                    k = kb + lanes
                    g = div_small(k, rcs, inv)
                    ok = (k < nch) & (g < nvalid)
                    vo = g * tsb + (k - g * rcs) * 16
                    assert np.all(vo[ok] + 16 <= extent)
                    assert offs[s] + kb * 16 + WAVE * 16 <= offs[s] + stage_slot_bytes(G, H, D, es)
                    assert np.all(g[k < nch] == k[k < nch] // rcs)
                    landed[k[k < nch]] += 1
            assert np.all(landed == 1)
        # phase 2
        i = np.arange(G * half)
        g = div_small(i, half, inv_half)
        assert np.all(g == i // half) and np.all(g < G)
        # v: chunks in output order straight to registers, then stored
        H = heads[2]
        if H:
            nch = H * G * cpr
            x_ts = H * D + x_pad
            tsb = x_ts * es
            in_extent = (nvalid - 1) * tsb + H * cpr * 16
            yhs = T * D + 8 * ec if head_major else D
            yts = D if head_major else H * D + 8 * ec
            out_extent = ((H - 1) * yhs + (nvalid - 1) * yts + D) * es
            inv_h = f32(f32(1.0) / f32(H))
            for j in range(STAGE_V):
                k = tid + j * BLOCK
                kk = np.where(k < nch, k, 0)
                o = div_small(kk, cpr, inv_cpr)
                c = kk - o * cpr
                if head_major:
                    h, g = o // G, o % G
                else:
                    g = div_small(o, H, inv_h)
                    h = o - g * H
                ok = (k < nch) & (g < nvalid)
                assert np.all(g[ok] * tsb + (h[ok] * cpr + c[ok]) * 16 + 16 <= in_extent)
                yo = (h * yhs + g * yts) * es + c * 16
                assert np.all(yo[ok] + 16 <= out_extent)
                for qq in np.nonzero(ok)[0]:
                    writes[2][t0 + g[qq], h[qq], c[qq] * ec:c[qq] * ec + ec] += 1
        # phase 3 (q and k from LDS): thread t owns chunk position t % (G * cpr)
        # and walks heads t // (G * cpr) + k * hl
        gc = G * cpr
        assert gc <= BLOCK
        hl = BLOCK // gc
        h0 = tid // gc
        pos = tid - h0 * gc
        g = pos // cpr
        c = pos - g * cpr
        row_bytes = D * es
        for s, H in enumerate(heads[:2]):
            if H == 0:
                continue
            yhs = T * D + 8 * ec if head_major else D
            yts = D if head_major else H * D + 8 * ec
            extent = ((H - 1) * yhs + (nvalid - 1) * yts + D) * es
            for m in range(ec // 2):
                col = c * ec + 2 * m
                rot = col < rd
                first = col < half
                pcol = np.where(~rot, col, np.where(first, col + half, col - half))
                j = np.where(~rot, 0, np.where(first, col, col - half))
                assert np.all(pcol * es + 2 * es <= row_bytes)
                assert np.all(j % 2 == 0) and np.all(g * half + j + 2 <= G * half)
            for h in range(H):
                t = np.nonzero((h0 < hl) & (h0 <= h) & ((h - h0) % np.maximum(hl, 1) == 0))[0]
                row = (g[t] * H + h) * row_bytes
                assert np.all(row + c[t] * 16 + 16 <= G * H * cpr * 16)
                live = g[t] < nvalid
                yo = (h * yhs + g[t] * yts) * es + c[t] * 16
                assert np.all(yo[live] + 16 <= extent)
                for q in t[live]:
                    writes[s][t0 + g[q], h, c[q] * ec:c[q] * ec + ec] += 1
    return writes


@pytest.mark.parametrize("T,heads,D,rd,es,G", [
    (22, (16, 16, 16), 72, 72, 2, 4),      # vision qkv bf16 planes
    (9, (16, 16, 16), 72, 72, 4, 2),       # vision qkv fp32 planes
    (11, (16, 16, 0), 72, 72, 4, 4),       # vision_2d fp32 (no v)
    (5, (28, 4, 0), 128, 128, 2, 2),
    (7, (5, 3, 2), 80, 48, 4, 4),          # partial rotary
    (3, (10, 2, 3), 384, 384, 4, 2),
    (37, (3, 1, 2), 8, 4, 2, 16),          # the smallest even half
])
@pytest.mark.parametrize("head_major", [False, True])
@pytest.mark.parametrize("x_pad", [0, 8])
def test_stage_every_output_written_once(T, heads, D, rd, es, G, head_major, x_pad):
    writes = simulate_stage(T, heads, D, rd, es, G, head_major, x_pad=x_pad)
    for s, H in enumerate(heads):
        if H:
            assert np.all(writes[s] == 1), (s, np.unique(writes[s]))


FLAT_BATCH = WAVE * FLAT_STEPS


def flat_in_place_hazard(H, D, rd, v):
    """True if a rotary chunk of the flat kernel reads its partner from a
    batch that was stored before (which breaks in-place calls)."""
    cpr, hc, rc = D // v, (rd // 2) // v, rd // v
    for f in range(H * cpr):
        c = f % cpr
        if c < rc:
            fp = f + hc if c < hc else f - hc
            if fp // FLAT_BATCH < f // FLAT_BATCH:
                return True
    return False


def test_flat_in_place_rule_covers_every_hazard():
    """The host keeps in-place tensors off the flat kernel when a token's
    rows exceed one batch; every geometry with a hazard is such a case."""
    seen = 0
    for D in (8, 16, 24, 40, 48, 72, 80, 96, 128, 144, 200, 256):
        for v in (1, 2, 4, 8):
            for rd in range(2 * v, D + 1, 2 * v):
                if D % (2 * v) or (rd // 2) % v or (D - rd) % (2 * v):
                    continue
                for H in (1, 3, 5, 16, 21, 32, 40):
                    if flat_in_place_hazard(H, D, rd, v):
                        seen += 1
                        assert H * (D // v) > FLAT_BATCH, (H, D, rd, v)
    assert seen > 0
