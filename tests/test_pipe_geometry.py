"""CPU model of the pipelined q/k kernel's step stream (qk_pipe_kernel).

Mirrors the kernel's per-lane walk: the tile of nt tokens, the cursor over
the tensors' row-steps (q, then k, then a copied v), the incremental head /
token advance, and the P steps issued ahead of the one being finished,
including the masked steps past the end of the stream.  For each geometry it
checks that every output element is written exactly once, that every load
and store offset of a live row stays inside its tile buffer and every masked
one is past it, that each row is loaded before it is stored (in place is
safe), and that every cos/sin read of a rotary lane stays inside the
wavefront's LDS slice.
"""
import numpy as np
import pytest

from tests.test_launch_geometry import OUT_OF_RANGE, WAVE, first_row_split_lanes, pick_vec


def host_tokens(heads, rpw, norm):
    """Tokens per tile the host takes: with RMSNorm the fewest of 1, 2, 4
    whose rows fill whole row-steps of every tensor, else 1."""
    if not norm:
        return 1
    for n in (1, 2, 4):
        if all(H == 0 or (n * H) % rpw == 0 for H in heads):
            return n
    return 1


def simulate_pipe(T, heads, D, rd, es, nt, P, head_major=False, in_place=False):
    v = pick_vec(es, D, rd)
    assert v * es == 16, "the pipelined kernel takes 16-byte chunks"
    half = rd // 2
    lpr = D // (2 * v)
    rpw = WAVE // lpr
    lrot = half // v
    CB = v * es
    lanes = np.arange(WAVE)
    grp = lanes // lpr
    l = lanes - grp * lpr
    lane_on = grp < rpw
    rot = l < lrot
    col_a = np.where(rot, l * v, rd + (l - lrot) * v)
    col_b = np.where(rot, half + l * v, rd + (lpr - lrot + (l - lrot)) * v)
    assert np.all(col_a + v <= D) and np.all(col_b + v <= D)
    ca, cb = col_a * es, col_b * es
    xts = [H * D + (0 if in_place else 8 * v) for H in heads]
    if head_major:
        yts, yhs = [D] * len(heads), [T * D + 4 * v] * len(heads)
    else:
        yts = [H * D + (0 if in_place else 4 * v) for H in heads]
        yhs = [D] * len(heads)
    writes = [np.zeros((T, H, D), dtype=np.int32) for H in heads]
    lds_slice = nt * half
    for w in range(-(-T // nt)):
        t0 = w * nt
        ntok = min(nt, T - t0)
        nsteps = [-(-ntok * H // rpw) if H > 0 else 0 for H in heads]
        N = sum(nsteps)
        assert N > 0
        loaded = {}           # (slot, token, head) -> issue index of its load
        # cursor
        state = {}

        def enter(frm):
            s = frm
            while s < len(heads) and nsteps[s] == 0:
                s += 1
            if s < len(heads):
                H = heads[s]
                tl, h = first_row_split_lanes(grp, H)
                state.update(slot=s, left=nsteps[s], r0=0, tl=tl, h=h, H=H,
                             dq=rpw // H, dr=rpw % H)
            else:
                state["slot"] = s
        enter(0)
        issued = []           # per issue: (slot, ok lanes, tl, h) or None past the end
        n_issue = -(-N // (P + 1)) * (P + 1) + P
        for i in range(n_issue):
            s = state["slot"]
            have = s < len(heads)
            if not have:
                issued.append(None)
                continue
            H = heads[s]
            nrows = ntok * H
            ok = lane_on & (state["r0"] + grp < nrows)
            tl, h = state["tl"].copy(), state["h"].copy()
            x_extent = ((ntok - 1) * xts[s] + H * D) * es
            y_extent = ((ntok - 1) * yts[s] + (H - 1) * yhs[s] + D) * es
            assert x_extent < OUT_OF_RANGE and y_extent < OUT_OF_RANGE
            xo = (tl * xts[s] + h * D) * es
            yo = (tl * yts[s] + h * yhs[s]) * es
            for c in (ca, cb):
                assert np.all(xo[ok] + c[ok] + CB <= x_extent)
                assert np.all(yo[ok] + c[ok] + CB <= y_extent)
            assert np.all(tl[ok] < ntok) and np.all(h[ok] < H)
            for lane in np.nonzero(ok)[0]:
                key = (s, int(tl[lane]), int(h[lane]))
                loaded.setdefault(key, i)
            issued.append((s, ok, tl, h))
            # advance as the kernel does
            state["h"] = state["h"] + state["dr"]
            state["tl"] = state["tl"] + state["dq"]
            wrap = state["h"] >= state["H"]
            state["h"] = np.where(wrap, state["h"] - state["H"], state["h"])
            state["tl"] = np.where(wrap, state["tl"] + 1, state["tl"])
            state["r0"] += rpw
            state["left"] -= 1
            if state["left"] == 0:
                enter(s + 1)
        # finish order: step j after the issue of step j + P
        for j in range(-(-N // (P + 1)) * (P + 1)):
            rec = issued[j]
            if j >= N:
                assert rec is None
                continue
            s, ok, tl, h = rec
            last_issue_before = j + P
            for lane in np.nonzero(ok)[0]:
                t, hh = int(tl[lane]), int(h[lane])
                assert loaded[(s, t, hh)] <= last_issue_before
                for c in (col_a[lane], col_b[lane]):
                    writes[s][t0 + t, hh, c:c + v] += 1
            if s < 2:
                tlr = np.where(ok, tl, 0)
                idx = tlr * half + col_a
                assert np.all(idx[rot] + v <= lds_slice)
    return writes


CASES = [
    # T, heads, D, rd, es, norm, P
    (37, (32, 4), 128, 128, 2, True, 2),       # the headline's shape, ragged last tile
    (37, (32, 4), 128, 128, 2, True, 3),
    (29, (24, 4), 256, 64, 2, True, 2),        # partial rotary, 16 lanes per row
    (29, (24, 4), 256, 64, 2, True, 3),
    (23, (28, 4), 128, 128, 2, False, 2),      # chunked video's shape, half steps
    (23, (28, 4), 128, 128, 2, False, 3),
    (19, (5, 3), 64, 32, 2, True, 2),          # 16 rows per step, nothing whole
    (19, (5, 3), 64, 64, 2, False, 3),
    (17, (7, 0), 128, 128, 4, True, 2),        # no k, binary32
    (17, (0, 6), 64, 64, 4, False, 2),         # no q
    (11, (3, 2), 512, 512, 2, True, 3),        # 32 lanes per row, 2 rows per step
    (70, (1, 1), 16, 16, 2, True, 2),          # one lane per row, 64 rows per step
    (13, (16, 16), 32, 32, 4, False, 3),
]


@pytest.mark.parametrize("T,heads,D,rd,es,norm,P", CASES)
def test_pipe_every_output_written_once(T, heads, D, rd, es, norm, P):
    v = pick_vec(es, D, rd)
    nt = host_tokens(heads, 64 // (D // (2 * v)), norm)
    for nt_try in sorted({nt, 1, 2}):
        writes = simulate_pipe(T, heads, D, rd, es, nt_try, P)
        for s, w in enumerate(writes):
            assert np.all(w == 1), (s, nt_try, np.argwhere(w != 1)[:5])


@pytest.mark.parametrize("P", [2, 3])
def test_pipe_packed_qkv_planes_and_in_place(P):
    for head_major in (False, True):
        writes = simulate_pipe(21, (4, 4, 4), 64, 64, 2, 1, P, head_major=head_major)
        assert all(np.all(w == 1) for w in writes)
    writes = simulate_pipe(21, (6, 2), 128, 128, 2, 2, P, in_place=True)
    assert all(np.all(w == 1) for w in writes)


def test_host_tile_tokens():
    assert host_tokens((32, 4), 8, True) == 2      # the headline: 4 k rows fill half a step
    assert host_tokens((24, 4), 4, True) == 1      # qwen35: whole steps with one token
    assert host_tokens((28, 4), 8, False) == 1
