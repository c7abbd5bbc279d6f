"""CPU model of the pipelined q/k kernel's step stream (qk_pipe_kernel).

Mirrors the kernel's per-lane walk: one token per wavefront, the cursor over
the tensors' row-steps (q, then k, then a copied v; row r of a tensor is head
r), the per-step advance of each lane's head and byte offsets, and the P steps
issued ahead of the one being finished, including the masked steps past the
end of the stream.  For each geometry it checks that every output element is
written exactly once, that every load and store offset of a live row stays
inside the token's buffer and every masked one is past it, that each row is
loaded before it is stored (a row is stored only over itself, so in place is
safe), that the steps finished are
exactly the steps issued, and that every cos/sin read of the prologue stays
inside the wavefront's LDS slice (2 * half binary32 values: cos, then sin).
"""
import numpy as np
import pytest

from tests.test_launch_geometry import OUT_OF_RANGE, WAVE, pick_vec


def host_hc(D, rd, es):
    """The launcher's layout choice: rotary chunks per half (HC > 0, the
    contiguous-halves layout) for bf16 rows of 8 or 16 lanes whose rotary
    columns fit in the first half of the row, else 0."""
    v = pick_vec(es, D, rd)
    lpr, lrot = D // (2 * v), rd // 2 // v
    if es == 2 and lpr in (8, 16) and rd < D and 2 * lrot <= lpr and lrot in (2, 4, 8):
        return 0 if (lrot == 8 and lpr != 16) else lrot
    return 0


def simulate_pipe(T, heads, D, rd, es, P, head_major=False):
    v = pick_vec(es, D, rd)
    assert v * es == 16, "the pipelined kernel takes 16-byte chunks"
    half = rd // 2
    lpr = D // (2 * v)
    rpw = WAVE // lpr
    lrot = half // v
    CB = v * es
    hc = host_hc(D, rd, es)
    lanes = np.arange(WAVE)
    grp = lanes // lpr
    l = lanes - grp * lpr
    lane_on = grp < rpw
    if hc:
        # one chunk in each half of the row; the rotary chunks are the first
        # 2 * hc of the row, x1 on lanes l < hc, x2 on the next hc lanes
        col_a, col_b = l * v, (lpr + l) * v
        rot = l < 2 * hc
        x2 = l >= hc
        cj = np.where(rot, np.where(x2, l - hc, l) * v, 0)
        partner = np.where(x2, lanes - hc, lanes + hc)
        # the partner holds the split-half column of the lane's rotary chunk,
        # in the same row group and the same 16-lane DPP row
        r = np.nonzero(rot)[0]
        assert np.all(col_a[partner[r]] == np.where(x2[r], col_a[r] - half, col_a[r] + half))
        assert np.all(partner[r] // lpr == grp[r]) and np.all(partner[r] // 16 == lanes[r] // 16)
        # each store instruction writes whole 128-byte lines of every row
        for col in (col_a, col_b):
            starts = sorted(set((col[:lpr] * es).tolist()))
            assert starts == list(range(starts[0], starts[0] + lpr * CB, CB))
            assert (starts[0] % 128) == 0 and (lpr * CB) % 128 == 0
    else:
        rot = l < lrot
        col_a = np.where(rot, l * v, rd + (l - lrot) * v)
        col_b = np.where(rot, half + l * v, rd + (lpr - lrot + (l - lrot)) * v)
        cj = np.where(rot, col_a, 0)
    assert np.all(col_a + v <= D) and np.all(col_b + v <= D)
    # every column of the row is owned by exactly one lane's chunk
    owned = np.zeros(D, dtype=int)
    for lane in range(lpr):
        owned[col_a[lane]:col_a[lane] + v] += 1
        owned[col_b[lane]:col_b[lane] + v] += 1
    assert np.all(owned == 1)
    ca, cb = col_a * es, col_b * es
    # Output head stride: token-major rows, or per-head planes of T rows.
    yhs = [T * D + 4 * v if head_major else D for _ in heads]
    writes = [np.zeros((T, H, D), dtype=np.int32) for H in heads]
    nsteps = [-(-H // rpw) for H in heads]
    N = sum(nsteps)
    # The LDS slice of one wavefront: cos at [0, half), sin at [half, 2 half).
    # Each rotary lane reads its V columns at cj of both tables.
    assert np.all(cj + v <= half) or half == 0
    if N == 0:
        return writes
    # Buffer extents the kernel gives each tensor's descriptors (bytes).
    x_extent = [H * D * es for H in heads]
    y_extent = [((H - 1) * yhs[s] + D) * es if H > 0 else 0 for s, H in enumerate(heads)]
    assert max(x_extent + y_extent) < OUT_OF_RANGE
    for t in range(T):
        cur = {}

        def enter(frm):
            s = frm
            while s < len(heads) and nsteps[s] == 0:
                s += 1
            cur["slot"] = s
            if s < len(heads):
                cur.update(left=nsteps[s], H=heads[s], h=grp.copy(),
                           xo=grp * D * es, yo=grp * yhs[s] * es)

        enter(0)
        issued = []          # per issue: (slot, ok lanes, head per lane, output offset)
        loaded = {}          # (slot, head) -> issue index of its load
        n_issue = -(-N // (P + 1)) * (P + 1) + P
        for i in range(n_issue):
            s = cur["slot"]
            have = s < len(heads)
            ok = have & lane_on & (cur["h"] < cur["H"]) if have else np.zeros(WAVE, bool)
            xoff = np.where(ok, cur["xo"], OUT_OF_RANGE) if have else np.full(WAVE, OUT_OF_RANGE)
            you = np.where(ok, cur["yo"], OUT_OF_RANGE) if have else np.full(WAVE, OUT_OF_RANGE)
            if have:
                for c in (ca, cb):
                    assert np.all(xoff[ok] + c[ok] + CB <= x_extent[s])
                    assert np.all(you[ok] + c[ok] + CB <= y_extent[s])
                    # masked lanes are past any extent (hardware drops them)
                    assert np.all(xoff[~ok] + c[~ok] >= x_extent[s])
                for lane in np.nonzero(ok)[0]:
                    loaded.setdefault((s, int(cur["h"][lane])), i)
                issued.append((s, ok, cur["h"].copy(), you))
                cur["xo"] = cur["xo"] + rpw * D * es
                cur["yo"] = cur["yo"] + rpw * yhs[s] * es
                cur["h"] = cur["h"] + rpw
                cur["left"] -= 1
                if cur["left"] == 0:
                    enter(s + 1)
            else:
                issued.append(None)
        # finish order: step j right after the issue of step j + P
        finished = 0
        for j in range(-(-N // (P + 1)) * (P + 1)):
            rec = issued[j]
            if j >= N:
                assert rec is None
                continue
            finished += 1
            s, ok, h, you = rec
            for lane in np.nonzero(ok)[0]:
                hh = int(h[lane])
                assert loaded[(s, hh)] <= j + P
                assert you[lane] == hh * yhs[s] * es
                for c in (col_a[lane], col_b[lane]):
                    writes[s][t, hh, c:c + v] += 1
        assert finished == N
    return writes


CASES = [
    # T, heads, D, rd, es, P
    (5, (32, 4), 128, 128, 2, 2),       # the headline's shape
    (4, (24, 4), 256, 64, 2, 2),        # partial rotary, 16 lanes per row (contiguous halves)
    (4, (24, 4), 256, 128, 2, 2),       # rotary over half the row (contiguous halves, hc 8)
    (4, (8, 2), 256, 32, 2, 2),         # hc 2
    (3, (6, 2), 128, 64, 2, 2),         # 8 lanes per row, hc 4
    (3, (6, 2), 128, 96, 2, 2),         # rotary over more than half the row (split halves)
    (3, (28, 4), 128, 128, 2, 2),       # chunked video's shape, half steps
    (3, (5, 3), 64, 32, 2, 2),          # 16 rows per step, nothing whole
    (3, (5, 3), 64, 64, 2, 2),
    (2, (7, 0), 128, 128, 4, 2),        # no k, binary32
    (2, (0, 6), 64, 64, 4, 2),          # no q
    (2, (3, 2), 512, 512, 2, 2),        # 32 lanes per row, 2 rows per step
    (3, (1, 1), 16, 16, 2, 2),          # one lane per row, 64 rows per step
    (2, (16, 16), 32, 32, 4, 2),
    (2, (64, 8), 128, 128, 2, 2),       # more steps than the unroll
]


def test_host_layout_choice():
    assert host_hc(256, 64, 2) == 4       # the Qwen3.5 shape
    assert host_hc(128, 128, 2) == 0      # full rotary: split halves already write whole lines
    assert host_hc(128, 96, 2) == 0
    assert host_hc(256, 64, 4) == 0       # binary32 rows keep the split-half layout


@pytest.mark.parametrize("T,heads,D,rd,es,P", CASES)
def test_pipe_every_output_written_once(T, heads, D, rd, es, P):
    writes = simulate_pipe(T, heads, D, rd, es, P)
    for s, w in enumerate(writes):
        assert np.all(w == 1), (s, np.argwhere(w != 1)[:5])


@pytest.mark.parametrize("rd", [64, 32])
def test_pipe_packed_qkv_token_major_and_planes(rd):
    for head_major in (False, True):
        writes = simulate_pipe(3, (4, 4, 4), 64, rd, 2, 2, head_major=head_major)
        assert all(np.all(w == 1) for w in writes)
