"""CPU model of the group kernel's indexing (planes_kernel, mrope_planes.hip).

Mirrors the host's choice of tokens per block (the fewest that make a plane's
run of rows a whole number of 128-byte lines, refused when the group's
chunks exceed the block) and the kernel's per-thread walk: chunk f of a
tensor's group on thread f mod 512, decomposed with the kernel's binary32
reciprocals into (plane, token, chunk), and the split-half partner read as
one 16-byte chunk or as two 8-byte pieces.  For each geometry it checks that
every output chunk is written exactly once, that every load stays inside its
row, that the partner pieces hold exactly the partner elements (including
the chunk that straddles the half), and that each sincos slot is one
(token, column) of the group.
"""
import numpy as np
import pytest

THREADS = 512
TASKS = 3
MAX_COS_SIN = THREADS


def host_group(es, D, H):
    """Tokens per block the launcher takes (0: another kernel serves it)."""
    V = 16 // es
    half = D // 2
    if (D * es) % 16 or (2 * half) % V:
        return 0
    G = 1
    while G < 16 and (G * D * es) % 128:
        G *= 2
    cpr = D // V
    if G * half > MAX_COS_SIN or H * G * cpr > THREADS * TASKS:
        return 0
    return G


def simulate(es, D, H, T, n_tensors=3):
    V = 16 // es
    cpr, half = D // V, D // 2
    G = host_group(es, D, H)
    assert G > 0
    run = G * cpr
    hc = half // V
    split = half % V != 0
    assert not split or half % V == V // 2
    inv_run = np.float32(1.0) / np.float32(run)
    inv_cpr = np.float32(1.0) / np.float32(cpr)
    written = np.zeros((n_tensors, H, T, cpr), np.int32)
    for b in range((T + G - 1) // G):
        t0 = b * G
        nvalid = min(G, T - t0)
        # sincos slots: thread tid < G * half forms (token tid // half, column tid % half)
        tid = np.arange(G * half)
        assert np.array_equal(np.unique(tid // half * half + tid % half), tid)
        for s in range(n_tensors):
            for u in range(TASKS):
                f = np.arange(THREADS) + u * THREADS
                h = (f.astype(np.float32) * inv_run).astype(np.int64)
                h -= h * run > f
                h += (h + 1) * run <= f
                r = f - h * run
                g = (r.astype(np.float32) * inv_cpr).astype(np.int64)
                g -= g * cpr > r
                g += (g + 1) * cpr <= r
                c = r - g * cpr
                ok = (f < H * run) & (g < nvalid)
                assert np.all((h[ok] < H) & (c[ok] >= 0) & (c[ok] < cpr) & (g[ok] >= 0))
                if s < 2:
                    e = c[:, None] * V + np.arange(V)[None, :]
                    want = np.where(e < half, e + half, e - half)
                    if split:
                        a = np.where(c < hc, c * V + half, np.where(c == hc, D - V // 2, c * V - half))
                        bb = np.where(c == hc, 0, a + V // 2)
                        assert np.all((a[ok] >= 0) & (a[ok] + V // 2 <= D))
                        assert np.all((bb[ok] >= 0) & (bb[ok] + V // 2 <= D))
                        got = np.where(np.arange(V)[None, :] < V // 2,
                                       a[:, None] + np.arange(V)[None, :],
                                       bb[:, None] + np.arange(V)[None, :] - V // 2)
                    else:
                        cp = np.where(c < hc, c + hc, c - hc)
                        assert np.all((cp[ok] >= 0) & (cp[ok] < cpr))
                        got = cp[:, None] * V + np.arange(V)[None, :]
                    assert np.array_equal(got[ok], want[ok])
                np.add.at(written, (s, h[ok], t0 + g[ok], c[ok]), 1)
    assert written.min() == 1 and written.max() == 1
    return G


@pytest.mark.parametrize("es,D,H,T,G", [
    (2, 72, 16, 32768, 8),    # the vision tower, bf16 (straddling chunk)
    (4, 72, 16, 32768, 4),    # the vision tower, fp32
    (2, 72, 16, 2051, 8),     # ragged last group
    (4, 72, 21, 4099, 4),     # the block's capacity nearly full
    (2, 72, 21, 2099, 8),
    (4, 36, 16, 2050, 8),     # fp32 with a straddling chunk
    (2, 128, 8, 2050, 1),
    (2, 256, 24, 2053, 1),
    (2, 16, 1, 2048, 4),
])
def test_group_kernel_indexing(es, D, H, T, G):
    assert simulate(es, D, H, T) == G


@pytest.mark.parametrize("es,D,H", [(2, 72, 96), (4, 72, 96), (2, 72, 22), (4, 72, 22)])
def test_groups_too_large_for_the_block_are_refused(es, D, H):
    assert host_group(es, D, H) == 0
