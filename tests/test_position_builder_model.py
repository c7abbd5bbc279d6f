"""CPU model of the GPU position builder's three passes (chunk summaries, the
one-block carry walk, the per-chunk apply), mirroring the kernels' per-thread
runs and block scans, checked against the position oracle on random batches.

The model takes the block size and tokens per thread as parameters, so small
values put chunk and run boundaries everywhere (inside segments, on segment
starts, inside padding).  It also checks that every index the kernels form
stays inside its buffer.
"""
import numpy as np
import pytest

from oracle import positions_oracle as P
import workloads as W

BAD_TYPE, NO_GRID, LENGTH = 1, 2, 4


def _read_run(types, mask, b, L, l0, per):
    ty = []
    nv = nt = ni = nvd = 0
    ft = lt = lsF = lsT = -1
    flags = 0
    for k in range(per):
        l = l0 + k
        t = -1
        if l < L:
            if mask is None or mask[b, l] != 0:
                t = int(types[b, l])
                if t < 0 or t > 2:
                    flags |= BAD_TYPE
                    t = 0
        ty.append(t)
        if t < 0:
            continue
        if ft < 0:
            ft = t
        elif t != lt:
            ni += t == 1
            nvd += t == 2
            lsF, lsT = nv, t
        lt = t
        nv += 1
        nt += t == 0
    return dict(ty=ty, nv=nv, nt=nt, ft=ft, lt=lt, ni=ni, nvd=nvd, lsF=lsF, lsT=lsT, flags=flags)


def _excl_sum(vals):
    out, acc = [], 0
    for v in vals:
        out.append(acc)
        acc += v
    return out, acc


def _excl_max(vals, lo):
    out, acc = [], lo
    for v in vals:
        out.append(acc)
        acc = max(acc, v)
    return out, acc


def _prev_types(runs):
    enc = [(i << 2 | r["lt"]) if r["lt"] >= 0 else -1 for i, r in enumerate(runs)]
    ex, _ = _excl_max(enc, -1)
    return [(m & 3) if m >= 0 else -1 for m in ex]


class Tables:
    def __init__(self, images, videos, merge):
        self.images, self.videos, self.merge = images, videos, merge
        self.adv_i = np.zeros(len(images) + 1, dtype=np.int64)
        for k, (t, h, w) in enumerate(images):
            self.adv_i[k + 1] = self.adv_i[k] + max(h, w) // merge
        self.cum_t = np.zeros(len(videos) + 1, dtype=np.int64)
        self.adv_v = np.zeros(len(videos) + 1, dtype=np.int64)
        for v, (t, h, w) in enumerate(videos):
            t = max(t, 0)
            self.cum_t[v + 1] = self.cum_t[v] + t
            self.adv_v[v + 1] = self.adv_v[v] + t * (max(h, w) // merge)

    def video_of_slice(self, k):
        lo, hi = 0, len(self.videos) - 1
        while lo < hi:
            mid = (lo + hi + 1) >> 1
            if self.cum_t[mid] <= k:
                lo = mid
            else:
                hi = mid - 1
        return lo

    def grid(self, ty, k):
        m = self.merge
        if ty == 1:
            if k < 0 or k >= len(self.images):
                return None
            t, h, w = self.images[k]
        else:
            if k < 0 or k >= self.cum_t[-1]:
                return None
            v = self.video_of_slice(k)
            assert 0 <= v < len(self.videos)
            t, (h, w) = 1, self.videos[v][1:]
        g = dict(t=t, hm=h // m, wm=w // m, adv=max(h, w) // m)
        g["slots"] = t * g["hm"] * g["wm"]
        g["ok"] = t > 0 and g["hm"] > 0 and g["wm"] > 0
        return g

    def img_adv(self, k):
        return int(self.adv_i[min(k, len(self.images))])

    def vid_adv(self, k):
        n = int(self.cum_t[-1])
        k = min(k, n)
        if k <= 0:
            return 0
        if k == n:
            return int(self.adv_v[-1])
        v = self.video_of_slice(k)
        h, w = self.videos[v][1:]
        return int(self.adv_v[v] + (k - self.cum_t[v]) * (max(h, w) // self.merge))


def carry_parallel(summaries, B, C, threads):
    """The carry pass as the kernel runs it: contiguous chunk ranges per
    thread, block scans between rounds, per-sample values as batch-wide
    prefixes minus the sample's first chunk.  Returns the carries and the
    per-sample (valid, end record)."""
    n = B * C
    per = -(-n // threads) if n else 0
    rng = [(min(n, t * per), min(n, t * per + per)) for t in range(threads)]
    S = [list(x) for x in summaries]
    # pass 1
    t_nv = [sum(S[c][0] for c in range(a, b)) for a, b in rng]
    t_nt = [sum(S[c][1] for c in range(a, b)) for a, b in rng]
    t_lt = []
    for a, b in rng:
        v = -1
        for c in range(a, b):
            if S[c][5] >= 0:
                v = c << 2 | S[c][5]
        t_lt.append(v)
    gF_ex, _ = _excl_sum(t_nv)
    gA_ex, _ = _excl_sum(t_nt)
    lt_ex, _ = _excl_max(t_lt, -1)
    # pass 2
    t_ni, t_nvd, t_st = [], [], []
    for t, (a, b) in enumerate(rng):
        gF, gA, lt = gF_ex[t], gA_ex[t], lt_ex[t]
        ni_s = nvd_s = 0
        st = -1
        for c in range(a, b):
            first = (c // C) * C
            nv, nt, ni, nvd, ft, lts, lsF, lsT, _ = S[c]
            prevT = (lt & 3) if lt >= 0 and (lt >> 2) >= first else -1
            fs = ft >= 0 and ft != prevT
            ni_all, nvd_all = ni + (fs and ft == 1), nvd + (fs and ft == 2)
            cand = ((gF + lsF) << 2 | lsT) if lsF >= 0 else ((gF << 2 | ft) if fs else -1)
            S[c] = [gF, gA, prevT, ni_all, nvd_all, cand, None, None, nv]
            ni_s += ni_all
            nvd_s += nvd_all
            st = max(st, cand)
            gF += nv
            gA += nt
            if lts >= 0:
                lt = c << 2 | lts
        t_ni.append(ni_s)
        t_nvd.append(nvd_s)
        t_st.append(st)
    img_ex, img_tot = _excl_sum(t_ni)
    vid_ex, vid_tot = _excl_sum(t_nvd)
    st_ex, _ = _excl_max(t_st, -1)
    for t, (a, b) in enumerate(rng):
        img, vid = img_ex[t], vid_ex[t]
        for c in range(a, b):
            S[c][6], S[c][7] = img, vid
            img += S[c][3]
            vid += S[c][4]
    carries = [None] * n
    valid, ends = [0] * B, [None] * B
    for t, (a, b) in enumerate(rng):
        st = st_ex[t]
        for c in range(a, b):
            bb, j = divmod(c, C)
            s, s0 = S[c], S[bb * C]
            F0 = s0[0]
            S_in = (st >> 2) - F0 if st >= 0 and (st >> 2) >= F0 else -1
            segT_in = (st & 3) if S_in >= 0 else -1
            carries[c] = [s[0] - F0, s[1] - s0[1], s[2], s[6], s[7], s0[6], s0[7], S_in, segT_in]
            st = max(st, s[5])
            if j == C - 1:
                v = s[0] + s[8] - F0
                S_end = (st >> 2) - F0 if st >= 0 and (st >> 2) >= F0 else -1
                segT_end = (st & 3) if S_end >= 0 else -1
                valid[bb] = v
                ends[bb] = (v - S_end, segT_end,
                            (s[6] + s[3] - 1) if segT_end == 1 else (s[7] + s[4] - 1))
    return carries, valid, ends, img_tot, vid_tot


def model(types, mask, images, videos, merge, PT, PER, carry_threads=None):
    B, L = types.shape
    CH = PT * PER
    C = -(-L // CH)
    tab = Tables(images, videos, merge)
    # pass 1
    summaries = []
    for b in range(B):
        for j in range(C):
            runs = [_read_run(types, mask, b, L, j * CH + i * PER, PER) for i in range(PT)]
            pts = _prev_types(runs)
            ni_l, nvd_l, cand = [], [], []
            nv_ex, nv_tot = _excl_sum([r["nv"] for r in runs])
            for r, pt, nx in zip(runs, pts, nv_ex):
                fs = r["ft"] >= 0 and pt >= 0 and r["ft"] != pt
                ni_l.append(r["ni"] + (fs and r["ft"] == 1))
                nvd_l.append(r["nvd"] + (fs and r["ft"] == 2))
                if r["lsF"] >= 0:
                    cand.append((nx + r["lsF"]) << 2 | r["lsT"])
                elif fs:
                    cand.append(nx << 2 | r["ft"])
                else:
                    cand.append(-1)
            last = max(cand)
            firsts = [r["ft"] for r in runs if r["ft"] >= 0]
            lasts = [r["lt"] for r in runs if r["lt"] >= 0]
            flags = 0
            for r in runs:
                flags |= r["flags"]
            summaries.append([nv_tot, sum(r["nt"] for r in runs), sum(ni_l), sum(nvd_l),
                              firsts[0] if firsts else -1, lasts[-1] if lasts else -1,
                              (last >> 2) if last >= 0 else -1, (last & 3) if last >= 0 else -1,
                              flags])
    # pass 2
    status = 0
    img = vid = 0
    carries, valid = [], [0] * B
    seq_ends = [None] * B
    delta = [0] * B
    F = A = 0
    prevT = S = segT = -1
    img0 = vid0 = 0
    for c, s in enumerate(summaries):
        b, j = divmod(c, C)
        if j == 0:
            F = A = 0
            prevT = S = segT = -1
            img0, vid0 = img, vid
        carries.append([F, A, prevT, img, vid, img0, vid0, S, segT])
        status |= s[8]
        fs = s[4] >= 0 and s[4] != prevT
        img += s[2] + (fs and s[4] == 1)
        vid += s[3] + (fs and s[4] == 2)
        if s[6] >= 0:
            S, segT = F + s[6], s[7]
        elif fs:
            S, segT = F, s[4]
        F += s[0]
        A += s[1]
        if s[5] >= 0:
            prevT = s[5]
        if j == C - 1:
            valid[b] = F
            delta[b] = 0 if F == 0 else None
            seq_ends[b] = (F - S, segT, (img if segT == 1 else vid) - 1)
            if segT in (1, 2):
                g = tab.grid(segT, (img if segT == 1 else vid) - 1)
                if g is not None and g["ok"] and F - S != g["slots"]:
                    status |= LENGTH
    if img > len(images) or vid > tab.cum_t[-1]:
        status |= NO_GRID
    if carry_threads is not None:
        # the kernel's parallel carry must reproduce the sequential walk
        pc, pvalid, pends, pimg, pvid = carry_parallel(summaries, B, C, carry_threads)
        assert pc == carries, (pc, carries)
        assert pvalid == valid and (pimg, pvid) == (img, vid)
        assert pends == seq_ends, (pends, seq_ends)
    # pass 3
    pos = np.zeros((3, B * L), dtype=np.int64)
    written = np.zeros(B * L, dtype=np.int64)
    for c in range(B * C):
        b, j = divmod(c, C)
        F_in, A_in, prevT_in, img_in, vid_in, img0, vid0, S_in, segT_in = carries[c]
        runs = [_read_run(types, mask, b, L, j * CH + i * PER, PER) for i in range(PT)]
        pts = _prev_types(runs)
        prevs = [pt if pt >= 0 else prevT_in for pt in pts]
        fss = [r["ft"] >= 0 and r["ft"] != pv for r, pv in zip(runs, prevs)]
        F_ex, _ = _excl_sum([r["nv"] for r in runs])
        A_ex, _ = _excl_sum([r["nt"] for r in runs])
        I_ex, _ = _excl_sum([r["ni"] + (fs and r["ft"] == 1) for r, fs in zip(runs, fss)])
        V_ex, _ = _excl_sum([r["nvd"] + (fs and r["ft"] == 2) for r, fs in zip(runs, fss)])
        cands = []
        for r, fs, fx in zip(runs, fss, F_ex):
            f_run = F_in + fx
            if r["lsF"] >= 0:
                cands.append((f_run + r["lsF"]) << 2 | r["lsT"])
            elif fs:
                cands.append(f_run << 2 | r["ft"])
            else:
                cands.append(-1)
        before, _ = _excl_max(cands, -1)
        bmax = None
        for i, r in enumerate(runs):
            F, A = F_in + F_ex[i], A_in + A_ex[i]
            img, vid = img_in + I_ex[i], vid_in + V_ex[i]
            prevT = prevs[i]
            if before[i] >= 0:
                S, segT = before[i] >> 2, before[i] & 3
            else:
                S, segT = S_in, segT_in
            g = tab.grid(segT, (img if segT == 1 else vid) - 1) if segT in (1, 2) else None
            a0 = tab.img_adv(img0) + tab.vid_adv(vid0)
            badv = tab.img_adv(img) + tab.vid_adv(vid) - a0
            l0 = j * CH + i * PER
            for k in range(PER):
                l = l0 + k
                if l >= L:
                    break
                ty = r["ty"][k]
                p = (0, 0, 0)
                if ty >= 0:
                    if ty != prevT:
                        if segT in (1, 2) and g is not None and g["ok"] and F - S != g["slots"]:
                            status |= LENGTH
                        S, segT = F, ty
                        img += ty == 1
                        vid += ty == 2
                        if ty != 0:
                            g = tab.grid(ty, (img if ty == 1 else vid) - 1)
                            badv = tab.img_adv(img) + tab.vid_adv(vid) - a0
                    prevT = ty
                    if ty == 0 or g is None or not g["ok"]:
                        if ty != 0:
                            status |= NO_GRID
                        p = (A + badv,) * 3
                    else:
                        ii = F - S
                        if ii >= g["slots"]:
                            status |= LENGTH
                            ii = g["slots"] - 1
                        base = A + badv - g["adv"]
                        plane = g["hm"] * g["wm"]
                        tt, rem = divmod(ii, plane)
                        row, col = divmod(rem, g["wm"])
                        p = (base + tt, base + row, base + col)
                    A += ty == 0
                    F += 1
                    bmax = max(p) if bmax is None else max(bmax, max(p))
                o = b * L + l
                assert 0 <= o < B * L
                pos[:, o] = p
                written[o] += 1
        if bmax is not None:
            cur = delta[b]
            val = bmax + 1 - valid[b]
            delta[b] = val if cur is None else max(cur, val)
    assert np.all(written == 1)
    return pos.reshape(3, B, L), np.array(delta, dtype=np.int64), status


@pytest.mark.parametrize("PT,PER", [(4, 3), (2, 5), (8, 2), (1, 7), (16, 16)])
@pytest.mark.parametrize("seed", range(6))
def test_model_matches_oracle(PT, PER, seed):
    rng = np.random.default_rng(seed * 31 + PT)
    B, L = int(rng.integers(1, 4)), int(rng.integers(20, 90))
    types, mask, images, videos = W.random_mm_batch(rng, B, L)
    want, wd = P.get_rope_index(types, image_grid_thw=images or None,
                                video_grid_thw=videos or None, attention_mask=mask)
    got, gd, status = model(types, mask, images, videos, 2, PT, PER,
                            carry_threads=[1, 3, 256][seed % 3])
    assert status == 0
    assert np.array_equal(got, want)
    assert np.array_equal(gd, wd)


def test_model_on_the_printed_table():
    types = np.array([[0, 0, 1, 1, 1, 1, 1, 1, 0, 0]])
    for PT, PER in [(1, 1), (2, 2), (3, 1), (4, 3)]:
        pos, d, st = model(types, None, [(1, 4, 6)], [], 2, PT, PER)
        assert pos[0, 0].tolist() == [0, 1, 2, 2, 2, 2, 2, 2, 5, 6]
        assert pos[2, 0].tolist() == [0, 1, 2, 3, 4, 2, 3, 4, 5, 6]
        assert d.tolist() == [-3] and st == 0


def test_model_flags_bad_inputs():
    # no grid for the image run
    _, _, st = model(np.array([[0, 1, 1, 1, 1]]), None, [], [], 2, 2, 2)
    assert st & NO_GRID
    # run shorter than its grid (3 tokens for 4 slots), run longer
    _, _, st = model(np.array([[0, 1, 1, 1, 0]]), None, [(1, 4, 4)], [], 2, 2, 2)
    assert st & LENGTH
    _, _, st = model(np.array([[1, 1, 1, 1, 1]]), None, [(1, 4, 4)], [], 2, 2, 2)
    assert st & LENGTH
    _, _, st = model(np.array([[0, 1, 1, 1]]), None, [(1, 4, 4)], [], 2, 2, 2)   # at the end
    assert st & LENGTH
    _, _, st = model(np.array([[0, 3, 0]]), None, [], [], 2, 2, 2)
    assert st & BAD_TYPE
