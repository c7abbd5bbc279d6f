"""Host side of the C ABI, on the CPU: the library loads, exports every
declared entry point, its host tables match the oracle bit for bit, and bad
arguments are rejected before anything reaches the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import mrope_oracle as O
import workloads as W
from vlm_multimodal_rotary_amd import _lib
import vlm_multimodal_rotary_amd as M

HEADER = os.path.join(os.path.dirname(__file__), "..", "include", "mrope.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text,
                                 flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_functions()
    assert declared == sorted(_lib.SIGNATURES), declared
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("dim,theta", [(16, 1e4), (128, 1e6), (64, 1e7), (36, 1e4), (8, 1e4),
                                       (6, 100.0), (256, 5e5), (512, 1e4), (2, 3.0)])
def test_inv_freq_matches_oracle_bitwise(dim, theta):
    assert np.array_equal(M.mrope_inv_freq(dim, theta).view(np.uint32),
                          O.inv_freq(dim, theta).view(np.uint32))


def _valid_interleaved_sections(half):
    out = []
    for sh in range(0, half + 1):
        for sw in range(0, half + 1 - sh):
            st = half - sh - sw
            try:
                O.axis_table(half, (st, sh, sw), "interleaved")
            except AssertionError:
                continue
            out.append((st, sh, sw))
    return out


def test_axis_table_matches_oracle_for_every_valid_interleaved_section():
    for half in (2, 5, 8, 10, 32, 36, 64):
        secs = _valid_interleaved_sections(half)
        assert secs
        for sec in secs:
            assert np.array_equal(M.mrope_axis_table(half, sec, "interleaved"),
                                  O.axis_table(half, sec, "interleaved")), (half, sec)


def test_axis_table_rejects_what_the_oracle_rejects():
    for half in (8, 10, 32):
        for sh in range(0, half + 1):
            for sw in range(0, half + 1 - sh):
                sec = (half - sh - sw, sh, sw)
                try:
                    O.axis_table(half, sec, "interleaved")
                    oracle_ok = True
                except AssertionError:
                    oracle_ok = False
                if oracle_ok:
                    continue
                with pytest.raises(_lib.MropeError) as e:
                    M.mrope_axis_table(half, sec, "interleaved")
                assert e.value.code == _lib.MROPE_EINVAL


def test_axis_table_chunked_and_vision():
    for half, sec in [(64, (16, 24, 24)), (10, (4, 3, 3)), (8, (8,)), (8, (3, 5))]:
        assert np.array_equal(M.mrope_axis_table(half, sec, "chunked"),
                              O.axis_table(half, sec, "chunked"))
    assert np.array_equal(M.mrope_axis_table(36, None, "vision_2d"),
                          O.axis_table(36, None, "vision_2d"))
    with pytest.raises(_lib.MropeError):
        M.mrope_axis_table(8, (4, 3, 3), "chunked")          # sum != half
    with pytest.raises(_lib.MropeError):
        M.mrope_axis_table(7, None, "vision_2d")             # odd half


# -- argument checks of the device entry points (rejected before any HIP call) --

FAKE = 0x10000000  # never dereferenced: every call below fails its checks first


def _no_gpu():
    """The fake-pointer calls below must never reach a launch; on a machine
    with a visible GPU they are skipped outright."""
    try:
        import torch
        return not torch.cuda.is_available()
    except ImportError:
        return True


fake_ptr_test = pytest.mark.skipif(not _no_gpu(), reason="fake device pointers: CPU-only check")


def _fused(**kw):
    args = dict(q=FAKE, q_ts=32 * 128, hq=32, k=FAKE + 0x4000000, k_ts=4 * 128, hk=4, T=16,
                D=128, rd=128, pos=FAKE + 0x8000000, pos_stride=16, n_axes=3,
                section=(24, 20, 20), layout=_lib.LAYOUT_INTERLEAVED, theta=1e6,
                wq=FAKE + 0xC000000, wk=FAKE + 0xC001000, eps=1e-6, dtype=_lib.DTYPE_BF16,
                prec=_lib.PRECISION_EXACT, qo=FAKE + 0x20000000, qo_ts=32 * 128,
                ko=FAKE + 0x24000000, ko_ts=4 * 128)
    args.update(kw)
    a = args
    sec = list(a["section"]) if a["section"] is not None else []
    return _lib.load().rmsnorm_mrope_qk(
        a["q"], a["q_ts"], a["hq"], a["k"], a["k_ts"], a["hk"], a["T"], a["D"], a["rd"],
        a["pos"], a["pos_stride"], a["n_axes"], _lib.int_array(sec), len(sec), a["layout"],
        a["theta"], a["wq"], a["wk"], a["eps"], a["dtype"], a["prec"], a["qo"], a["qo_ts"],
        a["ko"], a["ko_ts"], None)


@fake_ptr_test
@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _lib.MROPE_EUNSUPPORTED),
    (dict(prec=3), _lib.MROPE_EINVAL),
    (dict(prec=-1), _lib.MROPE_EINVAL),
    (dict(rd=127), _lib.MROPE_EINVAL),
    (dict(rd=256), _lib.MROPE_EINVAL),               # > D
    (dict(D=127, rd=126), _lib.MROPE_EINVAL),        # odd D
    (dict(section=(24, 20, 21)), _lib.MROPE_EINVAL), # sum != half
    (dict(section=(4, 40, 20)), _lib.MROPE_EINVAL),  # rule cannot place 40 H columns
    (dict(n_axes=2), _lib.MROPE_EINVAL),
    (dict(layout=9), _lib.MROPE_EINVAL),
    (dict(q=0), _lib.MROPE_EINVAL),
    (dict(pos=0), _lib.MROPE_EINVAL),
    (dict(wk=0), _lib.MROPE_EINVAL),                 # one weight only
    (dict(q_ts=100), _lib.MROPE_EINVAL),             # token stride < heads*D
    (dict(theta=0.0), _lib.MROPE_EINVAL),
    (dict(theta=float("nan")), _lib.MROPE_EINVAL),
    (dict(eps=-1.0), _lib.MROPE_EINVAL),
    (dict(T=-1), _lib.MROPE_EINVAL),
    (dict(hq=-2), _lib.MROPE_EINVAL),
    (dict(qo=FAKE + 64), _lib.MROPE_EINVAL),         # q_out partially overlaps q
    (dict(ko=FAKE + 16), _lib.MROPE_EINVAL),         # k_out overlaps q
    (dict(ko=FAKE + 0x20000000 + 256), _lib.MROPE_EINVAL),   # k_out overlaps q_out
    (dict(qo=FAKE + 0x8000000), _lib.MROPE_EINVAL),  # q_out overlaps positions
    (dict(q=FAKE + 1, qo=FAKE + 0x20000001), _lib.MROPE_EUNSUPPORTED),  # odd address, bf16
    (dict(rd=1024, D=1024), _lib.MROPE_EUNSUPPORTED),
    # vision layout with an odd number of frequency columns (half = 35)
    (dict(layout=_lib.LAYOUT_VISION_2D, n_axes=2, section=None, D=70, rd=70, q_ts=32 * 70,
          k_ts=4 * 70, qo_ts=32 * 70, ko_ts=4 * 70), _lib.MROPE_EINVAL),
])
def test_fused_rejects_bad_arguments(kw, code):
    rc = _fused(**kw)
    assert rc == code, (rc, _lib.load().mrope_last_error())
    assert _lib.load().mrope_last_error()


@fake_ptr_test
def test_fused_T_zero_is_a_noop():
    assert _fused(T=0) == _lib.MROPE_OK
    assert _fused(T=0, q=0, k=0, qo=0, ko=0, pos=0) == _lib.MROPE_OK


@fake_ptr_test
def test_last_kernel_names_no_launch_without_one():
    # argument checks and T = 0 launch nothing, so the name stays empty
    assert _fused(T=0) == _lib.MROPE_OK
    assert _lib.load().mrope_last_kernel() == b""


@fake_ptr_test
def test_in_place_alias_is_allowed_by_the_checks():
    # exact alias passes every check; with T = 0 nothing is launched
    assert _fused(T=0, qo=FAKE, ko=FAKE + 0x4000000) == _lib.MROPE_OK


@fake_ptr_test
def test_rms_norm_and_apply_rotary_reject_bad_arguments():
    lib = _lib.load()
    rc = lib.rms_norm(FAKE, 128, 4, 1, 128, None, 1e-6, _lib.DTYPE_BF16, FAKE + 0x100000, 128, None)
    assert rc == _lib.MROPE_EINVAL                     # no weight
    rc = lib.rms_norm(FAKE, 128, 4, 1, 127, FAKE + 0x200000, 1e-6, _lib.DTYPE_BF16,
                      FAKE + 0x100000, 127, None)
    assert rc == _lib.MROPE_EINVAL                     # odd D
    rc = lib.apply_rotary_qk(FAKE, 128, 1, None, 0, 0, 4, 128, 128, None, None, 128,
                             _lib.DTYPE_F32, 0, FAKE + 0x100000, 128, None, 0, None)
    assert rc == _lib.MROPE_EINVAL                     # no cos/sin
    rc = lib.apply_rotary_qk(FAKE, 128, 1, None, 0, 0, 4, 128, 128, FAKE + 0x300000,
                             FAKE + 0x100000, 128, _lib.DTYPE_F32, 0, FAKE + 0x100000, 128, None,
                             0, None)
    assert rc == _lib.MROPE_EINVAL                     # q_out overlaps sin
    rc = lib.apply_rotary_qk(FAKE, 128, 1, None, 0, 0, 4, 128, 128, FAKE + 0x300000,
                             FAKE + 0x400000, 128, _lib.DTYPE_F32, 5, FAKE + 0x100000, 128, None,
                             0, None)
    assert rc == _lib.MROPE_EINVAL                     # unknown precision


@fake_ptr_test
def test_cos_sin_rejects_bad_arguments():
    lib = _lib.load()
    inv = _lib.float_array([1.0] * 4)
    sec = _lib.int_array([4, 2, 2])
    rc = lib.mrope_cos_sin(FAKE, 16, 2, 16, inv, sec, 3, _lib.LAYOUT_INTERLEAVED, 16,
                           FAKE + 0x1000, FAKE + 0x2000, 16, None)
    assert rc == _lib.MROPE_EINVAL                     # n_axes != 3
    rc = lib.mrope_cos_sin(FAKE, 16, 3, 16, inv, sec, 3, _lib.LAYOUT_INTERLEAVED, 16,
                           FAKE + 0x1000, FAKE + 0x1010, 16, None)
    assert rc == _lib.MROPE_EINVAL                     # cos and sin overlap
    rc = lib.mrope_cos_sin(FAKE, 16, 3, 0, inv, sec, 3, _lib.LAYOUT_INTERLEAVED, 16,
                           FAKE + 0x1000, FAKE + 0x2000, 16, None)
    assert rc == _lib.MROPE_OK                         # T = 0: nothing to do


def test_binding_builds_no_cpu_path():
    # The binding has no CPU implementation to fall back on: a CPU tensor is
    # handed to the library as a host pointer only through these wrappers,
    # which always call the HIP entry points.
    import inspect
    src = inspect.getsource(M)
    assert "oracle" not in src and "numpy.cos" not in src and "np.cos" not in src


@fake_ptr_test
def test_decode_rejects_bad_arguments():
    lib = _lib.load()

    def call(**kw):
        a = dict(q=FAKE, q_ts=32 * 128, hq=32, k=FAKE + 0x4000000, k_ts=4 * 128, hk=4, batch=8,
                 n=1, D=128, rd=128, cl=FAKE + 0x8000000, rdel=FAKE + 0x8001000, theta=1e6,
                 wq=FAKE + 0xC000000, wk=FAKE + 0xC001000, eps=1e-6, dtype=_lib.DTYPE_BF16,
                 prec=_lib.PRECISION_EXACT, qo=FAKE + 0x20000000, qo_ts=32 * 128,
                 kc=FAKE + 0x30000000,
                 kc_seq=64 * 4 * 128, kc_tok=4 * 128, cap=64)
        a.update(kw)
        return lib.mrope_decode_qk(a["q"], a["q_ts"], a["hq"], a["k"], a["k_ts"], a["hk"],
                                   a["batch"], a["n"], a["D"], a["rd"], a["cl"], a["rdel"],
                                   a["theta"], a["wq"], a["wk"], a["eps"], a["dtype"],
                                   a["prec"], a["qo"], a["qo_ts"], a["kc"], a["kc_seq"],
                                   a["kc_tok"], a["cap"], None)

    assert call(batch=0) == _lib.MROPE_OK                      # nothing to do
    assert call(batch=-1) == _lib.MROPE_EINVAL
    assert call(cl=0) == _lib.MROPE_EINVAL                     # no cache lengths
    assert call(cap=0) == _lib.MROPE_EINVAL
    assert call(kc_tok=100) == _lib.MROPE_EINVAL               # row stride < hk*D
    assert call(kc_seq=10 * 4 * 128) == _lib.MROPE_EINVAL      # sequences overlap
    assert call(kc=FAKE + 64) == _lib.MROPE_EINVAL             # cache overlaps q
    assert call(kc=FAKE + 0x8000000 - 4 * 128) == _lib.MROPE_EINVAL   # cache overlaps cache_len
    assert call(wk=0) == _lib.MROPE_EINVAL
    assert call(rd=129) == _lib.MROPE_EINVAL
    assert call(theta=-1.0) == _lib.MROPE_EINVAL
    assert call(prec=9) == _lib.MROPE_EINVAL


def test_rope_index_workspace_size():
    lib = _lib.load()
    a = lib.mrope_rope_index_workspace_size(1, 32768, 0, 0)
    b = lib.mrope_rope_index_workspace_size(4, 32768, 10, 3)
    assert 0 < a < b
    assert lib.mrope_rope_index_workspace_size(-1, 10, 0, 0) == 0
    assert lib.mrope_rope_index_workspace_size(1, 0, 0, 0) > 0     # grid tables only


@fake_ptr_test
def test_position_builders_reject_bad_arguments():
    lib = _lib.load()
    ws_bytes = lib.mrope_rope_index_workspace_size(2, 100, 1, 1)

    def call(**kw):
        a = dict(types=FAKE, mask=0, B=2, L=100, img=FAKE + 0x1000, ni=1, vid=FAKE + 0x2000, nv=1,
                 merge=2, pos=FAKE + 0x10000, ps=200, delta=FAKE + 0x20000, status=FAKE + 0x20100,
                 ws=FAKE + 0x100000, wsb=ws_bytes)
        a.update(kw)
        return lib.mrope_rope_index(a["types"], a["mask"], a["B"], a["L"], a["img"], a["ni"],
                                    a["vid"], a["nv"], a["merge"], a["pos"], a["ps"], a["delta"],
                                    a["status"], a["ws"], a["wsb"], None)

    assert call(B=-1) == _lib.MROPE_EINVAL
    assert call(merge=0) == _lib.MROPE_EINVAL
    assert call(types=0) == _lib.MROPE_EINVAL
    assert call(status=0) == _lib.MROPE_EINVAL
    assert call(img=0) == _lib.MROPE_EINVAL
    assert call(ps=199) == _lib.MROPE_EINVAL                  # axis stride < B*L
    assert call(wsb=ws_bytes - 1) == _lib.MROPE_EINVAL        # short workspace
    assert call(ws=FAKE + 0x100004) == _lib.MROPE_EINVAL      # misaligned workspace
    assert call(pos=FAKE + 0x800) == _lib.MROPE_EINVAL        # pos overlaps the types
    assert call(delta=FAKE + 0x10000 + 4 * 150) == _lib.MROPE_EINVAL   # delta inside pos
    assert call(ws=FAKE + 0x10000) == _lib.MROPE_EINVAL       # workspace overlaps pos

    def vcall(**kw):
        a = dict(grid=FAKE, n=2, merge=2, N=64, pos=FAKE + 0x1000, ps=64, status=FAKE + 0x2000)
        a.update(kw)
        return lib.mrope_vision_pos_ids(a["grid"], a["n"], a["merge"], a["N"], a["pos"], a["ps"],
                                        a["status"], None)

    assert vcall(n=-1) == _lib.MROPE_EINVAL
    assert vcall(n=_lib.MAX_VISION_IMAGES + 1) == _lib.MROPE_EINVAL
    assert vcall(merge=0) == _lib.MROPE_EINVAL
    assert vcall(ps=63) == _lib.MROPE_EINVAL
    assert vcall(status=0) == _lib.MROPE_EINVAL
    assert vcall(pos=FAKE + 8) == _lib.MROPE_EINVAL           # pos overlaps the grids


@fake_ptr_test
def test_cache_arguments_are_checked():
    lib = _lib.load()
    assert lib.mrope_cos_sin_cache(7, 1e4, 10, FAKE, None) == _lib.MROPE_EINVAL     # odd dim
    assert lib.mrope_cos_sin_cache(16, 0.0, 10, FAKE, None) == _lib.MROPE_EINVAL
    assert lib.mrope_cos_sin_cache(16, 1e4, -1, FAKE, None) == _lib.MROPE_EINVAL
    assert lib.mrope_cos_sin_cache(16, 1e4, 10, FAKE + 4, None) == _lib.MROPE_EINVAL  # alignment
    assert lib.mrope_cos_sin_cache(16, 1e4, 0, None, None) == _lib.MROPE_OK          # nothing
    sec = _lib.int_array([24, 20, 20])

    def fused(cache, rows, qo=FAKE + 0x20000000):
        return lib.rmsnorm_mrope_qk_cached(
            FAKE, 32 * 128, 32, FAKE + 0x4000000, 4 * 128, 4, 16, 128, 128, FAKE + 0x8000000, 16,
            3, sec, 3, _lib.LAYOUT_INTERLEAVED, 1e6, None, None, 1e-6, _lib.DTYPE_BF16, 0, qo,
            32 * 128, FAKE + 0x24000000, 4 * 128, cache, rows, None)

    assert fused(None, 5) == _lib.MROPE_EINVAL                  # rows without a cache
    assert fused(FAKE + 0x30000004, 10) == _lib.MROPE_EINVAL    # misaligned cache
    assert fused(FAKE + 0x30000000, -1) == _lib.MROPE_EINVAL
    assert fused(FAKE + 0x20000000, 10) == _lib.MROPE_EINVAL    # cache overlaps q_out


@fake_ptr_test
def test_vision_qkv_rejects_bad_arguments():
    lib = _lib.load()
    n, H, D = 64, 4, 72

    def call(**kw):
        a = dict(qkv=FAKE, ts=3 * H * D, n=n, H=H, D=D, rd=72, pos=FAKE + 0x100000, ps=n,
                 theta=1e4, dtype=_lib.DTYPE_F32, prec=_lib.PRECISION_EXACT,
                 qo=FAKE + 0x200000, ko=FAKE + 0x300000, vo=FAKE + 0x400000, hs=n * D, ots=D,
                 cache=None, rows=0)
        a.update(kw)
        return lib.mrope_vision_qkv(a["qkv"], a["ts"], a["n"], a["H"], a["D"], a["rd"], a["pos"],
                                    a["ps"], a["theta"], a["dtype"], a["prec"], a["qo"], a["ko"],
                                    a["vo"], a["hs"], a["ots"], a["cache"], a["rows"], None)

    assert call(n=0) == _lib.MROPE_OK                         # nothing to do, nothing launched
    for kw, code in [
            (dict(H=-1), _lib.MROPE_EINVAL),
            (dict(ts=3 * H * D - 1), _lib.MROPE_EINVAL),         # token stride below the rows
            (dict(hs=0), _lib.MROPE_EINVAL),
            (dict(ots=-D), _lib.MROPE_EINVAL),
            (dict(hs=D, ots=D), _lib.MROPE_EINVAL),              # rows of two heads coincide
            (dict(rd=74), _lib.MROPE_EINVAL),                    # rotary_dim > D
            (dict(rd=70), _lib.MROPE_EINVAL),                    # odd vision half (35)
            (dict(theta=0.0), _lib.MROPE_EINVAL),
            (dict(pos=0), _lib.MROPE_EINVAL),
            (dict(qkv=0), _lib.MROPE_EINVAL),
            (dict(qo=0), _lib.MROPE_EINVAL),
            (dict(prec=5), _lib.MROPE_EINVAL),
            (dict(dtype=7), _lib.MROPE_EUNSUPPORTED),
            (dict(qo=FAKE + 64), _lib.MROPE_EINVAL),             # q planes overlap the input
            (dict(ko=FAKE + 0x200000 + 256), _lib.MROPE_EINVAL),  # k planes overlap q planes
            (dict(vo=FAKE + 0x100000), _lib.MROPE_EINVAL),       # v planes overlap positions
            (dict(cache=FAKE + 0x500004, rows=10), _lib.MROPE_EINVAL),   # misaligned cache
    ]:
        rc = call(**kw)
        assert rc == code, (kw, rc, lib.mrope_last_error())
        assert lib.mrope_last_error()


@fake_ptr_test
def test_buffers_beyond_32_bit_offsets_are_refused():
    """A kernel addresses one token's rows (or one block's planes) through a
    buffer descriptor with 32-bit byte offsets: a token whose rows span 2^31
    bytes or more is refused before anything is enqueued."""
    lib = _lib.load()
    big = 1 << 20                      # heads of 1024 bf16: one token's q rows = 2^31 bytes
    rc = _fused(hq=big, D=1024, q_ts=big * 1024, qo_ts=big * 1024, hk=4, k_ts=4 * 1024,
                ko_ts=4 * 1024, T=1, pos_stride=1,
                k=FAKE + (1 << 36), qo=FAKE + (1 << 37), ko=FAKE + (1 << 38),
                pos=FAKE + (1 << 39), wq=FAKE + (1 << 40), wk=FAKE + (1 << 40) + 4096)
    assert rc == _lib.MROPE_EUNSUPPORTED, lib.mrope_last_error()
    assert b"2^31" in lib.mrope_last_error()
    n, H, D = 1 << 20, 16, 72          # fp32 planes: (H - 1) * n * D * 4 bytes > 2^31
    rc = lib.mrope_vision_qkv(FAKE, 3 * H * D, n, H, D, 72, FAKE + (1 << 39), n, 1e4,
                              _lib.DTYPE_F32, _lib.PRECISION_EXACT, FAKE + (1 << 36),
                              FAKE + (1 << 37), FAKE + (1 << 38), n * D, D, None, 0, None)
    assert rc == _lib.MROPE_EUNSUPPORTED, lib.mrope_last_error()
    assert b"2^31" in lib.mrope_last_error()


@fake_ptr_test
def test_head_counts_are_bounded():
    """More than 2^20 heads per tensor is refused (row indices are split
    through binary32 reciprocals, exact within that bound)."""
    lib = _lib.load()
    big = (1 << 20) + 1
    rc = _fused(hq=big, q_ts=big * 128, qo_ts=big * 128, T=1, pos_stride=1,
                k=FAKE + (1 << 36), qo=FAKE + (1 << 37), ko=FAKE + (1 << 38),
                pos=FAKE + (1 << 39), wq=FAKE + (1 << 40), wk=FAKE + (1 << 40) + 4096)
    assert rc == _lib.MROPE_EUNSUPPORTED and b"heads" in lib.mrope_last_error()


@fake_ptr_test
def test_stream_copy_rejects_bad_arguments():
    lib = _lib.load()
    EINVAL = _lib.MROPE_EINVAL
    assert lib.mrope_stream_copy(FAKE, FAKE + 0x100000, 0, None) == _lib.MROPE_OK
    assert lib.mrope_stream_copy(FAKE, FAKE + 0x100000, -16, None) == EINVAL
    assert lib.mrope_stream_copy(FAKE, FAKE + 0x100000, 24, None) == EINVAL      # not 16 x n
    assert lib.mrope_stream_copy(FAKE + 8, FAKE + 0x100000, 64, None) == EINVAL  # misaligned
    assert lib.mrope_stream_copy(None, FAKE, 64, None) == EINVAL
    assert lib.mrope_stream_copy(FAKE, FAKE + 32, 64, None) == EINVAL            # overlap
    assert "overlap" in lib.mrope_last_error().decode()
    assert lib.mrope_stream_copy(FAKE, FAKE + 64, 1 << 41, None) == _lib.MROPE_EUNSUPPORTED


@fake_ptr_test
def test_rope_index_noalloc_rejects_before_any_hip_call():
    """The static-workspace form checks its arguments (and its size limit)
    before it takes the array's device address or launches anything."""
    lib = _lib.load()
    EINVAL, EUNSUP = _lib.MROPE_EINVAL, _lib.MROPE_EUNSUPPORTED

    def call(B=2, L=100, types=FAKE, pos=FAKE + 0x100000, delta=FAKE + 0x200000,
             status=FAKE + 0x300000, n_img=0, grids=None, merge=2):
        return lib.mrope_rope_index_noalloc(types, None, B, L, grids, n_img, None, 0, merge, pos,
                                            B * L, delta, status, None)
    assert call(B=-1) == EINVAL
    assert call(merge=0) == EINVAL
    assert call(types=None) == EINVAL
    assert call(status=None) == EINVAL
    assert call(n_img=3, grids=None) == EINVAL
    assert call(pos=FAKE + 2) == EINVAL                              # misaligned
    assert call(pos=FAKE + 40) == EINVAL                             # overlaps the token types
    n_img = _lib.ROPE_INDEX_SCRATCH_BYTES // 8 + 16
    assert lib.mrope_rope_index_workspace_size(2, 100, n_img, 0) > _lib.ROPE_INDEX_SCRATCH_BYTES
    assert call(n_img=n_img, grids=FAKE + 0x400000) == EUNSUP
    assert "static workspace" in lib.mrope_last_error().decode()
