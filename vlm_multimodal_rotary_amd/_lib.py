"""ctypes view of libmrope.so (the C ABI declared in include/mrope.h).

Loading needs no GPU; compute entry points need one.  The library is loaded
after torch so both share one HIP runtime (torch's copy carries the same
soname).  A missing library is an error: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MROPE_LIB", os.path.join(HERE, "libmrope.so"))

MROPE_OK = 0
MROPE_EINVAL = -1
MROPE_EUNSUPPORTED = -2
MROPE_EHIP = -3

LAYOUT_CHUNKED = 0
LAYOUT_INTERLEAVED = 1
LAYOUT_VISION_2D = 2
LAYOUTS = {"chunked": LAYOUT_CHUNKED, "interleaved": LAYOUT_INTERLEAVED,
           "vision_2d": LAYOUT_VISION_2D}

DTYPE_F32 = 0
DTYPE_BF16 = 1

PRECISION_EXACT = 0
PRECISION_DTYPE = 1
PRECISION_FP32 = 2
PRECISIONS = {"exact": PRECISION_EXACT, "dtype": PRECISION_DTYPE, "fp32": PRECISION_FP32}

MAX_ROTARY_DIM = 512

POS_BAD_TYPE = 1
POS_NO_GRID = 2
POS_LENGTH = 4
POS_NOT_DIVISIBLE = 8
POS_COUNT = 16
POS_FLAGS = {POS_BAD_TYPE: "token type not 0/1/2", POS_NO_GRID: "visual run without a grid",
             POS_LENGTH: "visual run length differs from its grid",
             POS_NOT_DIVISIBLE: "grid not divisible by the merge size",
             POS_COUNT: "patch total differs from n_tokens"}
MAX_VISION_IMAGES = 4096
ROPE_INDEX_SCRATCH_BYTES = 1 << 20

_c_int, _c_i64, _c_double, _c_float = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_float
_vp = ctypes.c_void_p
_ip = ctypes.POINTER(ctypes.c_int)
_fp = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)

# name -> (restype, argtypes), in the order of include/mrope.h
SIGNATURES = {
    "mrope_inv_freq": (_c_int, [_c_int, _c_double, _fp]),
    "mrope_axis_table": (_c_int, [_c_int, _ip, _c_int, _c_int, _u8p]),
    "mrope_cos_sin": (_c_int, [_vp, _c_i64, _c_int, _c_i64, _fp, _ip, _c_int, _c_int, _c_int,
                               _vp, _vp, _c_i64, _vp]),
    "rms_norm": (_c_int, [_vp, _c_i64, _c_i64, _c_int, _c_int, _vp, _c_float, _c_int, _vp,
                          _c_i64, _vp]),
    "apply_rotary_qk": (_c_int, [_vp, _c_i64, _c_int, _vp, _c_i64, _c_int, _c_i64, _c_int,
                                 _c_int, _vp, _vp, _c_i64, _c_int, _c_int, _vp, _c_i64, _vp,
                                 _c_i64, _vp]),
    "rmsnorm_mrope_qk": (_c_int, [_vp, _c_i64, _c_int, _vp, _c_i64, _c_int, _c_i64, _c_int,
                                  _c_int, _vp, _c_i64, _c_int, _ip, _c_int, _c_int, _c_double,
                                  _vp, _vp, _c_float, _c_int, _c_int, _vp, _c_i64, _vp, _c_i64,
                                  _vp]),
    "mrope_cos_sin_cache": (_c_int, [_c_int, _c_double, _c_int, _vp, _vp]),
    "rmsnorm_mrope_qk_cached": (_c_int, [_vp, _c_i64, _c_int, _vp, _c_i64, _c_int, _c_i64, _c_int,
                                         _c_int, _vp, _c_i64, _c_int, _ip, _c_int, _c_int,
                                         _c_double, _vp, _vp, _c_float, _c_int, _c_int, _vp,
                                         _c_i64, _vp, _c_i64, _vp, _c_int, _vp]),
    "mrope_decode_qk": (_c_int, [_vp, _c_i64, _c_int, _vp, _c_i64, _c_int, _c_int, _c_int,
                                 _c_int, _c_int, _vp, _vp, _c_double, _vp, _vp, _c_float, _c_int,
                                 _c_int, _vp, _c_i64, _vp, _c_i64, _c_i64, _c_int, _vp]),
    "mrope_vision_qkv": (_c_int, [_vp, _c_i64, _c_i64, _c_int, _c_int, _c_int, _vp, _c_i64,
                                  _c_double, _c_int, _c_int, _vp, _vp, _vp, _c_i64, _c_i64, _vp,
                                  _c_int, _vp]),
    "mrope_rope_index_workspace_size": (ctypes.c_size_t, [_c_int, _c_i64, _c_int, _c_int]),
    "mrope_rope_index": (_c_int, [_vp, _vp, _c_int, _c_i64, _vp, _c_int, _vp, _c_int, _c_int,
                                  _vp, _c_i64, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "mrope_rope_index_noalloc": (_c_int, [_vp, _vp, _c_int, _c_i64, _vp, _c_int, _vp, _c_int,
                                          _c_int, _vp, _c_i64, _vp, _vp, _vp]),
    "mrope_vision_pos_ids": (_c_int, [_vp, _c_int, _c_int, _c_i64, _vp, _c_i64, _vp, _vp]),
    "mrope_stream_copy": (_c_int, [_vp, _vp, _c_i64, _vp]),
    "mrope_last_error": (ctypes.c_char_p, []),
    "mrope_last_kernel": (ctypes.c_char_p, []),
}

_LIB = None


class MropeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"mrope error {code}: {message}")
        self.code = code


def load() -> ctypes.CDLL:
    """Load libmrope.so once (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m vlm_multimodal_rotary_amd.build` (hipcc, gfx950)")
    try:  # share torch's HIP runtime when torch is present
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(rc: int) -> None:
    if rc != MROPE_OK:
        msg = load().mrope_last_error().decode(errors="replace")
        raise MropeError(rc, msg)


_INT_ARRAYS: dict = {}


def int_array(vals) -> ctypes.Array:
    """A C int array of vals (kept per distinct tuple: the same sections are
    passed on every call of a model's layers; the C side only reads it)."""
    key = tuple(int(v) for v in vals) if vals is not None else ()
    arr = _INT_ARRAYS.get(key)
    if arr is None:
        arr = (ctypes.c_int * max(1, len(key)))(*key)
        if len(_INT_ARRAYS) < 256:
            _INT_ARRAYS[key] = arr
    return arr


def float_array(vals) -> ctypes.Array:
    vals = [float(v) for v in vals]
    return (ctypes.c_float * max(1, len(vals)))(*vals)
