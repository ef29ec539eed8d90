"""ctypes binding of libcpattn (include/cpattn.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step runs in the library's kernels.  There is no fallback:
if the shared library is missing or a call fails, a CpaError is raised.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcpattn.so")

CPA_OK, CPA_EINVAL, CPA_ESHAPE, CPA_EDTYPE, CPA_EUNSUPPORTED, CPA_EHIP = range(6)
CPA_BF16, CPA_F32 = 0, 1
CPA_ROPE_INTERLEAVED, CPA_ROPE_HALF = 0, 1
STATUS_NAMES = {0: "CPA_OK", 1: "CPA_EINVAL", 2: "CPA_ESHAPE", 3: "CPA_EDTYPE",
                4: "CPA_EUNSUPPORTED", 5: "CPA_EHIP"}

# name -> (restype, argtypes), in the order of include/cpattn.h
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_f64 = ctypes.c_double
SIGNATURES = {
    "cpa_zigzag_layout": (ctypes.c_int, [_i64, _i32, _c_i64p]),
    "cpa_partial": (ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i64, _i64, _i32,
                                   _vp, _vp, _i32, _f32, _vp, _vp, _vp]),
    "cpa_merge": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _vp]),
    "cpa_rank_forward_workspace": (_sz, [_i32, _i32, _i64, _i32, _i32]),
    "cpa_rank_forward": (ctypes.c_int, [_i32, _i32, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32,
                                        _i64, _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "cpa_rank_forward_noalloc": (ctypes.c_int, [_i32, _i32, _vp, _vp, _vp, _vp, ctypes.c_int,
                                                _i32, _i32, _i64, _i32, _i32, _f32, _vp, _vp,
                                                _vp]),
    "cpa_rank_forward_fused": (ctypes.c_int, [_i32, _i32, _vp, _vp, _vp, _vp, ctypes.c_int, _i32,
                                              _i32, _i64, _i32, _i32, _f32, _vp, _vp, _vp]),
    "cpa_share_forward": (ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i64, _i32,
                                         _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp]),
    "cpa_share_forward_precise": (ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i64,
                                                 _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp,
                                                 _vp]),
    "cpa_zigzag_permute": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i64, _i32, _vp, _i32,
                                          _i32, _i32, _i32, _vp]),
    "cpa_backward_delta": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i32, _vp, _vp]),
    "cpa_partial_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32,
                                            _i64, _i64, _i32, _vp, _vp, _i32, _f32, _vp, _vp, _vp,
                                            _vp]),
    "cpa_rank_backward": (ctypes.c_int, [_i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         ctypes.c_int, _i32, _i32, _i64, _i32, _i32, _f32, _vp, _vp,
                                         _vp, _vp, _vp]),
    "cpa_share_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i32,
                                          _i32, _i64, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                          _vp, _vp, _vp, _vp]),
    "cpa_rope": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i32, _i32, _i64, _i32, _vp, _f64, _i32,
                                _vp]),
    "cpa_zigzag_permute_rope": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i32, _i32, _i64, _i32, _vp,
                                               _i32, _i32, _i32, _f64, _i32, _vp]),
    "cpa_check_offsets": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "cpa_last_error": (ctypes.c_char_p, []),
    "cpa_version": (ctypes.c_char_p, []),
}

_lib = None


class CpaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


def load():
    """Load libcpattn.so (built in-tree) once and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CpaError(-1, f"{LIB_PATH} is not built; run `python -m sequence_attention_cpa_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != CPA_OK:
        raise CpaError(status, load().cpa_last_error().decode(errors="replace"))


def last_error() -> str:
    return load().cpa_last_error().decode(errors="replace")


def version() -> str:
    return load().cpa_version().decode()
