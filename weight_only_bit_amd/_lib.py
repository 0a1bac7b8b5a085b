"""ctypes loader for libweight_only_bit.so (the gfx950 C-ABI library).

The library is built in-tree by ``python -m weight_only_bit_amd.build``.  There
is no fallback: if the shared library is missing every operation raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libweight_only_bit.so")

# Status codes and dtype tags (include/weight_only_bit.h).
OK, INVALID_ARG, DTYPE, UNSUPPORTED, HIP = 0, 1, 2, 3, 4
F16, BF16, U4X8_I32, F32 = 0, 1, 2, 3
PATH_AUTO, PATH_SKINNY, PATH_TILED = 0, 1, 2
ACT_NONE, ACT_SILU_MUL = 0, 1

EXPORTS = [
    "wob_status_str", "wob_last_error", "wob_device_check",
    "w4a16_gemm", "w4a16_gemm_ex", "w4a16_gemm_grouped",
    "mxfp4_moe_gemm_workspace_size", "mxfp4_moe_gemm", "mxfp4_moe_gemm_tile_m",
    "mxfp4_moe_gemm_noalloc",
    "mxfp4_moe_stage2_workspace_size", "mxfp4_moe_stage2",
    "w4a16_dequant", "mxfp4_dequant", "wob_stream_read",
]

_vp = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

_SIGNATURES = {
    "wob_status_str": (ctypes.c_char_p, [_i]),
    "wob_last_error": (ctypes.c_char_p, []),
    "wob_device_check": (_i, []),
    "w4a16_gemm": (_i, [_vp, _i, _vp, _vp, _i, _vp, _i, _vp, _i64, _i64, _i64, _i64, _vp]),
    "w4a16_gemm_ex": (_i, [_vp, _i, _vp, _vp, _i, _vp, _i, _vp, _i64, _i64, _i64, _i64, _i, _vp]),
    "w4a16_gemm_grouped": (_i, [_vp, _i, _vp, _i64, _i64, _vp, _vp, _i, _vp, _i, _vp, _i64, _i64,
                                _i64, _vp]),
    "mxfp4_moe_gemm_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "mxfp4_moe_gemm": (_i, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i, _vp, _sz,
                            _vp]),
    "mxfp4_moe_gemm_tile_m": (_i, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i, _i,
                                   _vp, _sz, _vp]),
    "mxfp4_moe_gemm_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i,
                                    _vp]),
    "mxfp4_moe_stage2_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "mxfp4_moe_stage2": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _sz,
                              _vp]),
    "w4a16_dequant": (_i, [_vp, _vp, _i, _vp, _i, _vp, _i, _i64, _i64, _i64, _vp]),
    "mxfp4_dequant": (_i, [_vp, _vp, _vp, _i64, _i64, _vp]),
    "wob_stream_read": (_i, [_vp, _sz, _vp, _vp]),
}

_lib = None


class WobError(RuntimeError):
    """A non-OK status from the C library."""

    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({detail})")


class WobDtypeError(WobError, TypeError):
    pass


class WobArgError(WobError, ValueError):
    pass


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m weight_only_bit_amd.build` "
                "(there is no CPU fallback)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_str(status: int) -> str:
    return lib().wob_status_str(status).decode()


def last_error() -> str:
    return lib().wob_last_error().decode()


def check(status: int, where: str) -> None:
    if status == OK:
        return
    detail = last_error()
    if status == DTYPE:
        raise WobDtypeError(status, where, detail)
    if status == INVALID_ARG:
        raise WobArgError(status, where, detail)
    raise WobError(status, where, detail)
