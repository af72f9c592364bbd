"""ctypes loader for libfp8bs.so and the C-ABI declarations.

The library is the only implementation: if it is not built, loading raises.
There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8bs.so")

STATUS = {
    0: "FP8_OK", 1: "FP8_ERR_NULL", 2: "FP8_ERR_SHAPE", 3: "FP8_ERR_LD", 4: "FP8_ERR_ALIGN",
    5: "FP8_ERR_UNSUPPORTED", 6: "FP8_ERR_DEVICE", 7: "FP8_ERR_LAUNCH", 8: "FP8_ERR_ALIAS",
}
TILE_ROW, TILE_COL, TILE_COL_TILED = 0, 1, 2
LAYOUT = {"fprop": 0, "dgrad": 1, "wgrad": 2, "dgrad_t": 3, "fprop_tiled": 4, "dgrad_t_tiled": 5, "wgrad_tiled": 6}
OUT_BF16, OUT_FP32 = 0, 1

# name -> (restype, argtypes); mirrors include/fp8bs.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
SIGNATURES = {
    "fp8_quant_act_1x128": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.c_int, _P, _I64, _P, _I64,
                                           _P, _P, _P, _P]),
    "fp8_quant_act_dual": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64,
                                          _P]),
    "fp8_quant_act_dual_tiled": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _I64,
                                                _P]),
    "fp8_quant_weight_128x128": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P]),
    "fp8_block_gemm": (ctypes.c_int, [ctypes.c_int, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P,
                                      _I64, _P, ctypes.c_int, _I64, _P]),
    "fp8_block_gemm_noalloc": (ctypes.c_int, [ctypes.c_int, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64,
                                              _P, _I64, _P, ctypes.c_int, _I64, _P]),
    "fp8_quant_weight_128x128_tiled": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _I64, _P]),
    "fp8_block_gemm_grouped_tiled": (ctypes.c_int, [_I32, _P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P,
                                                    _P, _P, ctypes.c_int, _I64, _P]),
    "fp8_block_gemm_fused_quant": (ctypes.c_int, [_I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P,
                                                  ctypes.c_int, _I64, _P, _I64, _P, _I64, _P]),
    "fp8_block_gemm_grouped": (ctypes.c_int, [_I32, _P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64,
                                              _P, _P, ctypes.c_int, _I64, _P]),
    "fp8_amax_history_update": (ctypes.c_int, [_P, _P, _I64, _F, ctypes.c_int, _P, _P]),
    "fp8_cast_e4m3": (ctypes.c_int, [_P, _I64, _P, _P]),
    "fp8_quant_act_tiles": (ctypes.c_int, [_P, _I64, _I64, _I64, _I32, _I32, _P, _I64, _P, _I64, _P, _P]),
    "fp8_gemm_promotion": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _I64, _I64, _P, _I64, _P]),
    "fp8_probe_mfma": (ctypes.c_int, [_I64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "fp8_probe_recip_online": (ctypes.c_int, [_P, _P, _I64, _P]),
    "fp8_probe_gemm_split": (ctypes.c_int, [_I64, _I64, _P, _P, _P]),
    "fp8_pack_tokens": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "fp8_unpack_tokens": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "fp8_dequant_tokens": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P]),
    "fp8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp8_abi_version": (ctypes.c_int, []),
}

_lib = None
_lock = threading.Lock()


class FP8Error(RuntimeError):
    """A non-OK status from libfp8bs."""

    def __init__(self, fn: str, status: int):
        self.status = status
        msg = STATUS.get(status, str(status))
        detail = ""
        if _lib is not None:
            try:
                detail = _lib.fp8_status_string(status).decode()
            except Exception:  # pragma: no cover
                pass
        super().__init__(f"{fn}: {msg} ({detail})")


def load_library(path: str | None = None):
    """Load libfp8bs.so (once).  Raises OSError/RuntimeError if it is absent."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"{p} is not built; run `python -m fine_grained_fp8_amd.build` "
                "(there is no CPU fallback)")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        raise FP8Error(fn, status)
