"""ctypes declarations of libsvdq.so (see include/svdq.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsvdq.so")

MXFP4 = 1
INT4_G64 = 2
NVFP4 = 3
EPI_LOWRANK = 1
EPI_BIAS = 2
EPI_GELU = 4
EPI_OUT_F32 = 8

STATUS = {0: "SVDQ_OK", 1: "SVDQ_ERR_NULL", 2: "SVDQ_ERR_SHAPE", 3: "SVDQ_ERR_FORMAT", 4: "SVDQ_ERR_ALIGN",
          5: "SVDQ_ERR_WORKSPACE", 6: "SVDQ_ERR_DEVICE", 7: "SVDQ_ERR_LAUNCH", 8: "SVDQ_ERR_TOO_LARGE"}

# Every function the header declares, with (restype, argtypes).
_P = ctypes.c_void_p
_D = ctypes.c_void_p          # const svdq_layer_desc*
_I64 = ctypes.c_int64
SIGNATURES = {
    "svdq_weight_bytes": (ctypes.c_size_t, [_D]),
    "svdq_act_bytes": (ctypes.c_size_t, [_D, _I64]),
    "svdq_pack_weight": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P]),
    "svdq_quantize_act": (ctypes.c_int, [_D, _P, _P, _I64, _I64, _P, _P]),
    "svdq_gemm": (ctypes.c_int, [_D, _P, _P, _I64, _P, _I64, ctypes.c_uint32, _P]),
    "svdq_gemm_quant": (ctypes.c_int, [_D, _P, _P, _I64, ctypes.c_uint32, _D, _P, _P, _P]),
    "svdq_gemm_qkv": (ctypes.c_int, [_D, _P, _P, _I64, ctypes.c_uint32, ctypes.c_int32, _P, _P, ctypes.c_float,
                                     _P, _P, _P, _I64, _P]),
    "svdq_gemm_w4a16": (ctypes.c_int, [_D, _P, _P, _I64, _I64, _P, _I64, ctypes.c_uint32, _P]),
    "svdq_linear": (ctypes.c_int, [_D, _P, _P, _I64, _I64, _P, _I64, ctypes.c_uint32, _P, ctypes.c_size_t, _P]),
    "svdq_linear_noalloc": (ctypes.c_int, [_D, _P, _P, _I64, _I64, _P, _I64, ctypes.c_uint32, _P]),
    "svdq_unpack_weight": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P]),
    "svdq_unpack_act": (ctypes.c_int, [_D, _P, _I64, _P, _P, _P, _P]),
    "svdq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "svdq_device_check": (ctypes.c_int, []),
    "svdq_version": (ctypes.c_int, []),
    "svdq_test_force_device_error": (None, [ctypes.c_int]),
}


class LayerDesc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("K", ctypes.c_int32), ("N", ctypes.c_int32), ("rank", ctypes.c_int32)]


class SvdqError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m w4a4_quantized_linear_amd.build`")
        _warn_if_stale()
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _warn_if_stale() -> None:
    """Loud warning when the built library does not match the current sources."""
    import sys
    try:
        from .build import source_hash
        with open(LIB_PATH + ".srchash") as f:
            built = f.read().strip()
        if built != source_hash():
            print(f"WARNING: {LIB_PATH} was built from other sources than the ones in the tree; "
                  "rebuild with `python -m w4a4_quantized_linear_amd.build`", file=sys.stderr, flush=True)
    except OSError:
        print(f"WARNING: no source hash next to {LIB_PATH}; it may be stale", file=sys.stderr, flush=True)


def check(fn: str, status: int) -> None:
    if status != 0:
        raise SvdqError(fn, status, lib().svdq_status_str(status).decode())
