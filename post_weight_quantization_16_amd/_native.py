"""ctypes view of libgptq_mi355x.so (the C ABI in include/gptq.h).

Argument marshalling only.  Loading fails loudly when the library has not
been built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptq_mi355x.so")

# gptq_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NOT_SPD, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4, -5
# gptq_dtype
F32, BF16, F16 = 0, 1, 2
# workspace kinds
WS_HESSIAN, WS_PREPARE, WS_QUANTIZE = 0, 1, 2

EXPORTS = (
    "gptq_workspace_bytes",
    "gptq_hessian_accumulate",
    "gptq_prepare_hinv",
    "gptq_quantize_layer",
    "gptq_last_error",
    "gptq_version",
)


class Params(ctypes.Structure):
    """Mirror of ``gptq_params``."""

    _fields_ = [
        ("bits", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("percdamp", ctypes.c_float),
        ("act_order", ctypes.c_int32),
        ("sym", ctypes.c_int32),
    ]


_lib = None

_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_pp = ctypes.POINTER(Params)


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m post_weight_quantization_16_amd.build` "
            "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    L.gptq_workspace_bytes.argtypes = [_int, _i64, _i64, _i64, _pp]
    L.gptq_workspace_bytes.restype = _sz
    L.gptq_hessian_accumulate.argtypes = [_vp, _i64, _vp, _int, _i64, _i64, _vp, _sz, _vp]
    L.gptq_hessian_accumulate.restype = _int
    L.gptq_prepare_hinv.argtypes = [_vp, _i64, _pp, _vp, _vp, _vp, _vp, _sz,
                                    ctypes.POINTER(ctypes.c_int64), _vp]
    L.gptq_prepare_hinv.restype = _int
    L.gptq_quantize_layer.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _pp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.gptq_quantize_layer.restype = _int
    L.gptq_last_error.argtypes = []
    L.gptq_last_error.restype = ctypes.c_char_p
    L.gptq_version.argtypes = []
    L.gptq_version.restype = ctypes.c_char_p
    _lib = L
    return L


def last_error() -> str:
    return lib().gptq_last_error().decode()
