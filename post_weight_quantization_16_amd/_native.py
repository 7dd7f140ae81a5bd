"""ctypes view of libgptq_mi355x.so (the C ABI in include/gptq.h).

Argument marshalling only.  Loading fails loudly when the library has not
been built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptq_mi355x.so")

# gptq_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NOT_SPD, ERR_WORKSPACE, ERR_HIP, ERR_INTERNAL = 0, -1, -2, -3, -4, -5, -6
# gptq_dtype
F32, BF16, F16 = 0, 1, 2
# workspace kinds
WS_HESSIAN, WS_PREPARE, WS_QUANTIZE, WS_OBQ, WS_W4A16, WS_LAYER = 0, 1, 2, 3, 4, 5

EXPORTS = (
    "gptq_workspace_bytes",
    "gptq_hessian_accumulate",
    "gptq_hessian",
    "gptq_hessian_accumulate_noalloc",
    "gptq_prepare_hinv",
    "gptq_prepare_hinv_async",
    "gptq_prepare_status",
    "gptq_quantize_layer",
    "gptq_quantize_layers",
    "gptq_quantize_independent",
    "gptq_obq_layer",
    "gptq_export",
    "gptq_w4a16_gemm",
    "gptq_timing",
    "gptq_timing_read",
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


class Layer(ctypes.Structure):
    """Mirror of ``gptq_layer``."""

    _fields_ = [
        ("W", ctypes.c_void_p),
        ("w_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("d_out", ctypes.c_int64),
        ("ld_w", ctypes.c_int64),
        ("qweight", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("zeros", ctypes.c_void_p),
        ("W_hat", ctypes.c_void_p),
        ("row_loss", ctypes.c_void_p),
    ]


class LayerJob(ctypes.Structure):
    """Mirror of ``gptq_layer_job``."""

    _fields_ = [
        ("X", ctypes.c_void_p),
        ("x_dtype", ctypes.c_int32),
        ("w_dtype", ctypes.c_int32),
        ("n_tok", ctypes.c_int64),
        ("ld_x", ctypes.c_int64),
        ("W", ctypes.c_void_p),
        ("d_out", ctypes.c_int64),
        ("d_in", ctypes.c_int64),
        ("ld_w", ctypes.c_int64),
        ("H", ctypes.c_void_p),
        ("U", ctypes.c_void_p),
        ("perm", ctypes.c_void_p),
        ("dead_mask", ctypes.c_void_p),
        ("qweight", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("zeros", ctypes.c_void_p),
        ("W_hat", ctypes.c_void_p),
        ("g_idx", ctypes.c_void_p),
        ("row_loss", ctypes.c_void_p),
        ("ws", ctypes.c_void_p),
        ("ws_bytes", ctypes.c_size_t),
        ("status", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("info", ctypes.c_int64),
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
    L.gptq_hessian.argtypes = [_vp, _i64, _vp, _int, _i64, _i64, _vp, _sz, _vp]
    L.gptq_hessian.restype = _int
    L.gptq_hessian_accumulate_noalloc.argtypes = [_vp, _i64, _vp, _int, _i64, _i64, _vp]
    L.gptq_hessian_accumulate_noalloc.restype = _int
    L.gptq_prepare_hinv.argtypes = [_vp, _i64, _pp, _vp, _vp, _vp, _vp, _sz,
                                    ctypes.POINTER(ctypes.c_int64), _vp]
    L.gptq_prepare_hinv.restype = _int
    L.gptq_prepare_hinv_async.argtypes = [_vp, _i64, _pp, _vp, _vp, _vp, _vp, _sz, _vp, _vp]
    L.gptq_prepare_hinv_async.restype = _int
    L.gptq_prepare_status.argtypes = [_vp, _i64, ctypes.POINTER(ctypes.c_int64)]
    L.gptq_prepare_status.restype = _int
    L.gptq_quantize_layer.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _pp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.gptq_quantize_layer.restype = _int
    L.gptq_quantize_layers.argtypes = [_int, ctypes.POINTER(Layer), _i64, _vp, _vp, _vp, _pp, _vp,
                                       _vp, _sz, _vp]
    L.gptq_quantize_layers.restype = _int
    L.gptq_quantize_independent.argtypes = [_int, ctypes.POINTER(LayerJob), _pp, _vp]
    L.gptq_quantize_independent.restype = _int
    L.gptq_obq_layer.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _pp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _sz, _vp]
    L.gptq_obq_layer.restype = _int
    L.gptq_export.argtypes = [_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.gptq_export.restype = _int
    L.gptq_w4a16_gemm.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _int, _vp, _vp, _vp, _int,
                                  _i64, _i64, _vp, _i64, _vp, _sz, _vp]
    L.gptq_w4a16_gemm.restype = _int
    L.gptq_timing.argtypes = [_int]
    L.gptq_timing.restype = _int
    L.gptq_timing_read.argtypes = [ctypes.POINTER(ctypes.c_float), _int]
    L.gptq_timing_read.restype = _int
    L.gptq_last_error.argtypes = []
    L.gptq_last_error.restype = ctypes.c_char_p
    L.gptq_version.argtypes = []
    L.gptq_version.restype = ctypes.c_char_p
    _lib = L
    return L


def last_error() -> str:
    return lib().gptq_last_error().decode()
