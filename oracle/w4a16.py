"""Inference with the exported weights: dequantize, then multiply.

Oracle (test infrastructure only).  fp64 with the roundings the pages fix.

Source: "GPTQ: Mathematical Foundations ...", Inference Execution and Modern
Kernel Architectures -- the FP16xINT4 pipeline: load the packed codes,
dequantize in registers as W_fp16 = (W_int - zero) * scale, multiply with
the 16-bit activations, accumulate in FP16/FP32.  The metadata are the
16-bit scale and zero of Quantization Formats and Group Size.

Readings where the page leaves a step open:
* The dequantized weight is rounded once to the activations' 16-bit format
  (fp16 with fp16 activations, as the pipeline names; bf16 with bf16
  activations): (q − z) is an exact small integer and its product with the
  fp16 scale is exact in fp32, so the value is that exact product rounded to
  nearest-even in the activation format.
* The products and their sum are formed exactly here (fp64); the output is
  fp32, [M x N] for activations A [M x K] and weights [N x K] (Y = A·Ŵᵀ).
* g_idx maps each input column to its group (act-order layers); without it
  column k is in group k // g.
"""
from __future__ import annotations

import numpy as np

from .quantizer import unpack_dense


def _f16_value(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_to_act(x, act: str) -> np.ndarray:
    """Round fp64 values (each exact in fp32) to the activation format, RNE."""
    x = np.asarray(x, dtype=np.float64)
    if act == "f16":
        return x.astype(np.float16).astype(np.float64)
    if act == "bf16":
        u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
        r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
        return r.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(act)


def dequantize(qweight_dense, bits: int, K: int, scales_f16, zeros_f16, group_size: int,
               g_idx=None, act: str = "f16") -> np.ndarray:
    """Ŵ in the activation format, [N x K] fp64 values."""
    codes = unpack_dense(qweight_dense, K, bits).astype(np.float64)
    gi = (np.asarray(g_idx, dtype=np.int64) if g_idx is not None
          else np.arange(K) // (K if group_size in (-1, 0) or group_size >= K else group_size))
    s = _f16_value(scales_f16)[:, gi]
    z = _f16_value(zeros_f16)[:, gi]
    return round_to_act((codes - z) * s, act)


def w4a16_matmul(A, act: str, qweight_dense, bits: int, scales_f16, zeros_f16,
                 group_size: int, g_idx=None) -> np.ndarray:
    """Y = A·Ŵᵀ exactly (fp64) for A [M x K] given as 16-bit patterns."""
    A = np.asarray(A, dtype=np.uint16)
    K = A.shape[1]
    if act == "f16":
        a = A.view(np.float16).astype(np.float64)
    else:
        a = (A.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    W = dequantize(qweight_dense, bits, K, scales_f16, zeros_f16, group_size, g_idx, act)
    return a @ W.T


def accumulation_bound(A, act: str, W, K: int) -> np.ndarray:
    """Per output, the recursive-summation bound K·2⁻²⁴·Σ|a_k·w_k| of an fp32
    accumulation of exact products (each partial sum rounded once)."""
    A = np.asarray(A, dtype=np.uint16)
    if act == "f16":
        a = A.view(np.float16).astype(np.float64)
    else:
        a = (A.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return K * 2.0 ** -24 * (np.abs(a) @ np.abs(W).T)
