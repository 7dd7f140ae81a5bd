"""Uniform quantizers, per-group parameters, RTN baseline and the packed format.

Oracle (test infrastructure only).  fp64 throughout.

Sources:
* "INT4 and GPTQ Quantization", section Uniform INT4 Quantization: the affine
  map  ŵ = s·(q − z),  q = clamp(round(w/s + z), 0, 2ᵇ − 1)  with
  s = (max − min)/(2ᵇ − 1), and the symmetric variant
  s = max|w| / (2ᵇ⁻¹ − 1), q ∈ [−2ᵇ⁻¹, 2ᵇ⁻¹ − 1].
* same page, section Group Quantization: one (s, z) per g consecutive
  weights of a row; z = round(−min/s) clamped to [0, 2ᵇ − 1].
* "Quantization (INT8, INT4, GPTQ)", Deriving the scale and zero-point: the
  two endpoint equations give s = (x_max − x_min)/(q_max − q_min) and
  z = round(q_min − x_min/s); here q_min = 0.
* "GPTQ: Mathematical Foundations ...", Quantization Formats and Group Size:
  the same affine grid on {0..2ᵇ−1}; symmetric uses z = 2ᵇ⁻¹ in unsigned
  storage; the bit-rate b + (16+16)/g.
* same page, Inference Execution: eight 4-bit codes per 32-bit word.

Readings where the pages leave a step open:
* Rounding is round-half-to-even (numpy ``rint``) with z inside the round.
* A constant group (max == min == c) has no step size on the pages; it gets
  s = |c| (or 1 when c == 0), which reconstructs c exactly.
* The min/max range is the literal one (0 is not forced into it); z is
  clamped as in the Group Quantization listing.
* Symmetric codes are stored unsigned as q + 2ᵇ⁻¹ with z = 2ᵇ⁻¹; a group of
  zeros gets s = 1.
* Packing: along d_in, column 8k+i goes to bits 4i..4i+3 of word k (low
  nibble first); 2- and 3-bit codes use the same 4-bit container.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Params:
    """Quantizer settings ("GPTQ" card, Hyperparameters; "GPTQ: Mathematical
    Foundations ...", GPTQ Algorithm Execution Walkthrough signature)."""

    bits: int = 4
    group_size: int = 128      # -1: one group per row
    block_size: int = 128
    percdamp: float = 0.01
    act_order: bool = False
    sym: bool = False

    @property
    def maxq(self) -> int:
        return (1 << self.bits) - 1


def asym_params(mn, mx, bits: int):
    """Per-group affine parameters from the group's min and max.

    Returns (s, z, zraw): z is the clamped rounded zero-point, zraw = −min/s
    is its pre-round value (used to judge near-tie decisions).
    """
    mn = np.asarray(mn, dtype=np.float64)
    mx = np.asarray(mx, dtype=np.float64)
    maxq = (1 << bits) - 1
    s = (mx - mn) / maxq
    const = s == 0
    if np.any(const):
        c = np.abs(mn)
        s = np.where(const, np.where(c > 0, c, 1.0), s)
    zraw = -mn / s
    z = np.clip(np.rint(zraw), 0, maxq)
    return s, z, zraw


def asym_quantize(w, s, z, bits: int):
    """q = clamp(rint(w/s + z), 0, 2ᵇ−1),  ŵ = s(q − z).  Returns (v, q, ŵ)
    where v = w/s + z is the pre-round value in code units."""
    maxq = (1 << bits) - 1
    v = np.asarray(w, dtype=np.float64) / s + z
    q = np.clip(np.rint(v), 0, maxq)
    return v, q, s * (q - z)


def sym_params(absmax, bits: int):
    """Symmetric scale s = max|w| / (2ᵇ⁻¹ − 1) and its storage offset 2ᵇ⁻¹."""
    absmax = np.asarray(absmax, dtype=np.float64)
    s = absmax / ((1 << (bits - 1)) - 1)
    s = np.where(s > 0, s, 1.0)
    z = np.full_like(s, float(1 << (bits - 1)))
    return s, z


def sym_quantize(w, s, bits: int):
    """Signed symmetric codes q = clamp(rint(w/s), −2ᵇ⁻¹, 2ᵇ⁻¹ − 1), ŵ = s·q."""
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    q = np.clip(np.rint(np.asarray(w, dtype=np.float64) / s), lo, hi)
    return q, s * q


def group_bounds(d_in: int, group_size: int):
    """Column ranges [c0, c1) of the groups of a row (last one may be short)."""
    g = d_in if group_size in (-1, 0) or group_size >= d_in else group_size
    return [(c0, min(c0 + g, d_in)) for c0 in range(0, d_in, g)]


def rtn_grouped(W, bits: int, group_size: int, sym: bool = False):
    """Round-to-nearest baseline: per-group parameters from the original
    weights, no compensation ("INT4 and GPTQ Quantization", Group
    Quantization listing).  Returns (q, s, z, ŵ) with s, z of shape
    [d_out, n_groups] and q in unsigned storage."""
    W = np.asarray(W, dtype=np.float64)
    m, d = W.shape
    groups = group_bounds(d, group_size)
    q = np.zeros((m, d))
    what = np.zeros((m, d))
    S = np.zeros((m, len(groups)))
    Z = np.zeros((m, len(groups)))
    for gi, (c0, c1) in enumerate(groups):
        blk = W[:, c0:c1]
        if sym:
            s, z = sym_params(np.max(np.abs(blk), axis=1), bits)
        else:
            s, z, _ = asym_params(blk.min(axis=1), blk.max(axis=1), bits)
        _, qq, ww = asym_quantize(blk, s[:, None], z[:, None], bits)
        q[:, c0:c1], what[:, c0:c1] = qq, ww
        S[:, gi], Z[:, gi] = s, z
    return q.astype(np.uint8), S, Z, what


def pack_codes(q) -> np.ndarray:
    """Pack codes (< 16) eight to a uint32 word along d_in, low nibble first."""
    q = np.asarray(q)
    if q.size and (q.min() < 0 or q.max() > 15):
        raise ValueError("codes must lie in [0, 15]")
    m, d = q.shape
    words = (d + 7) // 8
    pad = np.zeros((m, words * 8), dtype=np.uint32)
    pad[:, :d] = q
    pad = pad.reshape(m, words, 8)
    out = np.zeros((m, words), dtype=np.uint32)
    for i in range(8):
        out |= pad[:, :, i] << np.uint32(4 * i)
    return out


def unpack_codes(words, d_in: int) -> np.ndarray:
    """Inverse of ``pack_codes``: uint32 [m, ceil(d/8)] -> uint8 [m, d]."""
    words = np.asarray(words, dtype=np.uint32)
    m = words.shape[0]
    out = np.zeros((m, words.shape[1] * 8), dtype=np.uint8)
    for i in range(8):
        out[:, i::8] = (words >> np.uint32(4 * i)) & np.uint32(0xF)
    return out[:, :d_in]


def bits_per_weight(bits: int, group_size: int) -> float:
    """Storage cost with a 16-bit scale and a 16-bit zero per group."""
    return bits + (16 + 16) / group_size


def pack_dense(q, bits: int) -> np.ndarray:
    """Dense b-bit storage ("GPTQ: Mathematical Foundations ...", Quantization
    Formats and Group Size: b bits per weight plus the per-group metadata;
    Inference Execution: codes packed into 32-bit words).

    Each row is one little-endian bit stream: code c occupies bits
    [c·b, c·b + b) of the row, and bit p of the stream is bit p % 32 of word
    p // 32.  Rows are padded to whole words with zeros.  For b = 4 this is
    the eight-per-word layout of ``pack_codes``; for b = 3, 32 codes fill
    exactly three words (codes 10 and 21 straddle a word boundary).
    """
    q = np.asarray(q, dtype=np.int64)
    if q.size and (q.min() < 0 or q.max() >= (1 << bits)):
        raise ValueError(f"codes must lie in [0, {(1 << bits) - 1}]")
    m, d = q.shape
    words = (d * bits + 31) // 32
    out = np.zeros((m, words), dtype=np.uint64)
    for c in range(d):
        for b in range(bits):
            p = c * bits + b
            bit = (q[:, c] >> b) & 1
            out[:, p // 32] |= bit.astype(np.uint64) << np.uint64(p % 32)
    return out.astype(np.uint32)


def unpack_dense(words, d_in: int, bits: int) -> np.ndarray:
    """Inverse of ``pack_dense``: uint32 [m, ceil(d·b/32)] -> codes [m, d]."""
    words = np.asarray(words, dtype=np.uint32).astype(np.int64)
    m = words.shape[0]
    out = np.zeros((m, d_in), dtype=np.int64)
    for c in range(d_in):
        for b in range(bits):
            p = c * bits + b
            out[:, c] |= ((words[:, p // 32] >> (p % 32)) & 1) << b
    return out.astype(np.uint8)


def fp16_bits(x) -> np.ndarray:
    """IEEE half precision of x, rounded to nearest-even, as uint16 bits
    (the 16-bit scale and zero of the metadata accounting)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def stored_bits_per_weight(d_in: int, bits: int, group_size: int) -> float:
    """Bits per weight a row actually occupies in the dense export: its
    packed words plus a 16-bit scale and a 16-bit zero per group."""
    g = d_in if group_size in (-1, 0) or group_size >= d_in else group_size
    n_groups = (d_in + g - 1) // g
    words = (d_in * bits + 31) // 32
    return (32 * words + 32 * n_groups) / d_in
