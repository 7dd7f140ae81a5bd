"""Seeded synthetic inputs for the GPTQ layer-quantization path.

This module only draws random numbers and rounds them to the storage types
the path consumes (fp32 or bf16 bit patterns).  It holds none of the
method's arithmetic, so both the CPU oracle and the GPU tests/bench may use
it: the same seed gives the same bits on both sides.

Workloads stand in for the pages' real models and calibration sets (OPT,
BLOOM, LLaMA weights and "~128 samples" of text, which are not available
here).  Each one is a weight matrix W [d_out x d_in] and a calibration
activation matrix stored token-major, X [n_tok x d_in] (the pages write X as
d_in x N; token-major storage is its transpose).

Random-number scheme (deterministic, chunk-parallel):
  * ``numpy.random.SeedSequence(seed)`` is spawned into four children in a
    fixed order: W values, W outlier positions/values, X channel choice and
    scales, X values.
  * X values are drawn in chunks of ``X_CHUNK`` tokens; chunk k uses the
    k-th child spawned from the X-values sequence, so any chunk can be
    regenerated alone and chunks can be drawn in parallel.
  * Draws are fp32; bf16 inputs are the fp32 draws rounded to nearest-even.
    The bf16 bit pattern (uint16) is the canonical input for both sides.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

X_CHUNK = 4096


# ----------------------------------------------------------------------------
# storage-type helpers (bit manipulation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a stored input ('bf16' bits or 'f32') to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# workload recipes
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic layer: shapes, value distributions and quantizer settings."""

    name: str
    seed: int
    d_out: int
    d_in: int
    n_tok: int
    w_dtype: str = "bf16"          # 'bf16' or 'f32'
    x_dtype: str = "bf16"
    w_std: float = 0.02
    w_outlier_frac: float = 0.001  # fraction of W entries replaced by +-U(lo, hi)
    w_outlier_lo: float = 0.1
    w_outlier_hi: float = 0.3
    x_kind: str = "normal"         # 'normal' or 'abs_lognormal'
    x_outlier_channels: int = -1   # exact count; -1 -> round(frac * d_in)
    x_outlier_frac: float = 0.01
    x_outlier_scale: float = 15.0
    x_lognormal_sigma: float = 0.5
    bits: int = 4
    group_size: int = 128
    block_size: int = 128
    percdamp: float = 0.01
    act_order: bool = False
    sym: bool = False

    def scaled(self, d_out=None, d_in=None, n_tok=None, name=None, **kw) -> "Workload":
        """Same distributions at other sizes (used for oracle-sized parity runs)."""
        fields = dict(
            d_out=d_out or self.d_out,
            d_in=d_in or self.d_in,
            n_tok=n_tok or self.n_tok,
            name=name or f"{self.name}@{d_out or self.d_out}x{d_in or self.d_in}x{n_tok or self.n_tok}",
        )
        fields.update(kw)
        return dataclasses.replace(self, **fields)

    @property
    def n_x_outlier_channels(self) -> int:
        if self.x_kind != "normal":
            return 0
        if self.x_outlier_channels >= 0:
            return self.x_outlier_channels
        return int(round(self.x_outlier_frac * self.d_in))

    @property
    def n_w_outliers(self) -> int:
        return int(round(self.w_outlier_frac * self.d_out * self.d_in))

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "d_out": self.d_out,
            "d_in": self.d_in,
            "n_tok": self.n_tok,
            "w_dtype": self.w_dtype,
            "x_dtype": self.x_dtype,
            "bits": self.bits,
            "group_size": self.group_size,
            "block_size": self.block_size,
            "percdamp": self.percdamp,
            "act_order": self.act_order,
        }


# The five layers the path is measured on.
WORKLOADS = {
    "tiny-256": Workload(
        name="tiny-256 (256x256, 2048 tok, fp32)", seed=1001, d_out=256, d_in=256, n_tok=2048,
        w_dtype="f32", x_dtype="f32", w_outlier_frac=0.0, x_outlier_channels=4, x_outlier_scale=20.0),
    "llama7b-attn": Workload(
        name="llama7b-attn-proj (4096x4096, 131072 tok, bf16)", seed=1002, d_out=4096, d_in=4096,
        n_tok=131072, x_outlier_scale=15.0),
    "llama7b-up": Workload(
        name="llama7b-mlp-up (11008x4096, 131072 tok, bf16)", seed=1003, d_out=11008, d_in=4096,
        n_tok=131072, x_outlier_scale=15.0),
    "llama7b-up-actorder": Workload(
        name="llama7b-mlp-up act-order (11008x4096, 131072 tok, bf16)", seed=1003, d_out=11008,
        d_in=4096, n_tok=131072, x_outlier_scale=15.0, act_order=True),
    "llama7b-down": Workload(
        name="llama7b-mlp-down (4096x11008, 131072 tok, bf16, 3-bit)", seed=1004, d_out=4096,
        d_in=11008, n_tok=131072, x_kind="abs_lognormal", bits=3),
    "llama70b-mlp": Workload(
        name="llama70b-mlp (28672x8192, 262144 tok, bf16, act-order)", seed=1005, d_out=28672,
        d_in=8192, n_tok=262144, w_std=0.015, x_outlier_scale=20.0, act_order=True),
}


def _children(wl: Workload):
    ss = np.random.SeedSequence(wl.seed)
    return ss.spawn(4)  # [W values, W outliers, X channels, X values]


def make_weights(wl: Workload) -> np.ndarray:
    """W [d_out x d_in]: N(0, w_std^2) with a fixed count of +-U(lo, hi) outliers.

    Returns fp32 values (w_dtype 'f32') or bf16 bits as uint16 (w_dtype 'bf16').
    """
    c_val, c_out, _, _ = _children(wl)
    rng = np.random.Generator(np.random.PCG64(c_val))
    w = rng.standard_normal((wl.d_out, wl.d_in), dtype=np.float32)
    w *= np.float32(wl.w_std)
    k = wl.n_w_outliers
    if k > 0:
        ro = np.random.Generator(np.random.PCG64(c_out))
        pos = ro.choice(wl.d_out * wl.d_in, size=k, replace=False)
        sign = ro.integers(0, 2, size=k).astype(np.float32) * 2 - 1
        mag = ro.uniform(wl.w_outlier_lo, wl.w_outlier_hi, size=k).astype(np.float32)
        w.reshape(-1)[pos] = sign * mag
    if wl.w_dtype == "bf16":
        return f32_to_bf16_bits(w)
    return w


def x_channel_scales(wl: Workload) -> np.ndarray:
    """Per-input-channel multiplier applied to the X draws (fp32, length d_in)."""
    _, _, c_ch, _ = _children(wl)
    rng = np.random.Generator(np.random.PCG64(c_ch))
    sc = np.ones(wl.d_in, dtype=np.float32)
    if wl.x_kind == "normal":
        k = wl.n_x_outlier_channels
        if k > 0:
            ch = rng.choice(wl.d_in, size=k, replace=False)
            sc[ch] = np.float32(wl.x_outlier_scale)
    elif wl.x_kind == "abs_lognormal":
        sc = rng.lognormal(0.0, wl.x_lognormal_sigma, size=wl.d_in).astype(np.float32)
    else:
        raise ValueError(wl.x_kind)
    return sc


def _x_chunk(wl: Workload, child, scales: np.ndarray, rows: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(child))
    x = rng.standard_normal((rows, wl.d_in), dtype=np.float32)
    if wl.x_kind == "abs_lognormal":
        np.abs(x, out=x)
    x *= scales[None, :]
    if wl.x_dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def make_activations(wl: Workload, tok_begin: int = 0, tok_end: int | None = None,
                     threads: int | None = None) -> np.ndarray:
    """X [tokens x d_in] token-major, rows tok_begin..tok_end of the workload.

    tok_begin must be a multiple of X_CHUNK (chunks are the unit of seeding).
    """
    tok_end = wl.n_tok if tok_end is None else min(tok_end, wl.n_tok)
    if tok_begin % X_CHUNK:
        raise ValueError("tok_begin must be a multiple of X_CHUNK")
    _, _, _, c_x = _children(wl)
    n_chunks = (wl.n_tok + X_CHUNK - 1) // X_CHUNK
    kids = c_x.spawn(n_chunks)
    scales = x_channel_scales(wl)
    dt = np.uint16 if wl.x_dtype == "bf16" else np.float32
    out = np.empty((tok_end - tok_begin, wl.d_in), dtype=dt)
    first, last = tok_begin // X_CHUNK, (tok_end + X_CHUNK - 1) // X_CHUNK

    def work(ci):
        r0 = ci * X_CHUNK
        rows = min(X_CHUNK, wl.n_tok - r0)
        blk = _x_chunk(wl, kids[ci], scales, rows)
        a, b = max(r0, tok_begin), min(r0 + rows, tok_end)
        out[a - tok_begin:b - tok_begin] = blk[a - r0:b - r0]

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or last - first <= 1:
        for ci in range(first, last):
            work(ci)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(first, last)))
    return out


def hadamard_rows(n_tok: int, d_in: int) -> np.ndarray:
    """Token-major X whose columns are distinct columns of a Sylvester Hadamard
    matrix of order n_tok (a power of two, n_tok >= d_in).  Entries are +-1, so
    the columns are exactly orthogonal: XᵀX = n_tok * I."""
    if n_tok & (n_tok - 1) or n_tok < d_in:
        raise ValueError("n_tok must be a power of two >= d_in")
    h = np.ones((1, 1), dtype=np.float32)
    while h.shape[0] < n_tok:
        h = np.block([[h, h], [h, -h]])
    return np.ascontiguousarray(h[:, :d_in])
