"""GPTQ layer quantization on MI355X (gfx950): Python binding.

Thin wrapper over the C ABI of ``libgptq_mi355x.so`` (include/gptq.h).
Every step of the path runs in the library's HIP kernels; this module only
checks tensor placement, passes device pointers and the current HIP stream,
and allocates outputs/workspaces with torch (PyTorch is used for device
memory and streams only).

    H = torch.zeros(d, d, device="cuda")
    hessian_accumulate(H, X)                      # H += 2 XᵀX, X token-major
    prep = prepare_hinv(H, params)                # U, perm, dead
    out = quantize_layer(W, prep, params)         # qweight, scales, zeros, ...
"""
from __future__ import annotations

import ctypes
import dataclasses

from . import _native

__all__ = [
    "GPTQParams", "GPTQError", "NotPositiveDefinite", "hessian_accumulate", "prepare_hinv",
    "quantize_layer", "quantize", "workspace_bytes", "version", "Prepared", "Quantized",
]


class GPTQError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class NotPositiveDefinite(GPTQError):
    def __init__(self, code, msg, pivot):
        super().__init__(code, msg)
        self.pivot = pivot


@dataclasses.dataclass(frozen=True)
class GPTQParams:
    bits: int = 4
    group_size: int = 128
    block_size: int = 128
    percdamp: float = 0.01
    act_order: bool = False
    sym: bool = False

    def c(self) -> _native.Params:
        return _native.Params(self.bits, self.group_size, self.block_size, self.percdamp,
                              int(self.act_order), int(self.sym))

    def n_groups(self, d_in: int) -> int:
        g = d_in if self.group_size <= 0 or self.group_size >= d_in else self.group_size
        return (d_in + g - 1) // g


@dataclasses.dataclass
class Prepared:
    U: "object"        # [d, d] fp32 upper factor of H_d⁻¹ (quantization order)
    perm: "object"     # [d] int32 quantization order
    dead: "object"     # [d] uint8 dead-channel mask (original order)
    natural: bool = False   # perm is the identity (prepared without act-order)


@dataclasses.dataclass
class Quantized:
    qweight: "object"  # [d_out, ceil(d_in/8)] int32 (bits <= 4) or [d_out, ceil(d_in/4)] (8-bit)
    scales: "object"   # [d_out, n_groups] fp32, groups in quantization order
    zeros: "object"    # [d_out, n_groups] uint8
    W_hat: "object"    # [d_out, d_in] fp32, original column order (or None)
    g_idx: "object"    # [d_in] int32
    row_loss: "object"  # [d_out] fp32, ½Σerr² per row


def _check(rc: int):
    if rc != _native.OK:
        raise GPTQError(rc, _native.last_error())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: _native.F32, torch.bfloat16: _native.BF16, torch.float16: _native.F16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def version() -> str:
    return _native.lib().gptq_version().decode()


def workspace_bytes(which: int, d_out: int, d_in: int, n_tok: int = 0,
                    params: GPTQParams | None = None) -> int:
    p = (params or GPTQParams()).c()
    return int(_native.lib().gptq_workspace_bytes(which, d_out, d_in, n_tok, ctypes.byref(p)))


def hessian_accumulate(H, X, ws=None):
    """H += 2·XᵀX (X token-major [n_tok, d_in]; row stride X.stride(0))."""
    L = _native.lib()
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    n_tok, d = X.shape
    if ws is None:
        ws = _workspace(L.gptq_workspace_bytes(_native.WS_HESSIAN, 0, d, n_tok, None), X.device)
    _check(L.gptq_hessian_accumulate(_dev(H, "H"), d, _dev(X, "X"), _dtype_code(X), n_tok,
                                     X.stride(0), _dev(ws, "ws"), ws.numel(), _stream(X.device)))
    return H


def prepare_hinv(H, params: GPTQParams, ws=None) -> Prepared:
    """Dead fix, damping, act-order and U (H is overwritten with H_d)."""
    torch = _torch()
    L = _native.lib()
    d = H.shape[0]
    p = params.c()
    dev = H.device
    U = torch.empty(d, d, dtype=torch.float32, device=dev)
    perm = torch.empty(d, dtype=torch.int32, device=dev)
    dead = torch.empty(d, dtype=torch.uint8, device=dev)
    if ws is None:
        ws = _workspace(L.gptq_workspace_bytes(_native.WS_PREPARE, 0, d, 0, ctypes.byref(p)), dev)
    info = ctypes.c_int64(-1)
    rc = L.gptq_prepare_hinv(_dev(H, "H"), d, ctypes.byref(p), _dev(U, "U"), _dev(perm, "perm"),
                             _dev(dead, "dead"), _dev(ws, "ws"), ws.numel(), ctypes.byref(info),
                             _stream(dev))
    if rc == _native.ERR_NOT_SPD:
        raise NotPositiveDefinite(rc, _native.last_error(), info.value)
    _check(rc)
    return Prepared(U, perm, dead, natural=not params.act_order)


def quantize_layer(W, prep: Prepared, params: GPTQParams, want_what: bool = True,
                   ws=None) -> Quantized:
    """Run the sweep on W [d_out, d_in] with the factor from prepare_hinv."""
    torch = _torch()
    L = _native.lib()
    if W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be 2-D with unit column stride")
    m, d = W.shape
    dev = W.device
    p = params.c()
    cpw = 8 if params.bits <= 4 else 4
    ng = params.n_groups(d)
    qweight = torch.empty(m, (d + cpw - 1) // cpw, dtype=torch.int32, device=dev)
    scales = torch.empty(m, ng, dtype=torch.float32, device=dev)
    zeros = torch.empty(m, ng, dtype=torch.uint8, device=dev)
    W_hat = torch.empty(m, d, dtype=torch.float32, device=dev) if want_what else None
    g_idx = torch.empty(d, dtype=torch.int32, device=dev)
    row_loss = torch.empty(m, dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(L.gptq_workspace_bytes(_native.WS_QUANTIZE, m, d, 0, ctypes.byref(p)), dev)
    _check(L.gptq_quantize_layer(
        _dev(W, "W"), _dtype_code(W), m, d, W.stride(0), _dev(prep.U, "U"),
        None if prep.natural else _dev(prep.perm, "perm"),
        _dev(prep.dead, "dead"), ctypes.byref(p), _dev(qweight, "qweight"), _dev(scales, "scales"),
        _dev(zeros, "zeros"), _dev(W_hat, "W_hat"), _dev(g_idx, "g_idx"), _dev(row_loss, "row_loss"),
        _dev(ws, "ws"), ws.numel(), _stream(dev)))
    return Quantized(qweight, scales, zeros, W_hat, g_idx, row_loss)


def quantize(W, X, params: GPTQParams = GPTQParams()):
    """Whole layer: H from X, prepare, sweep.  Returns (Quantized, Prepared, H_d)."""
    torch = _torch()
    d = W.shape[1]
    H = torch.zeros(d, d, dtype=torch.float32, device=W.device)
    hessian_accumulate(H, X)
    prep = prepare_hinv(H, params)
    return quantize_layer(W, prep, params), prep, H
