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
    "GPTQParams", "GPTQError", "NotPositiveDefinite", "hessian_accumulate",
    "hessian_accumulate_noalloc", "prepare_hinv",
    "quantize_layer", "quantize", "workspace_bytes", "version", "Prepared", "Quantized",
    "Exported", "export", "quantize_layers", "obq_layer", "timing", "timing_read", "w4a16_gemm",
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
    status: "object" = None   # prepare_hinv(sync=False): pinned host status words
    event: "object" = None    # ... and the event recorded after their copy

    def check(self) -> "Prepared":
        """For prepare_hinv(sync=False): wait for the status words and raise
        as prepare_hinv would have; a no-op for a synchronous preparation."""
        if self.status is None:
            return self
        self.event.synchronize()
        info = ctypes.c_int64(-1)
        rc = _native.lib().gptq_prepare_status(ctypes.c_void_p(self.status.data_ptr()),
                                               self.U.shape[0], ctypes.byref(info))
        if rc == _native.ERR_NOT_SPD:
            raise NotPositiveDefinite(rc, _native.last_error(), info.value)
        _check(rc)
        self.status = self.event = None
        return self


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
        raise ValueError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)")
    return m[t.dtype]


def _require(t, name, dtype, shape, device=None):
    """Dense tensor of the given dtype and shape (on `device` when given):
    the library reads and writes it as a plain row-major buffer."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _matrix_rows(t, name):
    """2-D with unit column stride (rows may be padded: the row stride is passed)."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1) or t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} must be 2-D with unit column stride")


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _ws_check(ws, device):
    torch = _torch()
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("a workspace must be a contiguous uint8 tensor")
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")


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
    torch = _torch()
    _matrix_rows(X, "X")
    n_tok, d = X.shape
    xdt = _dtype_code(X)
    _require(H, "H", torch.float32, (d, d), X.device)
    L = _native.lib()
    if ws is None:
        ws = _workspace(L.gptq_workspace_bytes(_native.WS_HESSIAN, 0, d, n_tok, None), X.device)
    _ws_check(ws, X.device)
    _check(L.gptq_hessian_accumulate(_dev(H, "H"), d, _dev(X, "X"), xdt, n_tok,
                                     X.stride(0), _dev(ws, "ws"), ws.numel(), _stream(X.device)))
    return H


def hessian(H, X, ws=None):
    """H = 2·XᵀX (X token-major [n_tok, d_in]): hessian_accumulate on a zeroed
    H in one call, without reading H."""
    torch = _torch()
    _matrix_rows(X, "X")
    n_tok, d = X.shape
    xdt = _dtype_code(X)
    _require(H, "H", torch.float32, (d, d), X.device)
    L = _native.lib()
    if ws is None:
        ws = _workspace(L.gptq_workspace_bytes(_native.WS_HESSIAN, 0, d, n_tok, None), X.device)
    _ws_check(ws, X.device)
    _check(L.gptq_hessian(_dev(H, "H"), d, _dev(X, "X"), xdt, n_tok, X.stride(0), _dev(ws, "ws"),
                          ws.numel(), _stream(X.device)))
    return H


def hessian_accumulate_noalloc(H, X):
    """H += 2·XᵀX without a workspace: the library's static device scratch
    (for callers that cannot allocate; d_in <= 4096; calls that overlap on
    one GPU race)."""
    torch = _torch()
    _matrix_rows(X, "X")
    n_tok, d = X.shape
    xdt = _dtype_code(X)
    _require(H, "H", torch.float32, (d, d), X.device)
    _check(_native.lib().gptq_hessian_accumulate_noalloc(_dev(H, "H"), d, _dev(X, "X"), xdt, n_tok,
                                                         X.stride(0), _stream(X.device)))
    return H


def prepare_hinv(H, params: GPTQParams, ws=None, sync: bool = True) -> Prepared:
    """Dead fix, damping, act-order and U (H is overwritten with H_d).

    sync=False returns at once (gptq_prepare_hinv_async): the work, and the
    quantization queued behind it, run while the host goes on; call
    ``Prepared.check()`` later for the factorization's outcome."""
    torch = _torch()
    if H.dim() != 2:
        raise ValueError("H must be a square matrix")
    d = H.shape[0]
    _require(H, "H", torch.float32, (d, d))
    L = _native.lib()
    p = params.c()
    dev = H.device
    U = torch.empty(d, d, dtype=torch.float32, device=dev)
    perm = torch.empty(d, dtype=torch.int32, device=dev)
    dead = torch.empty(d, dtype=torch.uint8, device=dev)
    if ws is None:
        ws = _workspace(L.gptq_workspace_bytes(_native.WS_PREPARE, 0, d, 0, ctypes.byref(p)), dev)
    _ws_check(ws, dev)
    if not sync:
        status = torch.empty(2, dtype=torch.int32, pin_memory=True)
        _check(L.gptq_prepare_hinv_async(_dev(H, "H"), d, ctypes.byref(p), _dev(U, "U"),
                                         _dev(perm, "perm"), _dev(dead, "dead"), _dev(ws, "ws"),
                                         ws.numel(), ctypes.c_void_p(status.data_ptr()),
                                         _stream(dev)))
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream(dev))
        return Prepared(U, perm, dead, natural=not params.act_order, status=status, event=ev)
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
    _matrix_rows(W, "W")
    m, d = W.shape
    wdt = _dtype_code(W)
    dev = W.device
    _require(prep.U, "U", torch.float32, (d, d), dev)
    if params.act_order and prep.natural:
        raise ValueError("act_order needs a Prepared from prepare_hinv with act_order")
    if not prep.natural:
        _require(prep.perm, "perm", torch.int32, (d,), dev)
    if prep.dead is not None:
        _require(prep.dead, "dead", torch.uint8, (d,), dev)
    L = _native.lib()
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
    _ws_check(ws, dev)
    _check(L.gptq_quantize_layer(
        _dev(W, "W"), wdt, m, d, W.stride(0), _dev(prep.U, "U"),
        None if prep.natural else _dev(prep.perm, "perm"),
        _dev(prep.dead, "dead"), ctypes.byref(p), _dev(qweight, "qweight"), _dev(scales, "scales"),
        _dev(zeros, "zeros"), _dev(W_hat, "W_hat"), _dev(g_idx, "g_idx"), _dev(row_loss, "row_loss"),
        _dev(ws, "ws"), ws.numel(), _stream(dev)))
    return Quantized(qweight, scales, zeros, W_hat, g_idx, row_loss)


def quantize_layers(Ws, prep: Prepared, params: GPTQParams, want_what: bool = True,
                    ws=None) -> list:
    """Several layers with the same inputs (one H, one factor): one Quantized
    per W, bitwise what quantize_layer gives for each alone."""
    torch = _torch()
    if not Ws:
        raise ValueError("no layers")
    d = Ws[0].shape[1]
    dev = Ws[0].device
    _require(prep.U, "U", torch.float32, (d, d), dev)
    if params.act_order and prep.natural:
        raise ValueError("act_order needs a Prepared from prepare_hinv with act_order")
    if not prep.natural:
        _require(prep.perm, "perm", torch.int32, (d,), dev)
    if prep.dead is not None:
        _require(prep.dead, "dead", torch.uint8, (d,), dev)
    p = params.c()
    cpw = 8 if params.bits <= 4 else 4
    ng = params.n_groups(d)
    outs, descs = [], (_native.Layer * len(Ws))()
    for i, W in enumerate(Ws):
        _matrix_rows(W, f"W[{i}]")
        if W.shape[1] != d or W.device != dev:
            raise ValueError(f"W[{i}] must have {d} columns and live on {dev}")
        m = W.shape[0]
        o = Quantized(torch.empty(m, (d + cpw - 1) // cpw, dtype=torch.int32, device=dev),
                      torch.empty(m, ng, dtype=torch.float32, device=dev),
                      torch.empty(m, ng, dtype=torch.uint8, device=dev),
                      torch.empty(m, d, dtype=torch.float32, device=dev) if want_what else None,
                      None, torch.empty(m, dtype=torch.float32, device=dev))
        outs.append(o)
        descs[i] = _native.Layer(_dev(W, "W"), _dtype_code(W), 0, m, W.stride(0),
                                 _dev(o.qweight, "qweight"), _dev(o.scales, "scales"),
                                 _dev(o.zeros, "zeros"), _dev(o.W_hat, "W_hat"),
                                 _dev(o.row_loss, "row_loss"))
    g_idx = torch.empty(d, dtype=torch.int32, device=dev)
    L = _native.lib()
    total = sum(W.shape[0] for W in Ws)
    if ws is None:
        ws = _workspace(L.gptq_workspace_bytes(_native.WS_QUANTIZE, total, d, 0, ctypes.byref(p)), dev)
    _ws_check(ws, dev)
    _check(L.gptq_quantize_layers(len(Ws), descs, d, _dev(prep.U, "U"),
                                  None if prep.natural else _dev(prep.perm, "perm"),
                                  _dev(prep.dead, "dead"), ctypes.byref(p), _dev(g_idx, "g_idx"),
                                  _dev(ws, "ws"), ws.numel(), _stream(dev)))
    for o in outs:
        o.g_idx = g_idx
    return outs


def quantize_independent(layers, params: GPTQParams, want_what: bool = True, ws=None) -> list:
    """Independent layers, each with its own inputs: ``layers`` is a list of
    (W, X) device tensors (W [d_out, d_in], X [n_tok, d_in] token-major).
    Every layer gets a fresh H = 2·XᵀX, its own factor and its quantization;
    the library runs the layers concurrently and synchronizes once.  Returns
    one (Quantized, Prepared, H_d) per layer, bitwise what hessian_accumulate,
    prepare_hinv and quantize_layer give for that layer alone.  ``ws``: None,
    or one workspace per layer (GPTQ_WS_LAYER bytes each).  Raises like
    prepare_hinv when a layer's factorization fails (the first such layer);
    the exception's ``statuses`` and ``results`` give every layer's status
    and outputs (valid for the layers that succeeded)."""
    torch = _torch()
    if not layers:
        raise ValueError("no layers")
    if ws is not None and len(ws) != len(layers):
        raise ValueError("ws must hold one workspace per layer")
    L = _native.lib()
    p = params.c()
    cpw = 8 if params.bits <= 4 else 4
    jobs = (_native.LayerJob * len(layers))()
    out, keep = [], []
    dev0 = layers[0][0].device
    for i, (W, X) in enumerate(layers):
        _matrix_rows(W, f"W[{i}]")
        _matrix_rows(X, f"X[{i}]")
        m, d = W.shape
        n_tok = X.shape[0]
        dev = W.device
        if dev != dev0:
            raise ValueError(f"W[{i}] is on {dev}; every layer must live on {dev0}")
        if X.shape[1] != d or X.device != dev:
            raise ValueError(f"X[{i}] must have {d} columns and live on {dev}")
        ng = params.n_groups(d)
        H = torch.zeros(d, d, dtype=torch.float32, device=dev)
        prep = Prepared(torch.empty(d, d, dtype=torch.float32, device=dev),
                        torch.empty(d, dtype=torch.int32, device=dev),
                        torch.empty(d, dtype=torch.uint8, device=dev),
                        natural=not params.act_order)
        q = Quantized(torch.empty(m, (d + cpw - 1) // cpw, dtype=torch.int32, device=dev),
                      torch.empty(m, ng, dtype=torch.float32, device=dev),
                      torch.empty(m, ng, dtype=torch.uint8, device=dev),
                      torch.empty(m, d, dtype=torch.float32, device=dev) if want_what else None,
                      torch.empty(d, dtype=torch.int32, device=dev),
                      torch.empty(m, dtype=torch.float32, device=dev))
        w = ws[i] if ws is not None else _workspace(
            L.gptq_workspace_bytes(_native.WS_LAYER, m, d, n_tok, ctypes.byref(p)), dev)
        _ws_check(w, dev)
        keep.append(w)
        jobs[i] = _native.LayerJob(
            _dev(X, "X"), _dtype_code(X), _dtype_code(W), n_tok, X.stride(0), _dev(W, "W"), m, d,
            W.stride(0), _dev(H, "H"), _dev(prep.U, "U"), _dev(prep.perm, "perm"),
            _dev(prep.dead, "dead"), _dev(q.qweight, "qweight"), _dev(q.scales, "scales"),
            _dev(q.zeros, "zeros"), _dev(q.W_hat, "W_hat"), _dev(q.g_idx, "g_idx"),
            _dev(q.row_loss, "row_loss"), _dev(w, "ws"), w.numel(), 0, 0, -1)
        out.append((q, prep, H))
    with _torch().cuda.device(dev0):   # the library runs the jobs on the current device
        rc = L.gptq_quantize_independent(len(layers), jobs, ctypes.byref(p), _stream(dev0))
    if rc != _native.OK:
        if rc == _native.ERR_NOT_SPD:
            bad = next(j for j in jobs if j.status == _native.ERR_NOT_SPD)
            err = NotPositiveDefinite(rc, _native.last_error(), bad.info)
        else:
            err = GPTQError(rc, _native.last_error())
        # per-layer statuses and results: the layers that succeeded are valid
        err.statuses = [j.status for j in jobs]
        err.results = out
        raise err
    return out


def obq_layer(W, H, params: GPTQParams, ws=None):
    """OBQ (greedy order per row) of a tiny layer against the fp32 Hessian H.

    Returns (Quantized, order [d_out, d_in] int32).  params.group_size must
    be -1 (one grid per row) and act_order False; d_in <= 128.
    """
    torch = _torch()
    _matrix_rows(W, "W")
    m, d = W.shape
    wdt = _dtype_code(W)
    dev = W.device
    _require(H, "H", torch.float32, (d, d), dev)
    p = params.c()
    cpw = 8 if params.bits <= 4 else 4
    qweight = torch.empty(m, (d + cpw - 1) // cpw, dtype=torch.int32, device=dev)
    scales = torch.empty(m, 1, dtype=torch.float32, device=dev)
    zeros = torch.empty(m, 1, dtype=torch.uint8, device=dev)
    W_hat = torch.empty(m, d, dtype=torch.float32, device=dev)
    order = torch.empty(m, d, dtype=torch.int32, device=dev)
    row_loss = torch.empty(m, dtype=torch.float32, device=dev)
    L = _native.lib()
    if ws is None:
        ws = _workspace(L.gptq_workspace_bytes(_native.WS_OBQ, m, d, 0, ctypes.byref(p)), dev)
    _ws_check(ws, dev)
    rc = L.gptq_obq_layer(_dev(W, "W"), wdt, m, d, W.stride(0), _dev(H, "H"), ctypes.byref(p),
                          _dev(qweight, "qweight"), _dev(scales, "scales"), _dev(zeros, "zeros"),
                          _dev(W_hat, "W_hat"), _dev(order, "order"), _dev(row_loss, "row_loss"),
                          _dev(ws, "ws"), ws.numel(), _stream(dev))
    if rc == _native.ERR_NOT_SPD:
        raise NotPositiveDefinite(rc, _native.last_error(), -1)
    _check(rc)
    return Quantized(qweight, scales, zeros, W_hat, None, row_loss), order


TIMED_STAGES = ("block_update", "sweep", "cholesky", "inverse", "hessian", "lead_panel")


def timing(enable: bool) -> None:
    """Start (clearing earlier records) or stop per-stage event timing."""
    _native.lib().gptq_timing(1 if enable else 0)


def timing_read() -> dict:
    """Milliseconds per timed stage since timing was enabled (or last read)."""
    buf = (ctypes.c_float * len(TIMED_STAGES))()
    _check(_native.lib().gptq_timing_read(buf, len(TIMED_STAGES)))
    return {k: float(v) for k, v in zip(TIMED_STAGES, buf)}


@dataclasses.dataclass
class Exported:
    qweight: "object"     # [d_out, ceil(d_in·bits/32)] int32, dense little-endian bit stream per row
    scales_f16: "object"  # [d_out, n_groups] float16
    zeros_f16: "object"   # [d_out, n_groups] float16


def export(q: Quantized, params: GPTQParams, d_in: int) -> Exported:
    """Dense b-bit codes and 16-bit scales/zeros from a quantize_layer result."""
    torch = _torch()
    m = q.scales.shape[0]
    ng = q.scales.shape[1]
    dev = q.scales.device
    cpw = 8 if params.bits <= 4 else 4
    _require(q.qweight, "qweight", torch.int32, (m, (d_in + cpw - 1) // cpw), dev)
    _require(q.scales, "scales", torch.float32, (m, ng), dev)
    _require(q.zeros, "zeros", torch.uint8, (m, ng), dev)
    qd = torch.empty(m, (d_in * params.bits + 31) // 32, dtype=torch.int32, device=dev)
    s16 = torch.empty(m, ng, dtype=torch.float16, device=dev)
    z16 = torch.empty(m, ng, dtype=torch.float16, device=dev)
    _check(_native.lib().gptq_export(params.bits, m, d_in, ng, _dev(q.qweight, "qweight"),
                                     _dev(q.scales, "scales"), _dev(q.zeros, "zeros"),
                                     _dev(qd, "qweight_dense"), _dev(s16, "scales_f16"),
                                     _dev(z16, "zeros_f16"), _stream(dev)))
    return Exported(qd, s16, z16)


def w4a16_gemm(A, ex: Exported, bits: int, group_size: int, g_idx=None, out=None, ws=None):
    """C = A·Ŵᵀ from an export: A [M, K] float16/bfloat16, C [M, N] float32.
    ws: the split-K workspace (allocated here when None; pass one to reuse)."""
    torch = _torch()
    _matrix_rows(A, "A")
    M, K = A.shape
    dev = A.device
    if A.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("A must be float16 or bfloat16")
    N, ng = ex.scales_f16.shape
    _require(ex.qweight, "qweight", torch.int32, (N, (K * bits + 31) // 32), dev)
    _require(ex.scales_f16, "scales_f16", torch.float16, (N, ng), dev)
    _require(ex.zeros_f16, "zeros_f16", torch.float16, (N, ng), dev)
    if g_idx is not None:
        _require(g_idx, "g_idx", torch.int32, (K,), dev)
    C = out if out is not None else torch.empty(M, N, dtype=torch.float32, device=dev)
    _require(C, "C", torch.float32, (M, N), dev)
    L = _native.lib()
    if ws is None:
        ws = _workspace(L.gptq_workspace_bytes(_native.WS_W4A16, N, K, M, None), dev)
    _ws_check(ws, dev)
    _check(L.gptq_w4a16_gemm(
        _dev(A, "A"), _dtype_code(A), M, K, A.stride(0), _dev(ex.qweight, "qweight"), bits,
        _dev(ex.scales_f16, "scales_f16"), _dev(ex.zeros_f16, "zeros_f16"),
        _dev(g_idx, "g_idx"), group_size, ng, N, _dev(C, "C"), N, _dev(ws, "ws"), ws.numel(),
        _stream(dev)))
    return C


def quantize(W, X, params: GPTQParams = GPTQParams()):
    """Whole layer: H from X, prepare, sweep.  Returns (Quantized, Prepared, H_d)."""
    torch = _torch()
    d = W.shape[1]
    H = torch.zeros(d, d, dtype=torch.float32, device=W.device)
    hessian_accumulate(H, X)
    prep = prepare_hinv(H, params)
    return quantize_layer(W, prep, params), prep, H
