"""H = 2 X Xᵀ in fp64.

Oracle (test infrastructure only).

Source: "GPTQ: Mathematical Foundations ...", Second-Order Taylor Expansion
and the Hessian -- for the layer-wise squared error the Hessian with respect
to a weight row is twice the unnormalized input covariance, the same for
every row; also "INT4 and GPTQ Quantization", The Quantization Error and
Layerwise Objective, and "Quantization (INT8, INT4, GPTQ)", Where the Hessian
comes from.  The pages write X as d_in x N; stored X here is token-major
[N x d_in], so H = 2·Xᵀ·X of the stored array.  No 1/N normalization (the
pages use none).
"""
from __future__ import annotations

import numpy as np


def _widen(chunk, dtype: str) -> np.ndarray:
    if dtype == "f64":
        return np.asarray(chunk, dtype=np.float64)
    if dtype == "bf16":
        u = np.ascontiguousarray(chunk, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    return np.asarray(chunk, dtype=np.float32).astype(np.float64)


def hessian(X, dtype: str = "f32", chunk: int = 8192, H: np.ndarray | None = None) -> np.ndarray:
    """Return H (+)= 2 Σ_t x_t x_tᵀ over the rows x_t of token-major X.

    X may be an array [N x d] or an iterable of such arrays (token batches);
    ``dtype`` says how the stored values are to be read ('f32', 'bf16'
    bit patterns, or 'f64' for exact test inputs).  When H is given it is
    accumulated into, so batches can be added across calls.
    """
    chunks = [X] if isinstance(X, np.ndarray) else X
    for c in chunks:
        c = np.asarray(c)
        if H is None:
            H = np.zeros((c.shape[1], c.shape[1]))
        for t0 in range(0, c.shape[0], chunk):
            x = _widen(c[t0:t0 + chunk], dtype)
            H += 2.0 * (x.T @ x)
    return H
