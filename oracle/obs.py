"""Fixed-order OBS quantization with the explicit inverse-Hessian downdate.

Oracle (test infrastructure only).  fp64; O(d³) per layer, small d only.

This is the same greedy process as ``gptq.gptq_sweep`` written the long way,
to pin the Cholesky/blocked form against the derivation it comes from
("GPTQ: Mathematical Foundations ..."):
* Lagrangian Derivation: after fixing weight q to quant(w_q), the optimal
  change of the free weights is δ = −(w_q − quant(w_q)) / [H_F⁻¹]_qq · (H_F⁻¹)_{:,q},
  where H_F⁻¹ is the inverse of the Hessian restricted to the free set F.
* Recursive Inverse Hessian Updating: removing q from F updates the inverse by
  the symmetric rank-1 downdate
  H_{F∖q}⁻¹ = (H_F⁻¹)_{−q,−q} − (H_F⁻¹)_{−q,q}(H_F⁻¹)_{q,−q} / [H_F⁻¹]_qq.
* The Arbitrary Order Quantization section: the order is the fixed column
  order 0..d−1 for every row.

Group parameters are taken from the current values when a group starts, as
in the sweep.  Nothing is blocked.
"""
from __future__ import annotations

import numpy as np

from .quantizer import Params, asym_params, sym_params


def obs_sequential(W, Hd, params: Params) -> dict:
    """Quantize W [m x d] (sweep order, dead-fixed) against damped Hd [d x d]."""
    W = np.array(W, dtype=np.float64, copy=True)
    Hd = np.asarray(Hd, dtype=np.float64)
    m, d = W.shape
    g = d if params.group_size in (-1, 0) or params.group_size >= d else params.group_size
    maxq = params.maxq
    Hinv = np.linalg.inv(Hd)           # H_F⁻¹ with F = all columns
    Q = np.zeros((m, d), dtype=np.uint8)
    What = np.zeros((m, d))
    s = z = None
    for qi in range(d):
        if qi % g == 0:
            cur = W[:, qi:min(qi + g, d)]
            if params.sym:
                s, z = sym_params(np.max(np.abs(cur), axis=1), params.bits)
            else:
                s, z, _ = asym_params(cur.min(axis=1), cur.max(axis=1), params.bits)
        wq = W[:, qi]
        qq = np.clip(np.rint(wq / s + z), 0, maxq)
        quant = s * (qq - z)
        F = np.arange(qi, d)
        # δ over the free set (q itself moves to quant(w_q))
        coef = -(wq - quant) / Hinv[qi, qi]
        W[:, F] += np.outer(coef, Hinv[F, qi])
        W[:, qi] = quant               # exact constraint (the line above reaches it up to rounding)
        Q[:, qi], What[:, qi] = qq, quant
        # downdate: drop qi from F
        R = F[1:]
        if R.size:
            col = Hinv[R, qi].copy()
            Hinv[np.ix_(R, R)] -= np.outer(col, col) / Hinv[qi, qi]
        Hinv[qi, :] = 0.0
        Hinv[:, qi] = 0.0
    return {"q": Q, "what": What}
