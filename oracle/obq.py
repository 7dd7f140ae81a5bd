"""Optimal Brain Quantization: greedy order, one row at a time.

Oracle (test infrastructure only).  fp64.  O(d³) per row: tiny layers only.

Sources ("GPTQ: Mathematical Foundations ..."):
* Optimal Brain Surgeon (OBS) and Optimal Brain Quantization (OBQ), and the
  Lagrangian Derivation: quantizing w_q to quant(w_q) with the free weights F
  compensated optimally moves them by
      δ_F = −(w_q − quant(w_q)) / [H_F⁻¹]_qq · (H_F⁻¹)_{:,q}.
* Minimal Error Penalty: that step raises ½δᵀHδ by
      ΔE_q = (w_q − quant(w_q))² / (2 [H_F⁻¹]_qq).
* Recursive Inverse Hessian Updating: removing q from F,
      H_{F∖q}⁻¹ = (H_F⁻¹)_{−q,−q} − (H_F⁻¹)_{−q,q} (H_F⁻¹)_{q,−q} / [H_F⁻¹]_qq.
* The Computational Bottleneck of OBQ, and The GPTQ Algorithmic Innovations
  §1: OBQ picks, at every step and for every row separately, the free weight
  with the smallest ΔE_q (greedy order); GPTQ instead uses one fixed order
  for all rows.

Readings where the pages leave a step open:
* quant() is one fixed grid per row, set before the greedy steps from the
  row's own (dead-fixed) weights: the per-row asymmetric min/max grid of
  "INT4 and GPTQ Quantization" (Uniform INT4 Quantization), i.e. the grid
  GPTQ uses with one group per row.  Symmetric rows use max|w|.
* H is the damped Hessian of the walkthrough (dead fix, then
  λ = α·mean(diag H)), the same matrix GPTQ factors.
* Equal saliencies go to the lower column index.
* Follow mode, as for the GPTQ sweep: where another implementation chose a
  different column, the choice is allowed when its saliency lies within
  ``tie_rel`` (relative) of the minimum; a different code is allowed when
  the pre-round value lies within ``tie_tol`` code units of the boundary
  between the two codes.  Either way the other choice is adopted.
"""
from __future__ import annotations

import numpy as np

from .gptq import FollowReport
from .quantizer import Params, asym_params, sym_params


def obq_row(w, Hinv, s: float, z: float, maxq: int, follow_order=None, follow_q=None,
            tie_rel: float = 1e-9, tie_tol: float = 1e-4, report: FollowReport | None = None):
    """Greedy OBQ of one row w [d] against H_d⁻¹ (fp64, copied).

    Returns (codes [d], ŵ [d], order [d] (column quantized at each step),
    saliency [d] (ΔE of each step), pre-round values v [d] per column).
    """
    w = np.array(w, dtype=np.float64, copy=True)
    Hi = np.array(Hinv, dtype=np.float64, copy=True)
    d = w.size
    free = np.ones(d, dtype=bool)
    codes = np.zeros(d, dtype=np.int64)
    what = np.zeros(d)
    order = np.zeros(d, dtype=np.int64)
    sal = np.zeros(d)
    vpre = np.zeros(d)
    for step in range(d):
        idx = np.nonzero(free)[0]
        v = w[idx] / s + z
        qv = np.clip(np.rint(v), 0, maxq)
        wq = s * (qv - z)
        dE = (w[idx] - wq) ** 2 / (2.0 * np.diag(Hi)[idx])
        k = int(np.argmin(dE))            # first minimum: the lowest index
        q = int(idx[k])
        if follow_order is not None and int(follow_order[step]) != q:
            g = int(follow_order[step])
            kg = int(np.nonzero(idx == g)[0][0]) if free[g] else -1
            ok = kg >= 0 and dE[kg] <= dE[k] + tie_rel * max(dE[k], 1e-300) + 1e-300
            if report is not None:
                if ok:
                    report.order_allowed += 1
                else:
                    report.order_hard += 1
                    if len(report.hard_examples) < 32:
                        report.hard_examples.append(dict(kind="order", step=step, mine=q, theirs=g))
            if kg >= 0:
                q, k = g, kg
        vq = float(v[k])
        c = int(qv[k])
        if follow_q is not None and int(follow_q[q]) != c:
            cf = int(follow_q[q])
            lo = min(c, cf)
            ok = abs(c - cf) == 1 and abs(vq - (lo + 0.5)) <= tie_tol
            if report is not None:
                if ok:
                    report.code_allowed += 1
                    report.max_tie_dist = max(report.max_tie_dist, abs(vq - (lo + 0.5)))
                else:
                    report.code_hard += 1
                    if len(report.hard_examples) < 32:
                        report.hard_examples.append(dict(kind="code", step=step, col=q, pre=vq,
                                                         mine=c, theirs=cf))
            c = cf
        quant = s * (c - z)
        hqq = Hi[q, q]
        sal[step] = (w[q] - quant) ** 2 / (2.0 * hqq)
        # Lagrangian compensation of the free weights (q itself lands on quant)
        coef = (w[q] - quant) / hqq
        col = Hi[:, q].copy()
        w[free] -= coef * col[free]
        w[q] = quant
        codes[q], what[q], order[step], vpre[q] = c, quant, q, vq
        # drop q from F: rank-1 downdate, then clear its row and column
        free[q] = False
        rest = np.nonzero(free)[0]
        if rest.size:
            Hi[np.ix_(rest, rest)] -= np.outer(col[rest], col[rest]) / hqq
        Hi[q, :] = 0.0
        Hi[:, q] = 0.0
    return codes, what, order, sal, vpre


def obq_layer(W, Hd, params: Params, follow: dict | None = None, tie_rel: float = 1e-9,
              tie_tol: float = 1e-4) -> dict:
    """OBQ of every row of W [m x d] (dead-fixed) against the damped Hd.

    One grid per row (``params.group_size`` must mean one group per row).
    ``follow`` may hold another implementation's 'order' [m x d] and codes
    'q' [m x d].  Returns codes, ŵ, order, per-step saliencies, scales,
    zeros, pre-round values and the follow report.
    """
    W = np.asarray(W, dtype=np.float64)
    m, d = W.shape
    if params.group_size not in (-1, 0) and params.group_size < d:
        raise ValueError("OBQ runs with one grid per row (group_size -1)")
    Hinv = np.linalg.inv(np.asarray(Hd, dtype=np.float64))
    Hinv = 0.5 * (Hinv + Hinv.T)
    maxq = params.maxq
    if params.sym:
        S, Z = sym_params(np.max(np.abs(W), axis=1), params.bits)
    else:
        S, Z, _ = asym_params(W.min(axis=1), W.max(axis=1), params.bits)
    rep = FollowReport(n_codes=m * d, n_groups=m)
    Q = np.zeros((m, d), dtype=np.int64)
    What = np.zeros((m, d))
    Order = np.zeros((m, d), dtype=np.int64)
    Sal = np.zeros((m, d))
    V = np.zeros((m, d))
    for r in range(m):
        fo = follow["order"][r] if follow is not None else None
        fq = follow["q"][r] if follow is not None else None
        Q[r], What[r], Order[r], Sal[r], V[r] = obq_row(
            W[r], Hinv, float(S[r]), float(Z[r]), maxq, fo, fq, tie_rel, tie_tol, rep)
    return {"q": Q.astype(np.uint8), "what": What, "order": Order, "saliency": Sal, "s": S,
            "z": Z, "v": V, "report": rep}
