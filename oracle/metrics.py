"""Layer output error, tiny-layer brute force, and the OBS loss identity.

Oracle (test infrastructure only).  fp64.

Sources:
* "INT4 and GPTQ Quantization", The Quantization Error and Layerwise
  Objective, and "GPTQ: Mathematical Foundations ...", The Layer-Wise
  Reconstruction Problem: the objective ‖WX − ŴX‖²_F, a sum of independent
  per-row terms.
* "GPTQ: Mathematical Foundations ...", Minimal Error Penalty: quantizing w_q
  with optimal compensation raises ½δᵀHδ by (w_q − quant(w_q))²/(2[H_F⁻¹]_qq).
  With [H_F⁻¹]_qq = U_qq² (Cholesky section) and err_q = (w_q − ŵ_q)/U_qq this
  is ½err_q².  Summed over the sweep, on the damped H_d = H + λI
  (Hessian Damping section) with H = 2XXᵀ:
      ½δᵀH_dδ = ½Σerr²   ⇒   ‖δX‖² = ½Σerr² − (λ/2)‖δ‖²,
  an identity every exact run must satisfy (δ = Ŵ − W row by row).
"""
from __future__ import annotations

import itertools

import numpy as np


def layer_error_rows(W, What, H) -> np.ndarray:
    """Per-row ‖(w − ŵ)X‖² = δ(H/2)δᵀ for H = 2XXᵀ (undamped)."""
    D = np.asarray(What, dtype=np.float64) - np.asarray(W, dtype=np.float64)
    return 0.5 * np.einsum("ij,ij->i", D @ np.asarray(H, dtype=np.float64), D)


def layer_error(W, What, H) -> float:
    """‖WX − ŴX‖²_F computed as tr(ΔW (H/2) ΔWᵀ)."""
    return float(np.sum(layer_error_rows(W, What, H)))


def layer_error_direct(W, What, X) -> float:
    """‖WX − ŴX‖²_F computed directly from token-major X [N x d] (fp64)."""
    D = np.asarray(What, dtype=np.float64) - np.asarray(W, dtype=np.float64)
    Y = np.asarray(X, dtype=np.float64) @ D.T
    return float(np.sum(Y * Y))


def loss_identity_rhs(err, W, What, damp: float) -> np.ndarray:
    """Per-row ½Σerr² − (λ/2)‖ŵ − w‖², which must equal the per-row layer error."""
    D = np.asarray(What, dtype=np.float64) - np.asarray(W, dtype=np.float64)
    return 0.5 * np.sum(np.asarray(err) ** 2, axis=1) - 0.5 * damp * np.sum(D * D, axis=1)


def brute_force_row(w, H, s, z, maxq: int):
    """Exhaustive minimum of ‖(w − ŵ)X‖² over every code vector on one fixed
    grid ŵ_j = s(q_j − z), q_j ∈ {0..maxq} (d ≤ 4).  Returns (min, codes)."""
    w = np.asarray(w, dtype=np.float64)
    d = w.size
    if d > 4:
        raise ValueError("brute force is for d <= 4")
    best, arg = np.inf, None
    Hh = 0.5 * np.asarray(H, dtype=np.float64)
    for codes in itertools.product(range(maxq + 1), repeat=d):
        qv = np.asarray(codes, dtype=np.float64)
        dlt = s * (qv - z) - w
        e = float(dlt @ Hh @ dlt)
        if e < best:
            best, arg = e, qv
    return best, arg
