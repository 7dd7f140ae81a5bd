"""Dead-channel fix, damping, act-order and the inverse-Hessian Cholesky factor.

Oracle (test infrastructure only).  fp64, LAPACK factorizations.

Sources ("GPTQ: Mathematical Foundations ..."):
* GPTQ Algorithm Execution Walkthrough, step 1: channels with a zero Hessian
  diagonal are dead -- their diagonal entry becomes 1 and their weight column
  becomes 0; then the damping is added.
* Hessian Damping and Numerical Regularization: H_damped = H + λI with
  λ = α·mean(diag H), α = 0.01 typical (also the "GPTQ" card, Hyperparameters,
  Hessian damping 0.01).
* Activation Ordering: π = argsort(diag H, descending); W and H are permuted,
  GPTQ runs on the permuted problem, the result is un-permuted.
* Cholesky Decomposition and Pre-computation, and the walkthrough's step 2:
  H⁻¹ from the Cholesky factor of H, then the upper Cholesky factor U of H⁻¹
  (H⁻¹ = UᵀU, the lower factor L = Uᵀ of the page's formulas).

Readings:
* The dead fix comes first, so the damping mean includes the restored 1s
  (the walkthrough's order).
* Act-order sorts the dead-fixed, undamped diagonal (uniform damping cannot
  change the order); the sort is stable, ties go to the lower index.
* The three-step route (factor H_d, invert, factor H⁻¹) is the pages' route and
  is kept here on purpose.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


class NotSPDError(np.linalg.LinAlgError):
    def __init__(self, msg, pivot=-1):
        super().__init__(msg)
        self.pivot = pivot


def dead_fix(H: np.ndarray):
    """Return (H', dead): H' has H'_ii = 1 wherever H_ii == 0."""
    H = np.array(H, dtype=np.float64, copy=True)
    dead = np.diag(H) == 0
    idx = np.nonzero(dead)[0]
    H[idx, idx] = 1.0
    return H, dead


def act_order_perm(diag: np.ndarray) -> np.ndarray:
    """Stable descending order of the Hessian diagonal (ties: lower index first)."""
    return np.argsort(-np.asarray(diag, dtype=np.float64), kind="stable").astype(np.int64)


def _chol_lower(A: np.ndarray) -> np.ndarray:
    try:
        return scipy.linalg.cholesky(A, lower=True, check_finite=True)
    except (np.linalg.LinAlgError, ValueError) as e:
        # locate the failing pivot with LAPACK's info code
        _, info = scipy.linalg.lapack.dpotrf(np.nan_to_num(A), lower=1)
        raise NotSPDError(f"matrix is not positive definite ({e})", pivot=int(info) - 1) from None


def inverse_cholesky_upper(Hd: np.ndarray):
    """Return (H⁻¹, U) with U upper triangular, positive diagonal, H⁻¹ = UᵀU."""
    L = _chol_lower(Hd)
    n = Hd.shape[0]
    Hinv = scipy.linalg.cho_solve((L, True), np.eye(n))
    Hinv = 0.5 * (Hinv + Hinv.T)
    U = scipy.linalg.cholesky(Hinv, lower=False)
    return Hinv, U


def prepare(H: np.ndarray, percdamp: float = 0.01, act_order: bool = False,
            perm: np.ndarray | None = None) -> dict:
    """Dead fix, (act-order), damping and the Cholesky factor of H_d⁻¹.

    ``perm`` may supply the column order instead of sorting (used to check
    another implementation's equally valid order for near-equal diagonals).
    Returns dict with Hd (damped, permuted), Hinv, U, perm (or None), dead
    (original column order), damp (λ).
    """
    H, dead = dead_fix(H)
    d = H.shape[0]
    if act_order and perm is None:
        perm = act_order_perm(np.diag(H))
    damp = percdamp * float(np.mean(np.diag(H)))
    Hd = H + damp * np.eye(d)
    if perm is not None:
        perm = np.asarray(perm, dtype=np.int64)
        Hd = Hd[perm][:, perm]
    Hinv, U = inverse_cholesky_upper(Hd)
    return {"Hd": Hd, "Hinv": Hinv, "U": U, "perm": perm, "dead": dead, "damp": damp}
