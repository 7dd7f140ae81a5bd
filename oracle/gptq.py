"""The GPTQ column sweep: fixed order, OBS compensation, lazy block updates.

Oracle (test infrastructure only).  fp64, vectorized over rows.

Sources ("GPTQ: Mathematical Foundations ..."):
* The Layer-Wise Reconstruction Problem: rows are independent problems that
  share H, so every step below acts on all rows at once.
* The GPTQ Algorithmic Innovations, 1 (Arbitrary Order Quantization): one
  fixed column order for all rows.
* 2 (Lazy Batch Updates): columns are taken in blocks of B; inside a block
  each quantized column immediately updates only the block's remaining
  columns; after the block, the columns right of it receive the whole
  block's accumulated correction in one matrix product.
* 3 (Cholesky Decomposition and Pre-computation): with H⁻¹ = UᵀU (U upper,
  the transpose of the page's lower L), the compensation of column j onto a
  later column k is the ratio U_jk/U_jj and [H_F⁻¹]_jj = U_jj², so with
  err_j = (w_j − ŵ_j)/U_jj the update is w_k −= err_j·U_jk.
* GPTQ Algorithm Execution Walkthrough, step 3: the per-column quantizer,
  Err_block[:, j] = (w − q)/d with d the factor's diagonal, and the in-block
  rank-1 update.
* Group parameters: "INT4 and GPTQ Quantization", Group Quantization.

Readings where the pages are silent or disagree:
* U drives both the in-block and the between-block updates.  The
  walkthrough's between-block product uses H⁻¹ with the scaled errors, which
  does not reproduce the OBS update of the Lagrangian derivation; with U it
  does (the page's lazy-update formula E_B·([H⁻¹]_BB)⁻¹·[H⁻¹]_BF equals
  Err_B·U_BF when E_B is measured from the block-start weights and H⁻¹ is the
  remaining-set inverse).
* The walkthrough's re-quantization of the un-updated block after the loop is
  not performed; the codes are the per-column codes of the sweep.
* "w − q" in the error means w − ŵ (the dequantized value).
* A group's (s, z) come from the current, already compensated values of its
  columns when the sweep reaches the group's first column.  That needs the
  group starts to be block-aligned or the groups to sit inside blocks:
  B % g == 0, g % B == 0, or one group per row; other combinations are
  rejected.
* Follow mode: where another implementation's rounding decision (a code, or
  a group's zero-point) differs from the one taken here, the decision is
  checked -- it is *allowed* when the two values differ by one and the
  pre-round value here lies within ``tie_tol`` code units of the rounding
  boundary between them, *hard* otherwise -- and the other implementation's
  value is adopted so that both continue on the same state.  Nothing else
  is taken over: scales, errors and compensated weights stay this oracle's.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .hessian import hessian as _hessian
from .prepare import prepare as _prepare
from .quantizer import Params, asym_params, pack_codes, sym_params


@dataclasses.dataclass
class FollowReport:
    n_codes: int = 0
    n_groups: int = 0
    code_allowed: int = 0
    code_hard: int = 0
    zero_allowed: int = 0
    zero_hard: int = 0
    order_allowed: int = 0      # OBQ only: adopted choices of the next column
    order_hard: int = 0
    max_tie_dist: float = 0.0   # largest |pre-round − boundary| among adopted decisions
    hard_examples: list = dataclasses.field(default_factory=list)

    @property
    def ok(self) -> bool:
        return self.code_hard == 0 and self.zero_hard == 0 and self.order_hard == 0

    @property
    def frac_codes_identical(self) -> float:
        return 1.0 - self.code_allowed / max(self.n_codes, 1)


def _group_size(d: int, group_size: int) -> int:
    return d if group_size in (-1, 0) or group_size >= d else group_size


def _compatible(d: int, B: int, g: int) -> bool:
    """Group starts must be block starts, or groups must sit inside blocks."""
    return g >= d or B % g == 0 or g % B == 0


def _classify(mine, theirs, pre, tie_tol, report: FollowReport, kind: str, where):
    """Check adopted decisions; returns (#allowed, #hard)."""
    diff = np.nonzero(mine != theirs)[0]
    if diff.size == 0:
        return 0, 0
    lo = np.minimum(mine[diff], theirs[diff])
    dist = np.abs(pre[diff] - (lo + 0.5))
    ok = (np.abs(mine[diff] - theirs[diff]) == 1) & (dist <= tie_tol)
    n_ok = int(ok.sum())
    if n_ok:
        report.max_tie_dist = max(report.max_tie_dist, float(dist[ok].max()))
    bad = diff[~ok]
    for r in bad[:8]:
        if len(report.hard_examples) < 32:
            report.hard_examples.append(
                dict(kind=kind, row=int(r), where=int(where), pre=float(pre[r]),
                     mine=float(mine[r]), theirs=float(theirs[r])))
    return n_ok, int(bad.size)


def gptq_sweep(W, U, params: Params, follow: dict | None = None, tie_tol: float = 1e-4,
               on_block_end=None) -> dict:
    """Run the blocked sweep on an already permuted, dead-fixed W [m x d].

    ``U`` is the upper Cholesky factor of the damped inverse Hessian in the same
    column order.  ``follow`` may hold another implementation's decisions in
    sweep order: 'q' [m x d] codes and 'z' [m x n_groups] zero-points.
    ``on_block_end(b1, W)`` is called after each between-block update with
    the current weights (columns < b1 are final).

    Returns codes q (uint8), ŵ, err, pre-round values v (code units), scales
    s, zeros z, raw zeros −min/s, and the follow report.
    """
    W = np.array(W, dtype=np.float64, copy=True)
    U = np.asarray(U, dtype=np.float64)
    m, d = W.shape
    B = params.block_size
    g = _group_size(d, params.group_size)
    if not _compatible(d, B, g):
        raise ValueError("block size and group size must divide one another")
    maxq = params.maxq
    n_groups = (d + g - 1) // g
    Q = np.zeros((m, d), dtype=np.uint8)
    What = np.zeros((m, d))
    Err = np.zeros((m, d))
    V = np.zeros((m, d))
    S = np.zeros((m, n_groups))
    Z = np.zeros((m, n_groups))
    Zraw = np.zeros((m, n_groups))
    rep = FollowReport(n_codes=m * d, n_groups=m * n_groups)
    s = z = None
    for b0 in range(0, d, B):
        b1 = min(b0 + B, d)
        Wb = W[:, b0:b1].copy()
        Eb = np.zeros((m, b1 - b0))
        for j in range(b1 - b0):
            c = b0 + j
            if c % g == 0:
                gi = c // g
                c1 = min(c + g, d)
                cur = Wb[:, j:j + (c1 - c)] if c1 <= b1 else W[:, c:c1]
                if params.sym:
                    s, z = sym_params(np.max(np.abs(cur), axis=1), params.bits)
                    zraw = z.copy()
                else:
                    s, z, zraw = asym_params(cur.min(axis=1), cur.max(axis=1), params.bits)
                    if follow is not None:
                        zf = np.asarray(follow["z"][:, gi], dtype=np.float64)
                        a, h = _classify(z, zf, zraw, tie_tol, rep, "zero", gi)
                        rep.zero_allowed += a
                        rep.zero_hard += h
                        z = np.where(z != zf, zf, z)
                S[:, gi], Z[:, gi], Zraw[:, gi] = s, z, zraw
            w = Wb[:, j]
            v = w / s + z
            q = np.clip(np.rint(v), 0, maxq)
            if follow is not None:
                qf = np.asarray(follow["q"][:, c], dtype=np.float64)
                a, h = _classify(q, qf, v, tie_tol, rep, "code", c)
                rep.code_allowed += a
                rep.code_hard += h
                q = np.where(q != qf, qf, q)
            wq = s * (q - z)
            err = (w - wq) / U[c, c]
            Wb[:, j + 1:] -= np.outer(err, U[c, c + 1:b1])
            Eb[:, j] = err
            Q[:, c], What[:, c], Err[:, c], V[:, c] = q, wq, err, v
        W[:, b0:b1] = What[:, b0:b1]   # the block's weights are now fixed
        if b1 < d:
            W[:, b1:] -= Eb @ U[b0:b1, b1:]
        if on_block_end is not None:
            on_block_end(b1, W)
    return {"q": Q, "what": What, "err": Err, "v": V, "s": S, "z": Z, "zraw": Zraw, "report": rep}


def gptq_layer(W, H, params: Params, w_dtype: str = "f32", perm=None, follow: dict | None = None,
               tie_tol: float = 1e-4, X=None, x_dtype: str = "f32") -> dict:
    """Quantize one layer: prepare H, permute, sweep, un-permute, pack.

    W: stored weights [d_out x d_in] ('f32' values, 'bf16' bits, or 'f64'
       for exact test inputs).
    H: accumulated Hessian (fp64) or None, in which case it is built from X.
    perm: optional column order to use instead of act-order's own sort.
    follow: another implementation's decisions in ORIGINAL column order:
            'q' codes [m x d] and 'z' zeros [m x n_groups] (groups in sweep
            order).
    Returns prepare's outputs plus codes/ŵ/err in original column order, the
    packed codes, scales, zeros, g_idx, per-row loss ½Σerr², and the report.
    """
    if H is None:
        H = _hessian(X, x_dtype)
    prep = _prepare(H, params.percdamp, params.act_order, perm)
    if w_dtype == "bf16":
        W64 = (np.asarray(W, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    elif w_dtype == "f64":
        W64 = np.asarray(W, dtype=np.float64)
    else:
        W64 = np.asarray(W, dtype=np.float32).astype(np.float64)
    W64 = W64.copy()
    W64[:, prep["dead"]] = 0.0
    p = prep["perm"]
    m, d = W64.shape
    fol = None
    if follow is not None:
        fq = np.asarray(follow["q"])
        fol = {"q": fq[:, p] if p is not None else fq, "z": np.asarray(follow["z"])}
    Wp = W64[:, p] if p is not None else W64
    res = gptq_sweep(Wp, prep["U"], params, follow=fol, tie_tol=tie_tol)
    g = _group_size(d, params.group_size)
    if p is not None:
        inv = np.empty_like(p)
        inv[p] = np.arange(d)
        q, what, err = res["q"][:, inv], res["what"][:, inv], res["err"][:, inv]
        g_idx = inv // g
    else:
        q, what, err = res["q"], res["what"], res["err"]
        g_idx = np.arange(d) // g
    out = dict(prep)
    out.update(
        H=H, W=W64, q=q, what=what, err=err, s=res["s"], z=res["z"], zraw=res["zraw"],
        g_idx=g_idx.astype(np.int32), row_loss=0.5 * np.sum(err * err, axis=1),
        qweight=pack_codes(q) if params.bits <= 4 else None, report=res["report"],
        q_sweep=res["q"], v_sweep=res["v"],
    )
    return out
