"""Pins for the oracle's OBQ comparator (CPU only).

OBQ is the greedy-order form of the same OBS step GPTQ takes in a fixed
order ("GPTQ: Mathematical Foundations ...": OBS and OBQ, Lagrangian
Derivation, Minimal Error Penalty, Recursive Inverse Hessian Updating, The
Computational Bottleneck of OBQ).  Each test checks it against something
other than its own formula: the Cholesky-form GPTQ sweep in a forced order,
the exact loss identity, RTN on H = cI, and brute force.
"""
import numpy as np
import pytest

import oracle
import synth


def _problem(m, d, n, seed, shift=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)) + shift
    x[:, rng.choice(d, min(2, d), replace=False)] *= 10
    H = oracle.hessian(x, "f64")
    W = rng.standard_normal((m, d)) * 0.02
    return W, H, x


def _damped(H, percdamp=0.01):
    Hf, _ = oracle.dead_fix(H)
    lam = percdamp * np.mean(np.diag(Hf))
    return Hf + lam * np.eye(H.shape[0]), lam


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_forced_fixed_order_equals_gptq_sweep(bits):
    """With the order forced to 0..d−1 the OBS steps with the explicit
    downdate are GPTQ's: the Cholesky-form sweep (one group per row) gives
    the same codes and values."""
    W, H, _ = _problem(12, 40, 400, bits)
    Hd, _ = _damped(H)
    p = oracle.Params(bits=bits, group_size=-1)
    U = oracle.inverse_cholesky_upper(Hd)[1]
    g = oracle.gptq_sweep(W, U, p)
    forced = {"order": np.tile(np.arange(40), (12, 1)), "q": g["q"]}
    o = oracle.obq_layer(W, Hd, p, follow=forced)
    assert np.array_equal(o["q"], g["q"])
    np.testing.assert_allclose(o["what"], g["what"], atol=1e-12)
    np.testing.assert_allclose(o["s"], g["s"][:, 0], rtol=1e-15)


@pytest.mark.parametrize("shift", [0.0, 1.5])
def test_loss_identity(shift):
    """Each step raises ½δᵀH_dδ by its saliency, so over a row
    ‖δX‖² = Σ ΔE − (λ/2)‖δ‖² exactly (δ = Ŵ − W, H = 2XXᵀ)."""
    W, H, x = _problem(10, 24, 300, 7, shift)
    Hd, lam = _damped(H)
    o = oracle.obq_layer(W, Hd, oracle.Params(bits=3, group_size=-1))
    D = o["what"] - W
    lhs = np.sum((D @ x.T) ** 2, axis=1)
    rhs = o["saliency"].sum(axis=1) - 0.5 * lam * np.sum(D * D, axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9)


def test_scaled_identity_hessian_gives_rtn():
    """H = cI: no compensation, so every code is the row grid's nearest point."""
    d = 64
    X = synth.hadamard_rows(128, d).astype(np.float64)
    H = oracle.hessian(X, "f64")
    W = np.random.default_rng(5).standard_normal((9, d)) * 0.02
    Hd, _ = _damped(H)
    o = oracle.obq_layer(W, Hd, oracle.Params(bits=4, group_size=-1))
    q, S, Z, what = oracle.rtn_grouped(W, 4, -1)
    assert np.array_equal(o["q"], q)
    np.testing.assert_allclose(o["what"], what, atol=1e-15)


@pytest.mark.parametrize("d,bits", [(1, 3), (2, 3), (3, 2), (4, 2)])
def test_brute_force_bound(d, bits):
    """Tiny rows: the greedy result never beats the exhaustive optimum on the
    same grid; at d = 1 they coincide."""
    rng = np.random.default_rng(100 + d)
    for _ in range(5):
        x = rng.standard_normal((50, d))
        H = oracle.hessian(x, "f64")
        w = rng.standard_normal((1, d)) * 0.1
        Hd, _ = _damped(H)
        p = oracle.Params(bits=bits, group_size=-1)
        o = oracle.obq_layer(w, Hd, p)
        e_obq = oracle.layer_error(w, o["what"], H)
        best, _ = oracle.brute_force_row(w[0], H, o["s"][0], o["z"][0], p.maxq)
        assert e_obq >= best - 1e-12
        if d == 1:
            assert e_obq == pytest.approx(best, abs=1e-15)


def test_greedy_order_differs_per_row_and_matches_gptq_quality():
    """Every row takes its own order (the coupling GPTQ removes), and on a
    small layer the fixed order lands close to the greedy one (reported, not
    a bound)."""
    W, H, _ = _problem(16, 48, 600, 3)
    Hd, _ = _damped(H)
    p = oracle.Params(bits=3, group_size=-1)
    o = oracle.obq_layer(W, Hd, p)
    assert len({tuple(r) for r in o["order"].tolist()}) > 1
    g = oracle.gptq_sweep(W, oracle.inverse_cholesky_upper(Hd)[1], p)
    e_obq = oracle.layer_error(W, o["what"], H)
    e_gptq = oracle.layer_error(W, g["what"], H)
    e_rtn = oracle.layer_error(W, oracle.rtn_grouped(W, 3, -1)[3], H)
    assert e_obq < e_rtn and e_gptq < e_rtn
    assert 0.5 < e_gptq / e_obq < 2.0
