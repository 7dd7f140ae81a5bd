"""Pins for the oracle's Hessian and preparation steps (CPU only)."""
import numpy as np
import pytest
import scipy.linalg

import oracle
import synth
from oracle.prepare import NotSPDError


def _objective(delta, X):
    """‖δX‖² for a row perturbation δ, evaluated directly from token-major X."""
    y = X @ delta
    return float(y @ y)


def test_hessian_is_second_derivative_of_layer_objective(rng):
    """H must be the Hessian of ‖(w+δ)X − wX‖² (no formula reuse: second
    differences of the objective itself, exact for a quadratic)."""
    X = rng.normal(size=(40, 6))
    H = oracle.hessian(X, "f64")
    e = np.eye(6)
    for i in range(6):
        for j in range(6):
            fd = (_objective(e[i] + e[j], X) - _objective(e[i], X) - _objective(e[j], X)
                  + _objective(0 * e[i], X))
            assert H[i, j] == pytest.approx(fd, rel=1e-12, abs=1e-12)


def test_hessian_of_hadamard_columns_is_scaled_identity():
    X = synth.hadamard_rows(64, 48)
    H = oracle.hessian(X, "f64")
    assert np.array_equal(H, 2 * 64 * np.eye(48))


def test_hessian_accumulates_over_batches(rng):
    X = rng.normal(size=(1000, 17)).astype(np.float32)
    whole = oracle.hessian(X, "f32")
    parts = oracle.hessian([X[:300], X[300:701], X[701:]], "f32")
    np.testing.assert_allclose(parts, whole, rtol=1e-13, atol=1e-10)
    H = oracle.hessian(X[:500], "f32")
    H = oracle.hessian(X[500:], "f32", H=H)
    np.testing.assert_allclose(H, whole, rtol=1e-13, atol=1e-10)


def test_hessian_reads_bf16_bits_exactly(rng):
    x = rng.normal(size=(64, 8)).astype(np.float32)
    b = synth.f32_to_bf16_bits(x)
    xb = synth.bf16_bits_to_f32(b)
    assert np.all(np.abs(xb - x) <= np.abs(x) * 2.0 ** -8)
    np.testing.assert_array_equal(oracle.hessian(b, "bf16"), oracle.hessian(xb, "f32"))


def test_dead_channel_fix_and_relative_damping(rng):
    X = rng.normal(size=(200, 10))
    X[:, 3] = 0.0
    H = oracle.hessian(X, "f64")
    prep = oracle.prepare(H, percdamp=0.01)
    assert prep["dead"].tolist() == [i == 3 for i in range(10)]
    Hf = H.copy()
    Hf[3, 3] = 1.0
    lam = 0.01 * np.trace(Hf) / 10
    assert prep["damp"] == pytest.approx(lam, rel=1e-15)
    np.testing.assert_allclose(prep["Hd"] - Hf, lam * np.eye(10), atol=1e-12)
    # the dead channel is decoupled: no compensation reaches or leaves it
    U = prep["U"]
    assert np.all(U[3, 4:] == 0) and np.all(U[:3, 3] == 0)


def test_upper_factor_of_inverse(rng):
    X = rng.normal(size=(300, 40))
    X[:, 5] *= 20
    prep = oracle.prepare(oracle.hessian(X, "f64"), 0.01)
    U, Hd = prep["U"], prep["Hd"]
    assert np.allclose(U, np.triu(U)) and np.all(np.diag(U) > 0)
    np.testing.assert_allclose(U.T @ U @ Hd, np.eye(40), atol=1e-10)


def test_reverse_order_factor_equals_pages_route(rng):
    """The factor of H_d⁻¹ equals the inverse of H_d's reverse-order (upper)
    Cholesky factor: H_d = R Rᵀ, R upper  ⇒  H_d⁻¹ = R⁻ᵀR⁻¹ = UᵀU with U = R⁻¹."""
    X = rng.normal(size=(500, 64))
    prep = oracle.prepare(oracle.hessian(X, "f64"), 0.01)
    Hd = prep["Hd"]
    J = np.eye(64)[::-1]
    Lr = np.linalg.cholesky(J @ Hd @ J)
    R = J @ Lr @ J
    assert np.allclose(R, np.triu(R))
    np.testing.assert_allclose(R @ R.T, Hd, rtol=1e-12, atol=1e-9)
    U2 = scipy.linalg.solve_triangular(R, np.eye(64), lower=False)
    np.testing.assert_allclose(U2, prep["U"], rtol=1e-9, atol=1e-12 * np.abs(prep["U"]).max())


def test_act_order_permutation_is_stable_descending():
    diag = np.array([3.0, 5.0, 3.0, 9.0, 5.0, 1.0, 9.0])
    p = oracle.act_order_perm(diag)
    assert p.tolist() == [3, 6, 1, 4, 0, 2, 5]


def test_act_order_permutes_damped_hessian(rng):
    X = rng.normal(size=(100, 12)) * rng.uniform(0.5, 3, size=12)
    H = oracle.hessian(X, "f64")
    prep = oracle.prepare(H, 0.01, act_order=True)
    p = prep["perm"]
    assert np.all(np.diff(np.diag(H)[p]) <= 0)
    lam = prep["damp"]
    np.testing.assert_allclose(prep["Hd"], (H + lam * np.eye(12))[p][:, p], rtol=1e-15)


def test_not_positive_definite_is_reported():
    with pytest.raises(NotSPDError) as e:
        oracle.prepare(-np.eye(5), 0.0)
    assert e.value.pivot == 0
    H = np.eye(4)
    H[2, 2] = -3.0
    with pytest.raises(NotSPDError) as e:
        oracle.prepare(H, 0.0)
    assert e.value.pivot == 2
