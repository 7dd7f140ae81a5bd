"""Pins for the oracle's GPTQ sweep (CPU only).

The sweep is a heuristic, so it is pinned by what the mathematics fixes:
reduction to RTN when H = cI, the exact loss identity, OBS conditional
optimality at block boundaries, equality with the explicit-downdate OBS form,
independence from the block size, the 2x2 closed form and brute force on
tiny layers.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import Params


def _problem(rng, m=24, d=96, n=512, outlier=True):
    X = rng.normal(size=(n, d))
    if outlier:
        X[:, rng.choice(d, 3, replace=False)] *= 20
    W = rng.normal(size=(m, d)) * 0.02
    return W, X, oracle.hessian(X, "f64")


# ---------------------------------------------------------------- H = c·I
@pytest.mark.parametrize("bits,g", [(4, 128), (3, 64), (2, 32), (4, -1)])
def test_scaled_identity_hessian_reduces_to_rtn(bits, g, rng):
    d = 256
    X = synth.hadamard_rows(512, d)
    H = oracle.hessian(X)
    W = rng.normal(size=(16, d)) * 0.02
    for act in (False, True):
        p = Params(bits=bits, group_size=g, act_order=act)
        r = oracle.gptq_layer(W, H, w_dtype="f64", params=p)
        q, S, Z, what = oracle.rtn_grouped(W, bits, g)
        assert np.array_equal(r["q"], q)
        assert np.array_equal(r["s"], S) and np.array_equal(r["z"], Z)
        assert np.array_equal(r["what"], what)
        if act:
            assert r["perm"].tolist() == list(range(d))
        assert np.count_nonzero(np.triu(r["U"], 1)) == 0


# ---------------------------------------------------------------- loss identity
@pytest.mark.parametrize("bits,g,act", [(4, 128, False), (3, 128, False), (4, 64, True),
                                        (2, 256, False), (4, -1, True)])
def test_loss_identity(bits, g, act, rng):
    W, X, H = _problem(rng, d=300, n=2048)
    r = oracle.gptq_layer(W, H, w_dtype="f64", params=Params(bits=bits, group_size=g, act_order=act))
    direct = np.array([np.sum((X @ (r["what"][i] - r["W"][i])) ** 2) for i in range(W.shape[0])])
    rhs = oracle.loss_identity_rhs(r["err"], r["W"], r["what"], r["damp"])
    np.testing.assert_allclose(direct, rhs, rtol=1e-8)
    np.testing.assert_allclose(oracle.layer_error_rows(r["W"], r["what"], H), rhs, rtol=1e-8)
    assert np.allclose(r["row_loss"], 0.5 * np.sum(r["err"] ** 2, axis=1))


def test_loss_identity_catches_a_planted_sign_error(rng):
    """A sweep with the compensation sign flipped breaks the identity."""
    W, X, H = _problem(rng, n=2048)
    prep = oracle.prepare(H, 0.01)
    good = oracle.gptq_sweep(W, prep["U"], Params())
    lhs = oracle.layer_error_rows(W, good["what"], H)
    rhs = oracle.loss_identity_rhs(good["err"], W, good["what"], prep["damp"])
    assert np.max(np.abs(lhs - rhs) / rhs) < 1e-8
    Ubad = prep["U"].copy()
    Ubad[np.triu_indices_from(Ubad, 1)] *= -1
    bad = oracle.gptq_sweep(W, Ubad, Params())
    lhs = oracle.layer_error_rows(W, bad["what"], H)
    rhs = oracle.loss_identity_rhs(bad["err"], W, bad["what"], prep["damp"])
    assert np.max(np.abs(lhs - rhs) / rhs) > 1e-3


# ---------------------------------------------------------------- OBS optimality
def test_conditional_optimality_at_block_ends(rng):
    """After each block, the free weights minimise the damped quadratic given
    the quantized ones: H_d[F,F]δ_F + H_d[F,E]δ_E = 0."""
    W, X, H = _problem(rng, d=200)
    prep = oracle.prepare(H, 0.01)
    Hd = prep["Hd"]
    checked = []

    def on_end(b1, Wcur):
        if b1 >= W.shape[1]:
            return
        dlt = Wcur - W
        resid = dlt[:, b1:] @ Hd[b1:, b1:] + dlt[:, :b1] @ Hd[:b1, b1:]
        scale = np.abs(dlt[:, :b1] @ Hd[:b1, b1:]).max()
        checked.append(np.abs(resid).max() / scale)

    oracle.gptq_sweep(W, prep["U"], Params(block_size=32, group_size=32), on_block_end=on_end)
    assert len(checked) == 6
    assert max(checked) < 1e-10


def test_cholesky_sweep_equals_explicit_downdate_obs(rng):
    for g, bits in [(32, 4), (64, 3), (-1, 2)]:
        W, X, H = _problem(rng, d=128)
        prep = oracle.prepare(H, 0.01)
        p = Params(bits=bits, group_size=g, block_size=64 if g != -1 else 128)
        a = oracle.gptq_sweep(W, prep["U"], p)
        b = oracle.obs_sequential(W, prep["Hd"], p)
        assert np.array_equal(a["q"], b["q"])
        np.testing.assert_allclose(a["what"], b["what"], atol=1e-12)


@pytest.mark.parametrize("g", [32, 128, -1])
def test_block_size_does_not_change_result(g, rng):
    W, X, H = _problem(rng, d=256)
    prep = oracle.prepare(H, 0.01)
    ref = oracle.gptq_sweep(W, prep["U"], Params(group_size=g, block_size=1))
    for B in (32, 128, 256):
        if g != -1 and not (B % g == 0 or g % B == 0):
            continue
        r = oracle.gptq_sweep(W, prep["U"], Params(group_size=g, block_size=B))
        assert np.array_equal(r["q"], ref["q"])
        np.testing.assert_allclose(r["what"], ref["what"], atol=1e-12)


def test_incompatible_group_and_block_rejected(rng):
    W, X, H = _problem(rng, d=96)
    prep = oracle.prepare(H, 0.01)
    with pytest.raises(ValueError):
        oracle.gptq_sweep(W, prep["U"], Params(group_size=48, block_size=32))


def test_two_by_two_closed_form(rng):
    """With d = 2 the OBS update of the Lagrangian derivation reduces to
    w₂' = w₂ + (w₁ − ŵ₁)·H_d,12 / H_d,22 ; then w₂' is quantized."""
    for _ in range(20):
        X = rng.normal(size=(50, 2)) @ rng.normal(size=(2, 2))
        H = oracle.hessian(X, "f64")
        W = rng.normal(size=(5, 2))
        r = oracle.gptq_layer(W, H, w_dtype="f64", params=Params(bits=3, group_size=-1))
        Hd = r["Hd"]
        s, z = r["s"][:, 0], r["z"][:, 0]
        w1h = s * (np.clip(np.rint(W[:, 0] / s + z), 0, 7) - z)
        w2p = W[:, 1] + (W[:, 0] - w1h) * Hd[0, 1] / Hd[1, 1]
        w2h = s * (np.clip(np.rint(w2p / s + z), 0, 7) - z)
        np.testing.assert_allclose(r["what"][:, 0], w1h, rtol=1e-14)
        np.testing.assert_allclose(r["what"][:, 1], w2h, rtol=1e-14)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("d,bits", [(1, 4), (2, 3), (3, 3), (4, 2), (3, 4)])
def test_brute_force_lower_bound(d, bits, rng):
    worse = 0
    for trial in range(15):
        X = rng.normal(size=(30, d)) * rng.uniform(0.3, 3, size=d)
        if d > 1:
            X[:, 0] += 0.8 * X[:, -1]
        H = oracle.hessian(X, "f64")
        W = rng.normal(size=(4, d))
        r = oracle.gptq_layer(W, H, w_dtype="f64", params=Params(bits=bits, group_size=-1, percdamp=0.0 if d == 1 else 0.01))
        rtn = oracle.rtn_grouped(W, bits, -1)
        for i in range(4):
            best, codes = oracle.brute_force_row(W[i], H, r["s"][i, 0], r["z"][i, 0], (1 << bits) - 1)
            e = float(oracle.layer_error_rows(W[i:i + 1], r["what"][i:i + 1], H)[0])
            assert e >= best - 1e-12 * max(1.0, best)
            if d == 1:
                assert np.array_equal(r["q"][i], codes)
                assert np.array_equal(r["q"][i], rtn[0][i])
            else:
                worse += e > best + 1e-12
    assert worse < 15 * 4  # GPTQ is a heuristic; it is not always optimal but must sometimes be


# ---------------------------------------------------------------- invariances
def test_hessian_scale_invariance(rng):
    W, X, H = _problem(rng, d=160)
    a = oracle.gptq_layer(W, H, w_dtype="f64", params=Params())
    b = oracle.gptq_layer(W, 1024.0 * H, w_dtype="f64", params=Params())
    assert np.array_equal(a["q"], b["q"])
    np.testing.assert_allclose(a["what"], b["what"], atol=1e-12)


def test_act_order_equals_natural_order_on_prepermuted_problem(rng):
    W, X, H = _problem(rng, d=200)
    a = oracle.gptq_layer(W, H, w_dtype="f64", params=Params(act_order=True))
    p = a["perm"]
    assert np.all(np.diff(np.diag(H)[p]) <= 0)
    b = oracle.gptq_layer(W[:, p], H[p][:, p], w_dtype="f64", params=Params(act_order=False))
    assert np.array_equal(a["q"][:, p], b["q"])
    np.testing.assert_allclose(a["what"][:, p], b["what"], atol=1e-12)
    inv = np.argsort(p)
    assert np.array_equal(a["g_idx"], inv // 128)


def test_gptq_beats_rtn_on_tiny_workload():
    """Reported quality check on the 256x256 workload (not a theorem)."""
    wl = synth.WORKLOADS["tiny-256"]
    W, X = synth.make_weights(wl), synth.make_activations(wl)
    r = oracle.gptq_layer(W, None, Params(), X=X)
    rtn = oracle.rtn_grouped(r["W"], 4, 128)
    e_gptq = oracle.layer_error(r["W"], r["what"], r["H"])
    e_rtn = oracle.layer_error(r["W"], rtn[3], r["H"])
    assert e_gptq < e_rtn


# ---------------------------------------------------------------- follow mode
def test_follow_mode_self_and_planted_flips(rng):
    """Mistakes are planted in the oracle's own decisions, on the CPU."""
    W, X, H = _problem(rng, m=32, d=256)
    p = Params()
    r = oracle.gptq_layer(W, H, w_dtype="f64", params=p)
    same = oracle.gptq_layer(W, H, w_dtype="f64", params=p, follow={"q": r["q"], "z": r["z"]})
    rep = same["report"]
    assert rep.code_allowed == 0 and rep.zero_allowed == 0 and rep.ok
    np.testing.assert_array_equal(same["what"], r["what"])
    d = W.shape[1]
    # last column: a flip there has no downstream effect, so the planted data
    # stay consistent.  Pick the row whose pre-round value is nearest a boundary.
    v = r["v_sweep"][:, d - 1]
    frac = v - np.floor(v)
    dist = np.abs(frac - 0.5)
    inside = (v > 0.5) & (v < 14.5)
    i = int(np.argmin(np.where(inside, dist, np.inf)))
    q2 = r["q"].copy()
    q2[i, d - 1] = np.floor(v[i]) + (1 if r["q"][i, d - 1] == np.floor(v[i]) else 0)
    assert abs(int(q2[i, d - 1]) - int(r["q"][i, d - 1])) == 1
    ok = oracle.gptq_layer(W, H, w_dtype="f64", params=p, follow={"q": q2, "z": r["z"]},
                           tie_tol=dist[i] * 1.0001)
    assert ok["report"].code_allowed == 1 and ok["report"].ok
    bad = oracle.gptq_layer(W, H, w_dtype="f64", params=p, follow={"q": q2, "z": r["z"]},
                            tie_tol=dist[i] * 0.5)
    assert bad["report"].code_hard == 1 and bad["report"].code_allowed == 0
    ex = bad["report"].hard_examples[0]
    assert (ex["row"], ex["where"]) == (i, d - 1)
    # a two-step flip is hard whatever the tolerance
    q3 = r["q"].copy()
    q3[i, d - 1] = 0 if r["q"][i, d - 1] >= 2 else 15
    assert oracle.gptq_layer(W, H, w_dtype="f64", params=p, follow={"q": q3, "z": r["z"]},
                             tie_tol=0.5)["report"].code_hard == 1
    # a zero-point moved by two steps is hard
    z2 = r["z"].copy()
    z2[5, 1] = z2[5, 1] + 2 if z2[5, 1] <= 13 else z2[5, 1] - 2
    badz = oracle.gptq_layer(W, H, w_dtype="f64", params=p, follow={"q": r["q"], "z": z2}, tie_tol=0.5)
    assert badz["report"].zero_hard == 1


@pytest.mark.parametrize("plant", ["transposed", "diag_shift", "no_lazy_update", "hinv_lazy_update"])
def test_loss_identity_catches_planted_mistakes(plant, rng):
    """Plausible mistakes in the sweep's operands break the exact identity."""
    W, X, H = _problem(rng, d=256, n=2048)
    prep = oracle.prepare(H, 0.01)
    U = prep["U"]
    if plant == "transposed":
        Ub = U.T.copy()
    elif plant == "diag_shift":
        Ub = U.copy()
        Ub[np.diag_indices_from(Ub)] = np.roll(np.diag(U), 1)
    elif plant == "no_lazy_update":
        Ub = np.triu(U) * 0
        for b0 in range(0, 256, 128):
            Ub[b0:b0 + 128, b0:b0 + 128] = U[b0:b0 + 128, b0:b0 + 128]
    else:  # the walkthrough's between-block product with the full inverse
        Ub = U.copy()
        for b0 in range(0, 256, 128):
            Ub[b0:b0 + 128, b0 + 128:] = prep["Hinv"][b0:b0 + 128, b0 + 128:]
    r = oracle.gptq_sweep(W, Ub, Params())
    lhs = oracle.layer_error_rows(W, r["what"], H)
    rhs = oracle.loss_identity_rhs(r["err"], W, r["what"], prep["damp"])
    assert np.max(np.abs(lhs - rhs) / np.abs(rhs)) > 1e-3
