"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs, at sizes the oracle finishes in seconds that span
several 128-wide tiles/blocks and ragged tails."""
import numpy as np
import pytest

import oracle
import synth
from parity_utils import (compare_layer, gq, log, params_of, rel_fro, run_gpu, to_dev,
                          torch_mod, H_TOL, U_TOL)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq().version()  # the library must load: no fallback exists


def _inputs(wl):
    return synth.make_weights(wl), synth.make_activations(wl)


# ---------------------------------------------------------------- Hessian
@pytest.mark.parametrize("d,n_tok,dtype,ld_pad", [
    (256, 2048, "f32", 0), (320, 5000, "bf16", 0), (200, 777, "f16", 0), (384, 4100, "bf16", 24),
    (130, 64, "bf16", 0), (1, 9, "f32", 0), (129, 3, "bf16", 8),
])
def test_hessian_matches_oracle(d, n_tok, dtype, ld_pad):
    torch = torch_mod()
    rng = np.random.default_rng(d * 7 + n_tok)
    x = rng.standard_normal((n_tok, d + ld_pad)).astype(np.float32)
    x[:, : min(3, d)] *= 20
    if dtype == "bf16":
        xs = synth.f32_to_bf16_bits(x)
        H_ex = oracle.hessian(xs[:, :d], "bf16")
    elif dtype == "f16":
        xs = x.astype(np.float16).view(np.uint16)
        H_ex = oracle.hessian(x.astype(np.float16)[:, :d].astype(np.float64), "f64")
    else:
        xs = x
        H_ex = oracle.hessian(x[:, :d], "f32")
    Xd = to_dev(xs, dtype)[:, :d]
    H = torch.zeros(d, d, device="cuda")
    gq().hessian_accumulate(H, Xd)
    H1 = H.cpu().numpy().astype(np.float64)
    rel = rel_fro(H1, H_ex)
    log(f"HESSIAN d={d} n={n_tok} {dtype} ld+{ld_pad}: rel_fro={rel:.3e}")
    assert rel <= H_TOL
    assert rel <= 1e-5  # products are exact; only fp32 summation order differs
    assert np.array_equal(H1, H1.T)
    # determinism and accumulation across batches
    H2 = torch.zeros(d, d, device="cuda")
    gq().hessian_accumulate(H2, Xd)
    assert torch.equal(H, H2)
    if n_tok >= 2:
        H3 = torch.zeros(d, d, device="cuda")
        gq().hessian_accumulate(H3, Xd[: n_tok // 2])
        gq().hessian_accumulate(H3, Xd[n_tok // 2:])
        assert rel_fro(H3.cpu().numpy().astype(np.float64), H_ex) <= 1e-5


def test_hessian_of_hadamard_columns_is_exact():
    """±1 inputs: every partial sum is an exact integer in fp32."""
    torch = torch_mod()
    X = synth.hadamard_rows(1024, 384)
    H = torch.zeros(384, 384, device="cuda")
    gq().hessian_accumulate(H, to_dev(synth.f32_to_bf16_bits(X), "bf16"))
    assert np.array_equal(H.cpu().numpy(), 2 * 1024 * np.eye(384, dtype=np.float32))


# ---------------------------------------------------------------- prepare (fed the oracle's H)
@pytest.mark.parametrize("d,act", [(256, False), (320, True), (1000, False), (700, True), (64, False), (5, True),
                                   # several super-panels of far tasks, ragged end
                                   (2100, False), (3072, True)])
def test_prepare_matches_oracle(d, act):
    torch = torch_mod()
    rng = np.random.default_rng(d)
    x = rng.standard_normal((max(4 * d, 64), d))
    x[:, rng.choice(d, max(1, d // 100), replace=False)] *= 15
    x[:, d // 3] = 0.0  # a dead channel
    H_ex = oracle.hessian(x.astype(np.float32), "f32")
    H32 = H_ex.astype(np.float32).astype(np.float64)
    p, op = params_of(synth.WORKLOADS["llama7b-attn"], act_order=act)
    Hd_dev = torch.from_numpy(H32.astype(np.float32)).cuda()
    prep = gq().prepare_hinv(Hd_dev, p)
    torch.cuda.synchronize()
    perm = prep.perm.cpu().numpy().astype(np.int64)
    ora = oracle.prepare(H32, op.percdamp, act, perm=perm if act else None)
    if act:
        from parity_utils import check_perm
        ndiff = check_perm(perm, H32)
        log(f"PREPARE d={d}: perm positions differing from the oracle's own sort: {ndiff}")
    U = prep.U.cpu().numpy().astype(np.float64)
    Hd = Hd_dev.cpu().numpy().astype(np.float64)
    urel = rel_fro(U, ora["U"])
    hrel = rel_fro(Hd, ora["Hd"])
    inv_err = np.abs(U.T @ U @ ora["Hd"] - np.eye(d)).max()
    log(f"PREPARE d={d} act={act}: U rel_fro={urel:.3e} Hd rel_fro={hrel:.3e} |UᵀU·H_d − I|max={inv_err:.3e}")
    assert urel <= U_TOL and hrel <= 1e-6
    assert np.array_equal(Hd, Hd.T)
    assert np.all(np.tril(U, -1) == 0) and np.all(np.diag(U) > 0)
    assert np.array_equal(prep.dead.cpu().numpy().astype(bool), ora["dead"])
    assert inv_err < 1e-3


def test_prepare_reports_not_positive_definite():
    torch = torch_mod()
    g = gq()
    p = g.GPTQParams()
    for H in (-np.eye(100), np.diag(np.r_[np.ones(50), -5.0, np.ones(49)])):
        Hd = torch.from_numpy(H.astype(np.float32)).cuda()
        with pytest.raises(g.NotPositiveDefinite) as e:
            g.prepare_hinv(Hd, g.GPTQParams(percdamp=0.0))
        assert 0 <= e.value.pivot < 100
    # NaN in the Hessian is caught by the factorization
    H = np.eye(64, dtype=np.float32)
    H[10, 3] = H[3, 10] = np.nan
    with pytest.raises(g.NotPositiveDefinite):
        g.prepare_hinv(torch.from_numpy(H).cuda(), p)


# ---------------------------------------------------------------- sweep (fed the oracle's U)
@pytest.mark.parametrize("m,d,bits,g", [(300, 512, 4, 128), (64, 300, 3, 128), (129, 256, 4, 64),
                                        (100, 384, 2, 32), (70, 520, 4, 256), (33, 200, 4, -1),
                                        (65, 256, 8, 128),
                                        # >= 4096 rows: four-wave workgroups of 16-lane rows
                                        # (ragged last workgroup and super-block included)
                                        (4096, 640, 4, 128), (4100, 1000, 3, 64),
                                        # several super-blocks, ragged last one included
                                        (200, 2100, 4, 128), (96, 1536, 3, 64), (130, 1800, 4, 32),
                                        # degenerate shapes: one row, one column, a 9-column row group
                                        (1, 300, 4, 128), (7, 1, 4, -1), (2, 9, 3, -1)])
def test_sweep_matches_oracle_given_oracle_factor(m, d, bits, g):
    rng = np.random.default_rng(m * d + bits)
    x = rng.standard_normal((max(4 * d, 16), d))
    x[:, rng.choice(d, min(3, d), replace=False)] *= 20
    H_ex = oracle.hessian(x, "f64")
    W = (rng.standard_normal((m, d)) * 0.02).astype(np.float32)
    gp, op = params_of(synth.WORKLOADS["llama7b-attn"], bits=bits, group_size=g)
    prep = oracle.prepare(H_ex, op.percdamp)
    gpu = run_gpu(W, "f32", None, None, gp, H_in=H_ex, U_in=prep["U"])
    compare_layer(gpu, W, "f32", H_ex, op, label=f"sweep m={m} d={d} b={bits} g={g}",
                  check_h=False, check_u=False)


# ---------------------------------------------------------------- whole layer
CASES = {
    "tiny-256": synth.WORKLOADS["tiny-256"],
    "attn@512x1024": synth.WORKLOADS["llama7b-attn"].scaled(d_out=512, d_in=1024, n_tok=16384),
    "up-actorder@640x512": synth.WORKLOADS["llama7b-up"].scaled(d_out=640, d_in=512, n_tok=8192,
                                                                 act_order=True),
    "down-3bit@256x1000": synth.WORKLOADS["llama7b-down"].scaled(d_out=256, d_in=1000, n_tok=8192),
    "70b-actorder@384x768": synth.WORKLOADS["llama70b-mlp"].scaled(d_out=384, d_in=768, n_tok=8192),
    "attn@256x2560": synth.WORKLOADS["llama7b-attn"].scaled(d_out=256, d_in=2560, n_tok=8192),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_matches_oracle(name):
    wl = CASES[name]
    W, X = _inputs(wl)
    gp, op = params_of(wl)
    log(f"CASE {name}: {wl.describe()}")
    gpu = run_gpu(W, wl.w_dtype, X, wl.x_dtype, gp)
    H_ex = oracle.hessian(X, wl.x_dtype)
    compare_layer(gpu, W, wl.w_dtype, H_ex, op, label=name)


@pytest.mark.parametrize("kw", [dict(group_size=64), dict(group_size=32, bits=3),
                                dict(group_size=256), dict(group_size=-1), dict(sym=True),
                                dict(bits=2), dict(bits=8), dict(sym=True, act_order=True)])
def test_layer_variants(kw):
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=200, d_in=640, n_tok=4096)
    W, X = _inputs(wl)
    gp, op = params_of(wl, **kw)
    gpu = run_gpu(W, wl.w_dtype, X, wl.x_dtype, gp)
    compare_layer(gpu, W, wl.w_dtype, oracle.hessian(X, wl.x_dtype), op, label=str(kw))


def test_dead_channels():
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=128, d_in=384, n_tok=2048)
    W, X = _inputs(wl)
    X = X.copy()
    X[:, [5, 130, 383]] = 0
    for act in (False, True):
        gp, op = params_of(wl, act_order=act)
        gpu = run_gpu(W, wl.w_dtype, X, wl.x_dtype, gp)
        assert gpu["dead"].nonzero()[0].tolist() == [5, 130, 383]
        assert np.all(gpu["what"][:, [5, 130, 383]] == 0)
        compare_layer(gpu, W, wl.w_dtype, oracle.hessian(X, wl.x_dtype), op, label=f"dead act={act}")


def test_scaled_identity_hessian_gives_rtn_codes():
    """H = cI (Hadamard columns): U is diagonal, so there is no compensation and
    the codes are RTN's, up to decisions the oracle's own pre-round value puts
    within 1e-4 code units of a rounding boundary (bf16 grids make near-exact
    ties common; the kernel rounds w·(1/s) + z in fp32)."""
    d, m = 512, 96
    X = synth.f32_to_bf16_bits(synth.hadamard_rows(1024, d))
    W = synth.f32_to_bf16_bits(np.random.default_rng(3).standard_normal((m, d)).astype(np.float32) * 0.02)
    W64 = synth.to_f64(W, "bf16")
    for act in (False, True):
        gp, op = params_of(synth.WORKLOADS["llama7b-attn"], act_order=act)
        gpu = run_gpu(W, "bf16", X, "bf16", gp)
        assert np.count_nonzero(np.triu(gpu["U"], 1)) == 0
        if act:
            assert gpu["perm"].tolist() == list(range(d))
        q, S, Z, what = oracle.rtn_grouped(W64, 4, 128)
        zraw = np.stack([-W64[:, c0:c0 + 128].min(1) / S[:, i] for i, c0 in enumerate(range(0, d, 128))], 1)
        zd = gpu["zeros"] != Z.astype(np.uint8)
        assert np.all(np.abs(np.abs(zraw[zd] - np.floor(zraw[zd])) - 0.5) <= 1e-4)
        Zg = np.repeat(gpu["zeros"].astype(np.float64), 128, axis=1)[:, :d]
        v = W64 / np.repeat(S, 128, axis=1)[:, :d] + Zg
        qq = np.clip(np.rint(v), 0, 15)
        diff = gpu["codes"] != qq
        near = np.abs(np.abs(v - np.floor(v)) - 0.5) <= 1e-4
        log(f"RTN act={act}: zero flips {int(zd.sum())}, code flips {int(diff.sum())} of {diff.size}")
        assert np.all(near[diff]) and np.all(np.abs(gpu["codes"][diff] - qq[diff]) == 1)
        assert diff.mean() <= 1e-3
        np.testing.assert_allclose(gpu["scales"], S, rtol=1e-6)


def test_determinism():
    wl = CASES["attn@512x1024"].scaled(d_out=256, n_tok=8192, act_order=True)
    W, X = _inputs(wl)
    gp, _ = params_of(wl)
    a = run_gpu(W, wl.w_dtype, X, wl.x_dtype, gp)
    b = run_gpu(W, wl.w_dtype, X, wl.x_dtype, gp)
    for k in ("H", "U", "perm", "qweight", "scales", "zeros", "what", "row_loss"):
        assert np.array_equal(a[k], b[k]), k


def test_prepare_repeated_with_reused_workspace():
    """Regression: every panel launch has many workgroups that each read the
    panel's diagonal block; repeated calls on one workspace must agree
    bitwise and match the oracle (d = 2048: 32 panels, up to 31 workgroups)."""
    torch = torch_mod()
    g = gq()
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=64, d_in=2048, n_tok=8192)
    X = synth.make_activations(wl)
    H_ex = oracle.hessian(X, "bf16")
    p = g.GPTQParams()
    ws = torch.empty(g.workspace_bytes(1, 0, 2048, 0, p), dtype=torch.uint8, device="cuda")
    H0 = torch.from_numpy(H_ex.astype(np.float32)).cuda()
    Us = []
    for _ in range(4):
        H = H0.clone()
        Us.append(g.prepare_hinv(H, p, ws=ws).U.cpu().numpy())
    for U in Us[1:]:
        assert np.array_equal(U, Us[0])
    ora = oracle.prepare(H_ex.astype(np.float32).astype(np.float64), p.percdamp)
    assert rel_fro(Us[0].astype(np.float64), ora["U"]) <= U_TOL
