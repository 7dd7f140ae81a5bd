"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs, at sizes the oracle finishes in seconds that span
several 128-wide tiles/blocks and ragged tails."""
import numpy as np
import pytest

import oracle
import synth
from parity_utils import (compare_layer, gq, log, params_of, rel_fro, run_gpu, to_dev,
                          torch_mod, H_TOL, HINV_TOL, U_TOL)

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


@pytest.mark.parametrize("d,n_tok,dtype,pad", [(1024, 5000, "bf16", 0), (100, 3000, "bf16", 0),
                                              (96, 2000, "f32", 0), (256, 4096, "f16", 8),
                                              (512, 0, "bf16", 0)])
def test_hessian_set_equals_zero_then_accumulate(d, n_tok, dtype, pad):
    """gptq_hessian (H = 2·XᵀX, H not read) gives bitwise what
    gptq_hessian_accumulate gives on a zeroed H, on the fast bf16/fp16 path,
    the generic path (d not a multiple of 8), the fp32 path and with no
    tokens (H becomes zeros whatever it held)."""
    torch = torch_mod()
    g = gq()
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    rng = np.random.default_rng(d + n_tok)
    x = torch.from_numpy(rng.standard_normal((max(n_tok, 1), d + pad)).astype(np.float32)).to(tdt).cuda()
    X = x[:n_tok, :d]
    H1 = torch.full((d, d), 7.0, device="cuda")       # stale contents: must not be read
    H2 = torch.zeros(d, d, device="cuda")
    g.hessian(H1, X)
    g.hessian_accumulate(H2, X)
    torch.cuda.synchronize()
    assert torch.equal(H1, H2)
    if n_tok == 0:
        assert not torch.any(H1)


def test_hessian_of_hadamard_columns_is_exact():
    """±1 inputs: every partial sum is an exact integer in fp32."""
    torch = torch_mod()
    X = synth.hadamard_rows(1024, 384)
    H = torch.zeros(384, 384, device="cuda")
    gq().hessian_accumulate(H, to_dev(synth.f32_to_bf16_bits(X), "bf16"))
    assert np.array_equal(H.cpu().numpy(), 2 * 1024 * np.eye(384, dtype=np.float32))


# ---------------------------------------------------------------- prepare (fed the oracle's H)
@pytest.mark.parametrize("d,act,mean", [(256, False, 0), (320, True, 0), (1000, False, 0), (700, True, 0),
                                        (64, False, 0), (5, True, 0),
                                        # several super-panels of far tasks, ragged end
                                        (2100, False, 0), (3072, True, 0),
                                        # a shared channel mean: the leading panel runs in fp64
                                        (1000, False, 2.0), (1500, True, 1.0), (130, False, 3.0)])
def test_prepare_matches_oracle(d, act, mean):
    torch = torch_mod()
    rng = np.random.default_rng(d)
    x = rng.standard_normal((max(4 * d, 64), d)) + mean
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
        ndiff = check_perm(perm, H32, H32)
        log(f"PREPARE d={d}: perm positions differing from the oracle's own sort: {ndiff}")
    U = prep.U.cpu().numpy().astype(np.float64)
    Hd = Hd_dev.cpu().numpy().astype(np.float64)
    urel = rel_fro(U, ora["U"])
    hrel = rel_fro(Hd, ora["Hd"])
    inv_err = np.abs(U.T @ U @ ora["Hd"] - np.eye(d)).max()
    hinv_rel = rel_fro(U.T @ U, ora["Hinv"])
    log(f"PREPARE d={d} act={act} mean={mean}: U rel_fro={urel:.3e} Hinv rel_fro={hinv_rel:.3e} "
        f"Hd rel_fro={hrel:.3e} |UᵀU·H_d − I|max={inv_err:.3e}")
    assert urel <= U_TOL and hrel <= 1e-6 and hinv_rel <= HINV_TOL
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


@pytest.mark.parametrize("kw", [dict(group_size=1024), dict(group_size=512), dict(group_size=-1),
                                dict(group_size=128, act_order=True), dict(group_size=64, bits=3)])
def test_layer_wide_rows(kw):
    """Rows of four and a half 512-column super-blocks (2304 columns): the
    update after each super-block reaches every column to its right, the
    last super-block and block are ragged, and groups of 1024 start in one
    super-block and end in the next, so the columns their parameters read
    must be current at the group start."""
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=96, d_in=2304, n_tok=4096)
    W, X = _inputs(wl)
    gp, op = params_of(wl, **kw)
    log(f"CASE wide rows {kw}: {wl.describe()}")
    gpu = run_gpu(W, wl.w_dtype, X, wl.x_dtype, gp)
    compare_layer(gpu, W, wl.w_dtype, oracle.hessian(X, wl.x_dtype), op, label=f"wide rows {kw}")


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


def test_dead_group_and_dead_ties_under_act_order():
    """A whole 128-column group of dead channels is a constant (all-zero)
    group: s = 1, z = 0, codes 0, Ŵ = 0.  Under act-order the dead channels
    all have diagonal 1 after the fix, so their order is the index order
    (ties go to the lower index), checked exactly by check_perm."""
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=96, d_in=512, n_tok=4096)
    W, X = _inputs(wl)
    X = X.copy()
    dead = list(range(128, 256)) + [3, 301, 302, 511]
    X[:, dead] = 0
    # small live channels so the dead ones (diagonal 1 after the fix) sort among them
    X[:, 400:420] = synth.f32_to_bf16_bits(
        synth.bf16_bits_to_f32(X[:, 400:420]) * np.float32(1.0 / 512))
    H_ex = oracle.hessian(X, wl.x_dtype)
    for act in (False, True):
        gp, op = params_of(wl, act_order=act)
        gpu = run_gpu(W, wl.w_dtype, X, wl.x_dtype, gp)
        assert gpu["dead"].nonzero()[0].tolist() == sorted(dead)
        assert np.all(gpu["what"][:, dead] == 0)
        if not act:   # group 1 is the dead group: constant zero
            assert np.all(gpu["scales"][:, 1] == 1.0) and np.all(gpu["zeros"][:, 1] == 0)
            assert np.all(gpu["codes"][:, 128:256] == 0)
        else:
            pos = {c: i for i, c in enumerate(gpu["perm"].tolist())}
            order = sorted(dead, key=lambda c: pos[c])
            assert order == sorted(dead), "dead channels (equal diagonals) out of index order"
        compare_layer(gpu, W, wl.w_dtype, H_ex, op, label=f"dead group act={act}")


def test_one_signed_groups_clamp_the_zero_point():
    """Rows shifted to one sign: a group whose minimum is above 0 has
    −min/s < 0, so z clamps to 0 (and the top codes saturate); a group whose
    maximum is below 0 clamps z to 2ᵇ−1 (Group Quantization listing)."""
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=120, d_in=640, n_tok=4096)
    W, X = _inputs(wl)
    Wf = synth.bf16_bits_to_f32(W).copy()
    Wf[:40] = np.abs(Wf[:40]) + np.float32(0.2)
    Wf[40:80] = -np.abs(Wf[40:80]) - np.float32(0.2)
    W = synth.f32_to_bf16_bits(Wf)
    for bits in (4, 3):
        gp, op = params_of(wl, bits=bits)
        gpu = run_gpu(W, wl.w_dtype, X, wl.x_dtype, gp)
        maxq = (1 << bits) - 1
        assert np.mean(gpu["zeros"][:40] == 0) > 0.9
        assert np.mean(gpu["zeros"][40:80] == maxq) > 0.9
        compare_layer(gpu, W, wl.w_dtype, oracle.hessian(X, wl.x_dtype), op, label=f"one-signed b={bits}")


def test_constant_groups_reconstruct_exactly():
    """H = cI (Hadamard inputs: no compensation) and rows whose groups are
    constant c: s = |c| (1 when c = 0), and every value is reconstructed
    exactly (the constant-group reading of the quantizer)."""
    d, m = 384, 64
    X = synth.f32_to_bf16_bits(synth.hadamard_rows(1024, d))
    rng = np.random.default_rng(11)
    consts = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        rng.choice([0.0, 0.05, -0.03, 0.125, -0.3], size=(m, 3)).astype(np.float32)))
    Wf = np.repeat(consts, 128, axis=1).astype(np.float32)
    W = synth.f32_to_bf16_bits(Wf)
    for act in (False, True):
        gp, op = params_of(synth.WORKLOADS["llama7b-attn"], act_order=act)
        gpu = run_gpu(W, "bf16", X, "bf16", gp)
        want_s = np.where(consts == 0, 1.0, np.abs(consts))
        np.testing.assert_array_equal(gpu["scales"], want_s.astype(np.float32))
        assert np.array_equal(gpu["what"].astype(np.float32), Wf)
        compare_layer(gpu, W, "bf16", oracle.hessian(X, "bf16"), op, label=f"constant groups act={act}")


def test_stalled_panel_wait_is_reported():
    """Every flag wait in the factorization's panel is bounded; a wave whose
    wait runs out marks the call, which then returns GPTQ_ERR_INTERNAL (never
    a made-up pivot).  The bound is forced down from the host, so every
    kernel still runs to its end."""
    import os
    torch = torch_mod()
    g = gq()
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=64, d_in=1024, n_tok=4096)
    H_ex = oracle.hessian(synth.make_activations(wl), "bf16")
    H = torch.from_numpy(H_ex.astype(np.float32)).cuda()
    os.environ["GPTQ_PANEL_SPIN_LIMIT"] = "0"
    try:
        with pytest.raises(g.GPTQError) as e:
            g.prepare_hinv(H.clone(), g.GPTQParams())
        assert e.value.code == g._native.ERR_INTERNAL
        assert not isinstance(e.value, g.NotPositiveDefinite)
    finally:
        del os.environ["GPTQ_PANEL_SPIN_LIMIT"]
    prep = g.prepare_hinv(H.clone(), g.GPTQParams())   # back to normal on the same process
    ora = oracle.prepare(H_ex.astype(np.float32).astype(np.float64), 0.01)
    assert rel_fro(prep.U.cpu().numpy().astype(np.float64), ora["U"]) <= U_TOL


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


@pytest.mark.parametrize("act", [False, True])
def test_async_prepare_matches_prepare(act):
    """gptq_prepare_hinv_async queues the same work without waiting: the
    factor, H_d and the quantization queued right behind it are bitwise those
    of the synchronous call, and the status words decode to OK."""
    torch = torch_mod()
    g = gq()
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=192, d_in=1500, n_tok=6000, act_order=act)
    W, X = _inputs(wl)
    p = g.GPTQParams(act_order=act)
    H0 = torch.from_numpy(oracle.hessian(X, "bf16").astype(np.float32)).cuda()
    Wd = to_dev(W, wl.w_dtype)
    Ha, Hs = H0.clone(), H0.clone()
    pa = g.prepare_hinv(Ha, p, sync=False)
    qa = g.quantize_layer(Wd, pa, p)
    pa.check()
    ps = g.prepare_hinv(Hs, p)
    qs = g.quantize_layer(Wd, ps, p)
    torch.cuda.synchronize()
    assert pa.status is None
    for a, b in [(Ha, Hs), (pa.U, ps.U), (pa.perm, ps.perm), (pa.dead, ps.dead), (qa.qweight, qs.qweight),
                 (qa.scales, qs.scales), (qa.zeros, qs.zeros), (qa.W_hat, qs.W_hat)]:
        assert torch.equal(a, b)


def test_async_prepare_reports_not_positive_definite():
    torch = torch_mod()
    g = gq()
    H = torch.from_numpy(np.diag(np.r_[np.ones(50), -5.0, np.ones(49)]).astype(np.float32)).cuda()
    prep = g.prepare_hinv(H, g.GPTQParams(percdamp=0.0), sync=False)
    with pytest.raises(g.NotPositiveDefinite) as e:
        prep.check()
    assert 0 <= e.value.pivot < 100


# ---------------------------------------------------------------- independent layers
_INDEP = [  # (d_out, d_in, n_tok, w dtype, x dtype)
    (96, 256, 2048, "bf16", "bf16"), (200, 384, 4096, "f32", "bf16"), (64, 640, 3000, "bf16", "f16"),
    (130, 1000, 2500, "bf16", "bf16"), (33, 130, 777, "f32", "f32"), (300, 512, 1024, "bf16", "bf16"),
    (8, 64, 100, "bf16", "bf16"), (40, 2100, 4200, "bf16", "bf16"), (128, 256, 512, "f16", "f16"),
]


def _indep_inputs(torch, k, m, d, n_tok, wdt, xdt):
    rng = np.random.default_rng(1000 + k)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    W = torch.from_numpy((rng.standard_normal((m, d)) * 0.02).astype(np.float32)).to(tdt[wdt]).cuda()
    x = rng.standard_normal((n_tok, d)).astype(np.float32)
    x[:, rng.choice(d, max(1, d // 64), replace=False)] *= 12.0
    if k % 3 == 1:
        x += 1.5   # a shared channel mean: the fp64 leading panel runs for this layer
    return W, torch.from_numpy(x).to(tdt[xdt]).cuda()


@pytest.mark.parametrize("act", [False, True])
def test_independent_layers_match_separate_calls(act):
    """Nine layers with their own inputs, shapes and dtypes run concurrently
    (more layers than the library's streams): every output is bitwise what
    hessian_accumulate + prepare_hinv + quantize_layer give for that layer
    alone, and one layer is checked against the oracle as well."""
    torch = torch_mod()
    g = gq()
    p = g.GPTQParams(act_order=act)
    layers = [_indep_inputs(torch, k, *spec) for k, spec in enumerate(_INDEP)]
    res = g.quantize_independent(layers, p)
    torch.cuda.synchronize()
    for k, ((W, X), (q, prep, Hd)) in enumerate(zip(layers, res)):
        d = W.shape[1]
        H = torch.zeros(d, d, dtype=torch.float32, device="cuda")
        g.hessian_accumulate(H, X)
        pr = g.prepare_hinv(H, p)
        qq = g.quantize_layer(W, pr, p)
        torch.cuda.synchronize()
        pairs = [(Hd, H, "H_d"), (prep.U, pr.U, "U"), (prep.dead, pr.dead, "dead"),
                 (q.qweight, qq.qweight, "qweight"), (q.scales, qq.scales, "scales"),
                 (q.zeros, qq.zeros, "zeros"), (q.W_hat, qq.W_hat, "W_hat"),
                 (q.g_idx, qq.g_idx, "g_idx"), (q.row_loss, qq.row_loss, "row_loss")]
        if act:
            pairs.append((prep.perm, pr.perm, "perm"))
        for a, b, name in pairs:
            assert torch.equal(a, b), (k, _INDEP[k], name)
    # one layer against the oracle (the separate path's own parity tests cover the rest)
    W, X = layers[3]
    q, prep, _ = res[3]
    H_ex = oracle.hessian(X.float().cpu().numpy(), "f32")
    ora = oracle.prepare(H_ex, p.percdamp, act, perm=prep.perm.cpu().numpy().astype(np.int64) if act else None)
    assert rel_fro(prep.U.cpu().numpy().astype(np.float64), ora["U"]) <= U_TOL
    log(f"INDEPENDENT act={act}: {len(layers)} layers bitwise equal to separate calls")


def test_independent_layers_report_a_failed_factorization():
    """A layer whose Hessian holds NaN (natural order) fails its factorization:
    the call raises for it and the other layers' outputs are still those of
    separate calls."""
    torch = torch_mod()
    g = gq()
    p = g.GPTQParams()
    layers = [_indep_inputs(torch, k, *_INDEP[k]) for k in (0, 3, 5)]
    Xbad = layers[1][1].clone()
    Xbad[7, 11] = float("nan")
    layers[1] = (layers[1][0], Xbad)
    with pytest.raises(g.NotPositiveDefinite) as e:
        g.quantize_independent(layers, p)
    assert e.value.statuses == [g._native.OK, g._native.ERR_NOT_SPD, g._native.OK]
    torch.cuda.synchronize()
    for k in (0, 2):
        (W, X), (q, prep, Hd) = layers[k], e.value.results[k]
        d = W.shape[1]
        H = torch.zeros(d, d, dtype=torch.float32, device="cuda")
        g.hessian_accumulate(H, X)
        qq = g.quantize_layer(W, g.prepare_hinv(H, p), p)
        torch.cuda.synchronize()
        assert torch.equal(q.qweight, qq.qweight) and torch.equal(q.scales, qq.scales)


@pytest.mark.parametrize("bits,g,d", [(3, 128, 333), (3, 128, 1024), (2, 64, 200), (4, 128, 257),
                                      (8, 128, 300), (3, -1, 97)])
def test_export_dense_codes_and_half_metadata(bits, g, d):
    """gptq_export: the dense b-bit stream equals the oracle's packing of the
    same codes bit for bit, and the 16-bit scales/zeros are the IEEE half
    (nearest-even) of the fp32 values."""
    torch = torch_mod()
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=70, d_in=d, n_tok=2048)
    W, X = _inputs(wl)
    gp, op = params_of(wl, bits=bits, group_size=g)
    gpu = run_gpu(W, wl.w_dtype, X, wl.x_dtype, gp)
    dev = torch.device("cuda")
    q = gq().Quantized(torch.from_numpy(gpu["qweight"].view(np.int32)).to(dev),
                       torch.from_numpy(gpu["scales"]).to(dev), torch.from_numpy(gpu["zeros"]).to(dev),
                       None, None, None)
    ex = gq().export(q, gp, d)
    torch.cuda.synchronize()
    dense = ex.qweight.cpu().numpy().view(np.uint32)
    assert np.array_equal(dense, oracle.pack_dense(gpu["codes"], bits))
    assert np.array_equal(oracle.unpack_dense(dense, d, bits), gpu["codes"])
    assert np.array_equal(ex.scales_f16.cpu().numpy().view(np.uint16), oracle.fp16_bits(gpu["scales"]))
    assert np.array_equal(ex.zeros_f16.cpu().numpy().view(np.uint16), oracle.fp16_bits(gpu["zeros"]))
    bpw = 32 * (dense.shape[1] + ex.scales_f16.shape[1]) / d
    assert bpw == oracle.stored_bits_per_weight(d, bits, g)


@pytest.mark.parametrize("act", [False, True])
def test_quantize_layers_shares_one_factor(act):
    """Three layers fed the same X (one H, one factor), one call: each layer
    matches the oracle, and bit for bit the single-layer call."""
    torch = torch_mod()
    g = gq()
    base = synth.WORKLOADS["llama7b-attn"].scaled(d_out=200, d_in=640, n_tok=4096, act_order=act)
    X = synth.make_activations(base)
    H_ex = oracle.hessian(X, base.x_dtype)
    shapes = [(200, "bf16", 1002), (96, "f32", 1003), (130, "bf16", 1004)]
    Ws = []
    for m, dt, seed in shapes:
        wl = base.scaled(d_out=m, w_dtype=dt, seed=seed)
        Ws.append((synth.make_weights(wl), dt))
    gp, op = params_of(base)
    H = torch.zeros(640, 640, device="cuda")
    g.hessian_accumulate(H, to_dev(X, base.x_dtype))
    H_gpu = H.cpu().numpy().astype(np.float64)
    prep = g.prepare_hinv(H, gp)
    outs = g.quantize_layers([to_dev(W, dt) for W, dt in Ws], prep, gp)
    torch.cuda.synchronize()
    for (W, dt), o in zip(Ws, outs):
        one = g.quantize_layer(to_dev(W, dt), prep, gp)
        torch.cuda.synchronize()
        for k in ("qweight", "scales", "zeros", "W_hat", "g_idx", "row_loss"):
            assert torch.equal(getattr(o, k), getattr(one, k)), k
        gpu = dict(U=prep.U.cpu().numpy().astype(np.float64), perm=prep.perm.cpu().numpy().astype(np.int64),
                   dead=prep.dead.cpu().numpy().astype(bool), qweight=o.qweight.cpu().numpy().view(np.uint32),
                   scales=o.scales.cpu().numpy(), zeros=o.zeros.cpu().numpy(),
                   what=o.W_hat.cpu().numpy().astype(np.float64), g_idx=o.g_idx.cpu().numpy(),
                   row_loss=o.row_loss.cpu().numpy(), H=H_gpu)
        gpu["codes"] = oracle.unpack_codes(gpu["qweight"], 640)
        compare_layer(gpu, W, dt, H_ex, op, label=f"multi-layer {W.shape} {dt} act={act}",
                      check_h=False, free_run=False)


@pytest.mark.parametrize("m,d,bits,sym", [(64, 96, 3, False), (40, 128, 4, False), (33, 17, 2, False),
                                          (50, 64, 4, True), (9, 1, 3, False), (48, 100, 8, False)])
def test_obq_matches_oracle(m, d, bits, sym):
    """OBQ (greedy order per row) on tiny layers, fed the GPU's own fp32 H:
    the oracle replays every row in follow mode (the GPU's column choice must
    lie within 1e-9 relative of the smallest saliency, a different code
    within 1e-4 of its rounding boundary); both run in fp64."""
    torch = torch_mod()
    g = gq()
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=m, d_in=d, n_tok=max(8 * d, 512))
    W, X = _inputs(wl)
    X = X.copy()
    if d > 8:
        X[:, d // 2] = 0     # a dead channel
    H = torch.zeros(d, d, device="cuda")
    g.hessian_accumulate(H, to_dev(X, wl.x_dtype))
    p = g.GPTQParams(bits=bits, group_size=-1, sym=sym)
    q, order = g.obq_layer(to_dev(W, wl.w_dtype), H, p)
    torch.cuda.synchronize()
    H32 = H.cpu().numpy().astype(np.float64)
    Hf, dead = oracle.dead_fix(H32)
    Hd = Hf + 0.01 * np.mean(np.diag(Hf)) * np.eye(d)
    W64 = synth.to_f64(W, wl.w_dtype)
    W64[:, dead] = 0.0
    codes = (oracle.unpack_codes(q.qweight.cpu().numpy().view(np.uint32), d) if bits <= 4 else
             np.stack([(q.qweight.cpu().numpy().view(np.uint32) >> np.uint32(8 * i)) & 255
                       for i in range(4)], 2).reshape(m, -1)[:, :d].astype(np.uint8))
    gord = order.cpu().numpy().astype(np.int64)
    op = oracle.Params(bits=bits, group_size=-1, sym=sym)
    o = oracle.obq_layer(W64, Hd, op, follow={"order": gord, "q": codes})
    r = o["report"]
    own = oracle.obq_layer(W64, Hd, op)
    same_order = float(np.mean(np.all(own["order"] == gord, axis=1)))
    log(f"OBQ m={m} d={d} b={bits} sym={sym}: order adopted {r.order_allowed} hard {r.order_hard}, "
        f"codes adopted {r.code_allowed} hard {r.code_hard}; rows with the oracle's own order {same_order:.3f}")
    assert r.ok, r.hard_examples[:5]
    assert r.frac_codes_identical >= 0.999
    assert np.all(np.sort(gord, axis=1) == np.arange(d))
    s = q.scales.cpu().numpy()[:, 0]
    assert np.max(np.abs(s - o["s"]) / o["s"]) <= 1e-7
    assert np.array_equal(q.zeros.cpu().numpy()[:, 0], o["z"].astype(np.uint8))
    what = q.W_hat.cpu().numpy()
    rebuilt = s[:, None].astype(np.float32) * (codes.astype(np.float32) - q.zeros.cpu().numpy().astype(np.float32))
    assert np.array_equal(what, rebuilt)
    rl = q.row_loss.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(rl, o["saliency"].sum(1), rtol=1e-5, atol=1e-30)
    e_gpu = oracle.layer_error(W64, what.astype(np.float64), H32)
    e_ora = oracle.layer_error(W64, o["what"], H32)
    assert abs(e_gpu - e_ora) <= 0.01 * max(e_ora, 1e-12)
    if bits <= 4 and not sym and d > 8:   # the comparison the comparator exists for (reported)
        gp = g.GPTQParams(bits=bits, group_size=-1)
        prep = g.prepare_hinv(H.clone(), gp)
        gq_ = g.quantize_layer(to_dev(W, wl.w_dtype), prep, gp)
        e_gptq = oracle.layer_error(W64, gq_.W_hat.cpu().numpy().astype(np.float64), H32)
        e_rtn = oracle.layer_error(W64, oracle.rtn_grouped(W64, bits, -1)[3], H32)
        log(f"OBQ m={m} d={d} b={bits}: layer error OBQ {e_gpu:.4e}, GPTQ {e_gptq:.4e}, RTN {e_rtn:.4e} "
            f"(GPTQ/OBQ {e_gptq / e_gpu:.4f})")


@pytest.mark.parametrize("M,act,bits,g,act_order", [
    (1, "f16", 4, 128, False), (3, "bf16", 4, 128, False), (1, "f16", 3, 128, False),
    (4, "f16", 2, 64, False), (2, "bf16", 8, -1, False), (1, "f16", 4, 128, True),
    (64, "f16", 4, 128, False), (37, "bf16", 3, 128, False), (100, "f16", 4, 128, True)])
def test_w4a16_gemm_matches_oracle(M, act, bits, g, act_order):
    """The exported layer's product with 16-bit activations: Ŵ dequantized as
    (q − z)·s rounded once to the activation format, products exact, fp32
    accumulation within its recursive-summation bound of the exact sum."""
    torch = torch_mod()
    g_ = gq()
    wl = synth.WORKLOADS["llama7b-attn"].scaled(d_out=300, d_in=520, n_tok=4096, act_order=act_order)
    W, X = _inputs(wl)
    gp, _ = params_of(wl, bits=bits, group_size=g)
    Wd = to_dev(W, wl.w_dtype)
    H = torch.zeros(520, 520, device="cuda")
    g_.hessian_accumulate(H, to_dev(X, wl.x_dtype))
    prep = g_.prepare_hinv(H, gp)
    q = g_.quantize_layer(Wd, prep, gp)
    ex = g_.export(q, gp, 520)
    rng = np.random.default_rng(M * 7 + bits)
    a32 = (rng.standard_normal((M, 520)) * 2).astype(np.float32)
    A_bits = a32.astype(np.float16).view(np.uint16) if act == "f16" else synth.f32_to_bf16_bits(a32)
    A = (torch.from_numpy(A_bits.view(np.int16)).view(torch.float16 if act == "f16" else torch.bfloat16)
         .cuda())
    gi = q.g_idx if act_order else None
    C = g_.w4a16_gemm(A, ex, bits, g, g_idx=gi)
    torch.cuda.synchronize()
    qd = ex.qweight.cpu().numpy().view(np.uint32)
    s16 = ex.scales_f16.cpu().numpy().view(np.uint16)
    z16 = ex.zeros_f16.cpu().numpy().view(np.uint16)
    gidx = q.g_idx.cpu().numpy() if act_order else None
    ref = oracle.w4a16.w4a16_matmul(A_bits, act, qd, bits, s16, z16, g, g_idx=gidx)
    Wq = oracle.w4a16.dequantize(qd, bits, 520, s16, z16, g, g_idx=gidx, act=act)
    bound = oracle.w4a16.accumulation_bound(A_bits, act, Wq, 520)
    got = C.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    log(f"W4A16 M={M} {act} b={bits} g={g} act_order={act_order}: max |err| {err.max():.3e}, "
        f"max err/bound {np.max(err / np.maximum(bound, 1e-30)):.3e}")
    assert np.all(err <= bound + 1e-30)


@pytest.mark.parametrize("M,act,bits,K,split", [
    (1, "f16", 4, 4096, True), (3, "bf16", 4, 4000, True), (1, "bf16", 3, 4096, True),
    (64, "f16", 4, 4096, True), (64, "f16", 4, 4096, False), (200, "bf16", 3, 4000, True),
    (17, "f16", 8, 4096, False), (5, "bf16", 2, 4064, True), (40, "bf16", 4, 630, False)])
def test_w4a16_gemm_large_k(M, act, bits, K, split):
    """Long rows (K up to 4096, ragged; 630 leaves a GEMM tail of two 64-deep
    steps after its unrolled loop) and a ragged N: any word stream is a
    valid dense code stream, so the codes are random words; scales are random
    halves and zeros random codes.  With a workspace, products with few tiles
    split K (fixed-order sum of fp32 partials); without one they run unsplit.
    Both stay within the fp32 recursive-summation bound of the exact sum."""
    import ctypes
    torch = torch_mod()
    g_ = gq()
    n = g_._native
    N, g = 1000, 128
    ng = (K + g - 1) // g
    rng = np.random.default_rng(M * 1000 + K + bits)
    rw = (K * bits + 31) // 32
    qd = rng.integers(0, 2**32, size=(N, rw), dtype=np.uint64).astype(np.uint32)
    s16 = (rng.uniform(1e-3, 1e-2, size=(N, ng))).astype(np.float16).view(np.uint16)
    z16 = rng.integers(0, 2**bits, size=(N, ng)).astype(np.float16).view(np.uint16)
    a32 = (rng.standard_normal((M, K)) * 2).astype(np.float32)
    A_bits = a32.astype(np.float16).view(np.uint16) if act == "f16" else synth.f32_to_bf16_bits(a32)
    tdt = torch.float16 if act == "f16" else torch.bfloat16
    A = torch.from_numpy(A_bits.view(np.int16)).view(tdt).cuda()
    q_t = torch.from_numpy(qd.view(np.int32)).cuda()
    s_t = torch.from_numpy(s16.view(np.int16)).view(torch.float16).cuda()
    z_t = torch.from_numpy(z16.view(np.int16)).view(torch.float16).cuda()
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    L = n.lib()
    need = L.gptq_workspace_bytes(n.WS_W4A16, N, K, M, None)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if split else None
    rc = L.gptq_w4a16_gemm(
        ctypes.c_void_p(A.data_ptr()), n.F16 if act == "f16" else n.BF16, M, K, K,
        ctypes.c_void_p(q_t.data_ptr()), bits, ctypes.c_void_p(s_t.data_ptr()),
        ctypes.c_void_p(z_t.data_ptr()), None, g, ng, N, ctypes.c_void_p(C.data_ptr()), N,
        ctypes.c_void_p(ws.data_ptr()) if split else None, need if split else 0,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == n.OK, n.last_error()
    torch.cuda.synchronize()
    ref = oracle.w4a16.w4a16_matmul(A_bits, act, qd, bits, s16, z16, g)
    Wq = oracle.w4a16.dequantize(qd, bits, K, s16, z16, g, act=act)
    bound = oracle.w4a16.accumulation_bound(A_bits, act, Wq, K)
    got = C.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    log(f"W4A16 M={M} K={K} {act} b={bits} split={split} (ws {need} B): max |err| {err.max():.3e}, "
        f"max err/bound {np.max(err / np.maximum(bound, 1e-30)):.3e}")
    assert np.all(err <= bound + 1e-30)
