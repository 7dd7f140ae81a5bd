"""The no-allocation Hessian entry point (gptq_hessian_accumulate_noalloc),
for callers that cannot allocate device memory: called through the C ABI and
checked against the workspace entry point and the fp64 oracle on two calls
in a row, the second with a smaller input, and refused beyond its limit."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from parity_utils import gq, log, rel_fro, to_dev, torch_mod

pytestmark = pytest.mark.gpu


def _noalloc(H, X):
    n = gq()._native
    L = n.lib()
    torch = torch_mod()
    return L.gptq_hessian_accumulate_noalloc(
        ctypes.c_void_p(H.data_ptr()), X.shape[1], ctypes.c_void_p(X.data_ptr()),
        n.BF16 if X.dtype == torch.bfloat16 else n.F32, X.shape[0], X.stride(0),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_hessian_matches_workspace_entry_point():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    n = gq()._native
    # the larger input first, then a smaller one: the scratch keeps the first
    # call's contents, which must not leak into the second
    for d, n_tok, seed in ((4096, 16384, 1), (1000, 3000, 2)):
        wl = synth.WORKLOADS["llama7b-down"].scaled(d_out=8, d_in=d, n_tok=n_tok, seed=seed)
        Xb = synth.make_activations(wl)
        X = to_dev(Xb, "bf16")
        H0 = torch.zeros(d, d, device="cuda")
        assert _noalloc(H0, X) == n.OK, n.last_error()
        H1 = torch.zeros(d, d, device="cuda")
        gq().hessian_accumulate(H1, X)
        torch.cuda.synchronize()
        a = H0.cpu().numpy().astype(np.float64)
        b = H1.cpu().numpy().astype(np.float64)
        H_ex = oracle.hessian(Xb, "bf16")
        ra, rb, rab = rel_fro(a, H_ex), rel_fro(b, H_ex), rel_fro(a, b)
        log(f"NOALLOC d={d} n={n_tok}: rel to oracle {ra:.3e} (workspace call {rb:.3e}), to each other {rab:.3e}")
        assert ra <= 1e-5 and rab <= 1e-5
        assert np.array_equal(a, a.T)
        # accumulation over a second batch, as the workspace entry point does
        assert _noalloc(H0, X) == n.OK
        torch.cuda.synchronize()
        assert rel_fro(H0.cpu().numpy().astype(np.float64), 2 * H_ex) <= 1e-5


def test_noalloc_hessian_refuses_sizes_beyond_its_scratch():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    n = gq()._native
    H = torch.zeros(8, 8, device="cuda")
    X = torch.zeros(4, 8, dtype=torch.bfloat16, device="cuda")
    L = n.lib()
    rc = L.gptq_hessian_accumulate_noalloc(ctypes.c_void_p(H.data_ptr()), 4100,
                                           ctypes.c_void_p(X.data_ptr()), n.BF16, 4, 4100, None)
    assert rc == n.ERR_UNSUPPORTED and "4096" in n.last_error()
