"""Parity at the full size of the benchmarked layer (4096 x 4096, 131072
tokens, bf16, 4-bit g128), in the same launch configuration bench.py times.

The oracle computes the exact H (fp64 over all tokens) and its own U; the
sweep, whose rows are independent problems sharing H, is checked on a
sample of rows: the oracle quantizes exactly those rows with the full
factor and follows the GPU's decisions as in the small-size tests.
"""
import time

import numpy as np
import pytest

import oracle
import synth
from parity_utils import compare_layer, log, params_of, rel_fro, run_gpu, torch_mod

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.timeout(900)
def test_full_size_attention_projection():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = synth.WORKLOADS["llama7b-attn"]
    t0 = time.time()
    W = synth.make_weights(wl)
    X = synth.make_activations(wl)
    log(f"FULL inputs generated in {time.time() - t0:.1f}s: W{W.shape} X{X.shape}")
    gp, op = params_of(wl)
    gpu = run_gpu(W, wl.w_dtype, X, wl.x_dtype, gp)
    log(f"FULL gpu done at {time.time() - t0:.1f}s")
    H_ex = oracle.hessian(X, wl.x_dtype, chunk=4096)
    del X
    log(f"FULL oracle H done at {time.time() - t0:.1f}s; H rel_fro={rel_fro(gpu['H'], H_ex):.3e}")
    rows = np.sort(np.random.default_rng(0).choice(wl.d_out, 96, replace=False))
    sub = {k: (v[rows] if k in ("qweight", "scales", "zeros", "what", "row_loss", "codes") else v)
           for k, v in gpu.items()}
    compare_layer(sub, W[rows], wl.w_dtype, H_ex, op, label="full-size attn (96 sampled rows)")
    log(f"FULL compare done at {time.time() - t0:.1f}s")
