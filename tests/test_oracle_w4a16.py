"""Pins for the oracle's dequantize-and-multiply (CPU only).

The FP16xINT4 pipeline of "GPTQ: Mathematical Foundations ...", Inference
Execution and Modern Kernel Architectures: W = (W_int − zero)·scale, then the
product with the activations.  Checked against values worked out by hand,
exactness where the format makes it exact, and the orientation of every
index (transposes, g_idx).
"""
import numpy as np
import pytest

import oracle
from oracle import w4a16


def _h(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def test_dequantize_by_hand():
    """q = 0..15, z = 8, s = 0.5: w = (q − 8)·0.5 = −4 .. 3.5, all exact."""
    q = np.arange(16, dtype=np.uint8)[None, :]
    W = w4a16.dequantize(oracle.pack_dense(q, 4), 4, 16, _h([[0.5]]), _h([[8.0]]), -1)
    assert W.tolist() == [[-4.0 + 0.5 * i for i in range(16)]]


def test_dequantize_rounds_once_to_the_activation_format():
    """(q − z)·s with s = fp16(0.1): the exact product 7·s is not an fp16
    number; it is rounded to nearest even (fp16) or to bf16."""
    s16 = _h([[0.1]])
    s = float(s16.view(np.float16)[0, 0])
    q = np.array([[15]], dtype=np.uint8)
    exact = 7.0 * s
    f16 = w4a16.dequantize(oracle.pack_dense(q, 4), 4, 1, s16, _h([[8.0]]), -1, act="f16")[0, 0]
    bf = w4a16.dequantize(oracle.pack_dense(q, 4), 4, 1, s16, _h([[8.0]]), -1, act="bf16")[0, 0]
    assert f16 != exact and abs(f16 - exact) <= 2.0 ** -11 * abs(exact)
    assert f16 == float(np.float16(exact))
    # bf16 keeps 8 significant bits: the nearest such value to 0.7000...
    cands = [m * 2.0 ** -8 for m in range(128, 256)]
    assert bf == min(cands, key=lambda c: (abs(c - exact), c))


def test_groups_and_g_idx_orientation():
    """Two groups of 4 with different scales; an act-order g_idx that swaps
    them gives the swapped scales, column by column."""
    q = np.full((1, 8), 9, dtype=np.uint8)
    s = _h([[1.0, 2.0]])
    z = _h([[8.0, 8.0]])
    W = w4a16.dequantize(oracle.pack_dense(q, 4), 4, 8, s, z, 4)
    assert W.tolist() == [[1.0] * 4 + [2.0] * 4]
    gi = np.array([1, 1, 1, 1, 0, 0, 0, 0])
    W2 = w4a16.dequantize(oracle.pack_dense(q, 4), 4, 8, s, z, 4, g_idx=gi)
    assert W2.tolist() == [[2.0] * 4 + [1.0] * 4]


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_product_orientation_with_unit_activations(act, rng):
    """A = rows of the identity picks Ŵ's columns: Y[k, n] = Ŵ[n, k]."""
    N, K = 5, 12
    q = rng.integers(0, 8, size=(N, K)).astype(np.uint8)
    s, z = _h(rng.uniform(0.01, 0.1, size=(N, 3))), _h(np.full((N, 3), 4.0))
    eye = np.eye(K, dtype=np.float32)
    A = (eye.astype(np.float16).view(np.uint16) if act == "f16"
         else (eye.view(np.uint32) >> 16).astype(np.uint16))
    Y = w4a16.w4a16_matmul(A, act, oracle.pack_dense(q, 3), 3, s, z, 4)
    W = w4a16.dequantize(oracle.pack_dense(q, 3), 3, K, s, z, 4, act=act)
    assert np.array_equal(Y, W.T)


def test_dequantized_weights_track_the_quantizer(rng):
    """With exactly representable (power-of-two) scales the dequantized fp16
    weights equal the quantizer's own ŵ = s(q − z)."""
    W = rng.normal(size=(4, 256)) * 0.02
    q, S, Z, what = oracle.rtn_grouped(W, 4, 128)
    S2 = 2.0 ** np.round(np.log2(S))
    what2 = S2.repeat(128, 1) * (q.astype(np.float64) - Z.repeat(128, 1))
    Wd = w4a16.dequantize(oracle.pack_dense(q, 4), 4, 256, _h(S2), _h(Z), 128)
    np.testing.assert_array_equal(Wd, what2)
