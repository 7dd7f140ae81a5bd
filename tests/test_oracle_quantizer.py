"""Pins for the oracle's quantizers and packed format (CPU only).

Each test checks the oracle against something other than its own formula:
values printed on the pages, closed forms, or brute force.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import asym_params, asym_quantize, sym_params, sym_quantize

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_example_int8_symmetric_codes():
    """Worked example 1 of "Quantization (INT8, INT4, GPTQ)"."""
    ex = _load("worked_example_int8_symmetric.json")
    w = np.array(ex["w"])
    s, _ = sym_params(np.max(np.abs(w)), ex["bits"])
    assert s == pytest.approx(ex["scale_exact_num"] / ex["scale_exact_den"], rel=1e-15)
    assert round(float(s), 5) == ex["scale_printed"]
    q, what = sym_quantize(w, s, ex["bits"])
    assert q.astype(int).tolist() == ex["q"]
    # the page's w/s line is printed to one decimal (truncated)
    np.testing.assert_allclose(w / s, ex["w_over_s_printed"], atol=0.1)
    # the printed dequantized values use the rounded scale
    _, what_printed = sym_quantize(w, ex["scale_printed"], ex["bits"])
    half_ulp = 0.5 * 10.0 ** -np.array(ex["w_hat_printed_decimals"]) + 1e-12
    assert np.all(np.abs(what_printed - ex["w_hat_printed"]) <= half_ulp)
    # "≈" error line: within the page's rounding of the exact-scale errors
    np.testing.assert_allclose(np.abs(w - what), ex["abs_err_printed_approx"], atol=5e-4)


def test_worked_example_through_unsigned_storage():
    """Symmetric codes stored unsigned with offset 2ᵇ⁻¹ give the same values."""
    ex = _load("worked_example_int8_symmetric.json")
    w = np.array(ex["w"])
    s, z = sym_params(np.max(np.abs(w)), 8)
    _, qu, what = asym_quantize(w, s, z, 8)
    assert (qu - z).astype(int).tolist() == ex["q"]
    np.testing.assert_allclose(what, s * np.array(ex["q"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_affine_endpoints_closed_form(bits):
    """Deriving the scale and zero-point: x_min = s(q_min − z), x_max = s(q_max − z)
    when −x_min/s is an integer; the extremes map to codes 0 and 2ᵇ−1."""
    maxq = (1 << bits) - 1
    for z0 in [0, 1, maxq // 2, maxq]:
        step = 0.0078125  # power of two: every quantity below is exact
        mn, mx = -z0 * step, (maxq - z0) * step
        s, z, zraw = asym_params(mn, mx, bits)
        assert s == step and z == z0 and zraw == z0
        assert mn == s * (0 - z) and mx == s * (maxq - z)
        _, q, what = asym_quantize(np.array([mn, mx]), s, z, bits)
        assert q.tolist() == [0, maxq]
        assert what.tolist() == [mn, mx]


@pytest.mark.parametrize("c", [0.37, -0.21, 0.0])
def test_constant_group_reconstructs_exactly(c):
    for bits in (3, 4):
        s, z, _ = asym_params(c, c, bits)
        _, q, what = asym_quantize(np.array([c, c]), s, z, bits)
        assert np.all(what == c)
        assert 0 <= z <= (1 << bits) - 1


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_rounding_is_nearest_grid_point(bits, rng):
    """Brute force over the whole grid: the code chosen is the nearest grid
    point (ties aside), z inside the round, clamped at the edges."""
    maxq = (1 << bits) - 1
    for _ in range(50):
        w = rng.normal(size=32) * rng.uniform(0.01, 1)
        s, z, _ = asym_params(w.min(), w.max(), bits)
        v, q, what = asym_quantize(w, s, z, bits)
        grid = s * (np.arange(maxq + 1) - z)
        best = np.argmin(np.abs(w[:, None] - grid[None, :]), axis=1)
        assert np.array_equal(q.astype(int), best)
        inside = (q > 0) & (q < maxq)
        assert np.all(np.abs(w - what)[inside] <= s / 2 * (1 + 1e-12))


def test_zero_is_representable_and_zero_point_rounded(rng):
    """'The zero-point must itself be a valid integer so that 0 maps exactly.'"""
    for bits in (3, 4):
        for _ in range(20):
            w = rng.normal(size=64)
            s, z, _ = asym_params(w.min(), w.max(), bits)
            assert z == np.round(z)
            _, _, what0 = asym_quantize(np.array([0.0]), s, z, bits)
            assert what0[0] == 0.0


def test_rtn_grouped_matches_per_group_brute_force(rng):
    W = rng.normal(size=(6, 300)) * 0.02
    q, S, Z, what = oracle.rtn_grouped(W, 4, 128)
    assert S.shape == (6, 3)
    for gi, (c0, c1) in enumerate([(0, 128), (128, 256), (256, 300)]):
        blk = W[:, c0:c1]
        np.testing.assert_allclose(S[:, gi], (blk.max(1) - blk.min(1)) / 15, rtol=1e-15)
        grid = S[:, gi:gi + 1, None] * (np.arange(16)[None, None, :] - Z[:, gi:gi + 1, None])
        best = np.argmin(np.abs(blk[:, :, None] - grid), axis=2)
        assert np.array_equal(q[:, c0:c1], best)


def test_pack_known_words():
    """Eight 4-bit codes per 32-bit word, column 8k+i in nibble i."""
    q = np.array([[0, 1, 2, 3, 4, 5, 6, 7, 15, 0, 0, 0, 0, 0, 0, 9, 3]], dtype=np.uint8)
    w = oracle.pack_codes(q)
    assert w.shape == (1, 3)
    assert int(w[0, 0]) == 0x76543210
    assert int(w[0, 1]) == 0x9000000F
    assert int(w[0, 2]) == 0x3


def test_pack_roundtrip(rng):
    for d in (1, 7, 8, 9, 129, 4096):
        q = rng.integers(0, 16, size=(5, d)).astype(np.uint8)
        assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(q), d), q)


def test_bit_rate_matches_page():
    ex = _load("bit_rate.json")
    assert oracle.bits_per_weight(ex["bits"], ex["group_size"]) == ex["bits_per_weight"]


@pytest.mark.parametrize("bits", [3, 4])
def test_one_signed_group_clamps_zero_point_and_codes(bits):
    """Group Quantization listing: zero = round(−min/scale) clamped to [0, 2ᵇ−1],
    codes clamped to the same range; the range is the group's own min/max.
    A group with min > 0 has −min/s < 0, so z = 0 and every value above
    s·(2ᵇ−1) saturates at the top code; a group with max < 0 has z = 2ᵇ−1 and
    values below saturate at code 0.  Without the zero-point clamp the codes
    would spread over the whole grid instead."""
    maxq = (1 << bits) - 1
    step = 0.0078125
    w_pos = np.array([maxq, maxq + 1.25, maxq + 3, 2 * maxq]) * step     # min = maxq·step > 0
    s, z, zraw = asym_params(w_pos.min(), w_pos.max(), bits)
    assert s == step and zraw == -maxq and z == 0
    v, q, what = asym_quantize(w_pos, s, z, bits)
    assert q.tolist() == [maxq] * 4
    assert np.all(what == maxq * step)
    w_neg = -w_pos[::-1]                                                # max = −maxq·step < 0
    s, z, zraw = asym_params(w_neg.min(), w_neg.max(), bits)
    assert s == step and zraw == 2 * maxq and z == maxq
    _, q, what = asym_quantize(w_neg, s, z, bits)
    assert q.tolist() == [0] * 4
    assert np.all(what == -maxq * step)
    # the unclamped zero-point would have placed the codes across the grid
    _, q_free, _ = asym_quantize(w_pos, step, -maxq, bits)
    assert q_free.tolist() != [maxq] * 4


def test_dense_3bit_words_by_hand():
    """Dense 3-bit storage: 32 codes in three 32-bit words, code c at bits
    3c..3c+2 of the row's little-endian bit stream (codes 10 and 21 straddle
    a word boundary).  Words written out by hand."""
    def one(c, v, d=32):
        q = np.zeros((1, d), dtype=np.uint8)
        q[0, c] = v
        return [int(x) for x in oracle.pack_dense(q, 3)[0]]
    assert one(0, 5) == [0x5, 0, 0]
    assert one(10, 1) == [0x40000000, 0, 0]
    assert one(10, 2) == [0x80000000, 0, 0]
    assert one(10, 4) == [0, 0x1, 0]
    assert one(21, 5) == [0, 0x80000000, 0x2]
    assert one(31, 7) == [0, 0, 0xE0000000]
    assert [int(x) for x in oracle.pack_dense(np.full((1, 32), 7), 3)[0]] == [0xFFFFFFFF] * 3
    # a ragged row is padded to whole words: 33 codes need 99 bits -> 4 words
    assert oracle.pack_dense(np.full((2, 33), 7), 3).shape == (2, 4)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_dense_pack_roundtrip_and_4bit_layout(bits, rng):
    for d in (1, 7, 31, 32, 33, 96, 130):
        q = rng.integers(0, 1 << bits, size=(3, d)).astype(np.uint8)
        w = oracle.pack_dense(q, bits)
        assert w.shape == (3, (d * bits + 31) // 32)
        assert np.array_equal(oracle.unpack_dense(w, d, bits), q)
        if bits == 4:   # the nibble container is the dense 4-bit layout
            assert np.array_equal(w, oracle.pack_codes(q))


def test_stored_bit_rate_matches_page_accounting():
    """b + (16 + 16)/g bits per weight ("GPTQ: Mathematical Foundations ...",
    Quantization Formats and Group Size): 4.25 at b = 4, g = 128 (the page's
    figure, in the golden fixture) and 3.25 at b = 3 when d fills whole
    words, counted from the exported buffers' sizes."""
    ex = _load("bit_rate.json")
    assert oracle.stored_bits_per_weight(4096, ex["bits"], ex["group_size"]) == ex["bits_per_weight"]
    assert oracle.stored_bits_per_weight(11008, 3, 128) == 3.25
    assert oracle.stored_bits_per_weight(4096, 3, 128) == oracle.bits_per_weight(3, 128) == 3.25
    assert oracle.stored_bits_per_weight(4096, 2, 64) == 2.5


def test_fp16_metadata_rounding():
    """16-bit scale and zero: IEEE half, round to nearest even (bits checked
    against the half-precision encoding written out by hand)."""
    assert oracle.fp16_bits([1.0, -2.0, 0.5, 65504.0, 7.0]).tolist() == [0x3C00, 0xC000, 0x3800, 0x7BFF, 0x4700]
    # 1 + 2^-11 is halfway between 1 and 1 + 2^-10: ties to even (1.0)
    assert int(oracle.fp16_bits(1.0 + 2.0 ** -11)) == 0x3C00
    assert int(oracle.fp16_bits(1.0 + 3 * 2.0 ** -11)) == 0x3C02
