"""Checks of the seeded input generator (no method arithmetic involved)."""

import numpy as np

from kernelized_linear_attention_elu_amd import synth


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0], dtype=np.float32)
    got = synth.round_to_io(x, "bf16")
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa wins (1.0)
    # 1+3*2^-8 ties between 1+2^-7 and 1+2^-6: even is 1+2^-6
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0], dtype=np.float32))


def test_bf16_bits_roundtrip():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000, dtype=np.float32)
    b = synth.bf16_bits(x)
    v = synth.bf16_values(b)
    np.testing.assert_array_equal(synth.bf16_bits(v), b)
    assert np.max(np.abs(v - x) / np.abs(x)) <= 2 ** -8


def test_qkv_deterministic_and_scaled():
    a = synth.draw_qkv(1, 2, 512, 64, 64)
    b = synth.draw_qkv(1, 2, 512, 64, 64)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    q, k, v = a
    assert q.shape == (1, 2, 512, 64) and v.shape == (1, 2, 512, 64)
    assert abs(q.std() - 64 ** -0.25) < 0.01
    assert not np.array_equal(q, k)


def test_omega_block_orthogonal_rows():
    om = synth.draw_omega(256, 64, seed=1)
    assert om.shape == (256, 64) and om.dtype == np.float32
    for b in range(4):
        blk = om[64 * b: 64 * (b + 1)].astype(np.float64)
        g = blk @ blk.T
        off = g - np.diag(np.diag(g))
        assert np.max(np.abs(off)) < 1e-4 * np.max(np.diag(g))
    sq = np.sum(om.astype(np.float64) ** 2, axis=1)
    assert abs(sq.mean() / 64 - 1) < 0.1          # chi-square(d) row norms
