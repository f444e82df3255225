"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: values the
pages print for a worked example (fixtures in tests/golden/), closed forms,
invariants of a normalised non-negative weighting, agreement of the two
independent algorithms (explicit N x N weights vs token recurrence), and a
Monte Carlo check of the FAVOR+ expectation identity.  A plausible mistake in
the oracle (a dropped diagonal term, a transposed state, a wrong sign in the
FAVOR+ exponent, a missing 1/sqrt(r) or d**(1/4) factor, reading before
writing in the recurrence) fails at least one of them.
"""

import numpy as np
import pytest

from oracle import linear_attention as ora
from kernelized_linear_attention_elu_amd import synth
from tests.golden import load


# ---------------------------------------------------------------- worked example

@pytest.fixture(scope="module")
def ex():
    g = load("worked_example.txt")
    g["phi_q"] = np.tile(g["phi_q3"], (3, 1))   # phi(q1), phi(q2) are free; use [1,2]
    return g


def test_worked_example_recurrent_state_and_output(ex):
    out, S, z = ora.recurrent_attention(ex["phi_q"], ex["phi_k"], ex["v"], phi="identity")
    np.testing.assert_array_equal(S, ex["S3"])
    np.testing.assert_array_equal(z, ex["z3"])
    np.testing.assert_allclose(out[2], ex["o3"], rtol=0, atol=1e-15)


def test_worked_example_explicit_weights_and_output(ex):
    out = ora.explicit_attention(ex["phi_q"], ex["phi_k"], ex["v"], phi="identity", causal=True)
    np.testing.assert_allclose(out[2], ex["o3"], rtol=0, atol=1e-15)
    # one-hot values make each output row equal to that row's normalised weights
    w = ora.explicit_attention(ex["phi_q"], ex["phi_k"], np.eye(3), phi="identity", causal=True)
    np.testing.assert_allclose(w[2], ex["weight3"], rtol=0, atol=1e-15)
    # row 3's raw similarities are proportional to the printed weights
    np.testing.assert_allclose(w[2] / w[2][0], ex["similarity3"], rtol=0, atol=1e-14)
    # causal rows only see the past: row 1 puts all weight on token 1
    np.testing.assert_allclose(w[0], [1.0, 0.0, 0.0], atol=0)


def test_worked_example_decode_chain(ex):
    S = np.zeros((2, 2))
    z = np.zeros(2)
    for t in range(3):
        o, S, z = ora.decode_step(S, z, ex["phi_q"][t], ex["phi_k"][t], ex["v"][t], phi="identity")
    np.testing.assert_array_equal(S, ex["S3"])
    np.testing.assert_array_equal(z, ex["z3"])
    np.testing.assert_allclose(o, ex["o3"], rtol=0, atol=1e-15)


def test_worked_example_noncausal_state(ex):
    out, S, z = ora.noncausal_attention(ex["phi_q"], ex["phi_k"], ex["v"], phi="identity")
    np.testing.assert_array_equal(S, ex["S3"])
    np.testing.assert_array_equal(z, ex["z3"])
    # every query sees all three tokens; query 3 reproduces o3
    np.testing.assert_allclose(out[2], ex["o3"], rtol=0, atol=1e-15)


def test_worked_example_sampled_row(ex):
    row = ora.causal_rows(ex["phi_q"], ex["phi_k"], ex["v"], [2], phi="identity")
    np.testing.assert_allclose(row[0], ex["o3"], rtol=0, atol=1e-15)


def test_same_key_written_twice_reads_the_mean():
    g = load("same_key_twice.txt")
    k = g["phi_k"].reshape(2, 1)
    v = g["v"].reshape(2, 1)
    q = np.full((2, 1), g["phi_q"])
    out, S, z = ora.recurrent_attention(q, k, v, phi="identity")
    assert S[0, 0] == g["unnormalised_readout"]      # additive state, no normaliser
    assert out[1, 0] == g["normalised_readout"]      # normalised read-out: the mean
    assert out[0, 0] == 2.0
    dense = ora.explicit_attention(q, k, v, phi="identity")
    assert dense[1, 0] == g["normalised_readout"]


# ---------------------------------------------------------------- invariants on several inputs
#
# Three invariants of the definitions, each checked on a set of inputs: the
# explicit masked form equals the token recurrence; changing keys and values
# from token t0 on leaves every earlier output unchanged ("Efficient
# attention variants", sec. 11's self-test); the non-causal explicit form
# equals its reassociated product (sec. 4).  One input is the small case of
# the hands-on section (sec. 10): its seed, shapes, perturbation and reported
# error level are fixture data (tests/golden/numpy_check.txt); the others are
# a random small case and a case with a long tail of negative inputs.

def _inputs(name):
    """(q, k, v, t0, k_add, v_add, err_level) for the named case."""
    if name == "hands_on_sec10":
        g = load("numpy_check.txt")
        rng = np.random.default_rng(int(g["seed"]))
        n, d, dv = int(g["N"]), int(g["d"]), int(g["dv"])
        q, k, v = (rng.normal(size=(n, w)) for w in (d, d, dv))
        return q, k, v, int(g["perturb_from"]), g["perturb_k_add"], g["perturb_v_add"], g["reported_max_abs_error"]
    rng = np.random.default_rng(7 if name == "random_small" else 11)
    n, d = (40, 8) if name == "random_small" else (64, 16)
    q, k, v = (rng.normal(size=(n, d)) for _ in range(3))
    if name == "negative_tail":
        q -= 3.0
        k -= 3.0
    return q, k, v, n // 3, 0.75, -4.0, None


CASES = ["hands_on_sec10", "random_small", "negative_tail"]


@pytest.mark.parametrize("name", CASES)
def test_explicit_equals_recurrent(name):
    q, k, v, _, _, _, err_level = _inputs(name)
    dense = ora.explicit_attention(q, k, v)
    rec, _, _ = ora.recurrent_attention(q, k, v)
    np.testing.assert_allclose(dense, rec, rtol=1e-12, atol=1e-12)
    if err_level is not None:
        # the same order of magnitude as the rounding-level difference the page reports
        assert np.max(np.abs(dense - rec)) < 100 * err_level


@pytest.mark.parametrize("name", CASES)
def test_future_tokens_leave_earlier_rows_unchanged(name):
    q, k, v, t0, k_add, v_add, _ = _inputs(name)
    k2, v2 = k.copy(), v.copy()
    k2[t0:] += k_add
    v2[t0:] += v_add
    a, _, _ = ora.recurrent_attention(q, k, v)
    b, _, _ = ora.recurrent_attention(q, k2, v2)
    np.testing.assert_array_equal(a[:t0], b[:t0])
    assert np.max(np.abs(a[t0:] - b[t0:])) > 1e-3   # the change does reach the later rows
    np.testing.assert_allclose(ora.explicit_attention(q, k, v)[:t0], ora.explicit_attention(q, k2, v2)[:t0],
                               rtol=0, atol=1e-15)


@pytest.mark.parametrize("name", CASES)
def test_noncausal_explicit_equals_reassociated(name):
    q, k, v, _, _, _, _ = _inputs(name)
    dense = ora.explicit_attention(q, k, v, causal=False)
    reas, _, _ = ora.noncausal_attention(q, k, v)
    np.testing.assert_allclose(dense, reas, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- feature maps

def test_elu1_closed_form():
    x = np.array([0.0, 1.5, np.log(0.5), -30.0, 1e-12, -1e-12, 7.0])
    f = ora.phi_elu1(x)
    assert f[0] == 1.0                       # continuous at 0, value 1
    assert f[1] == 2.5                       # x + 1 for x > 0
    assert abs(f[2] - 0.5) < 1e-16           # e^x for x <= 0
    assert 0 < f[3] < 1e-12                  # tends to 0, stays positive
    assert abs(f[4] - 1.0) < 1e-11 and abs(f[5] - 1.0) < 1e-11
    assert f[6] == 8.0
    grid = np.linspace(-50, 50, 20001)
    fg = ora.phi_elu1(grid)
    assert np.all(fg > 0)
    assert np.all(np.diff(fg) > 0)           # strictly increasing


def test_favor_zero_input_gives_inverse_sqrt_r():
    omega = synth.draw_omega(32, 8, seed=5)
    f = ora.phi_favor(np.zeros(8), omega)
    np.testing.assert_allclose(f, np.full(32, 1 / np.sqrt(32)), rtol=1e-15)


@pytest.mark.parametrize("orthogonal", [True, False])
def test_favor_unbiased_kernel_estimate(orthogonal):
    """E over random rows of phi(q).phi(k) = exp(q.k / sqrt(d)) (Performer
    identity); checked by Monte Carlo within 4 standard errors."""
    d, r, trials = 8, 16, 2000
    rng = np.random.default_rng(123)
    q = rng.normal(size=d) * 0.6
    k = rng.normal(size=d) * 0.6
    target = np.exp(q @ k / np.sqrt(d))
    est = np.empty(trials)
    for s in range(trials):
        if orthogonal:
            om = synth.draw_omega(r, d, seed=1000 + s)
        else:
            om = np.random.default_rng(1000 + s).standard_normal((r, d))
        est[s] = ora.phi_favor(q, om) @ ora.phi_favor(k, om)
    se = est.std(ddof=1) / np.sqrt(trials)
    assert abs(est.mean() - target) < 4 * se
    # and it is not the unscaled kernel exp(q.k) (a dropped d**(1/4) would match that)
    assert abs(est.mean() - np.exp(q @ k)) > 4 * se


def test_favor_features_positive():
    omega = synth.draw_omega(256, 64)
    u = np.random.default_rng(3).normal(size=(100, 64)) * 64 ** -0.25
    f = ora.phi_favor(u, omega)
    assert f.shape == (100, 256)
    assert np.all(f > 0)


# ---------------------------------------------------------------- forms agree

@pytest.mark.parametrize("phi", ["elu1", "favor"])
def test_explicit_equals_recurrent_tiny_workload(phi):
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, std=w.std, io=w.io)
    omega = synth.draw_omega(256, w.d) if phi == "favor" else None
    dense = ora.explicit_attention(q, k, v, phi=phi, omega=omega)
    rec, _, _ = ora.recurrent_attention(q, k, v, phi=phi, omega=omega)
    np.testing.assert_allclose(dense, rec, rtol=1e-12, atol=1e-12)


def test_last_causal_row_equals_noncausal_row():
    q, k, v = synth.draw_qkv(2, 3, 40, 16, 8, std=1.0, io="f32")
    c, S, z = ora.recurrent_attention(q, k, v)
    nc, S2, z2 = ora.noncausal_attention(q, k, v)
    np.testing.assert_allclose(c[..., -1, :], nc[..., -1, :], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, S2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, z2, rtol=1e-12, atol=1e-12)


def test_decode_chain_equals_recurrence():
    q, k, v = synth.draw_qkv(1, 2, 30, 8, 5, std=1.0, io="f32")
    rec, S_N, z_N = ora.recurrent_attention(q, k, v)
    S = np.zeros((1, 2, 8, 5))
    z = np.zeros((1, 2, 8))
    for t in range(30):
        o, S, z = ora.decode_step(S, z, q[:, :, t], k[:, :, t], v[:, :, t])
        np.testing.assert_allclose(o, rec[:, :, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, S_N, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, z_N, rtol=1e-12, atol=1e-12)


def test_split_prefill_equals_one_shot():
    q, k, v = synth.draw_qkv(1, 2, 50, 8, 6, std=1.0, io="f32")
    full, S_full, z_full = ora.recurrent_attention(q, k, v)
    n1 = 23
    a, S1, z1 = ora.recurrent_attention(q[..., :n1, :], k[..., :n1, :], v[..., :n1, :])
    b, S2, z2 = ora.recurrent_attention(q[..., n1:, :], k[..., n1:, :], v[..., n1:, :], S0=S1, z0=z1)
    np.testing.assert_allclose(np.concatenate([a, b], axis=-2), full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S_full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z2, z_full, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("phi", ["elu1", "favor"])
def test_sampled_rows_match_full_forms(phi):
    q, k, v = synth.draw_qkv(1, 1, 64, 16, 8, std=0.7, io="f32")
    omega = synth.draw_omega(32, 16) if phi == "favor" else None
    rec, S, z = ora.recurrent_attention(q, k, v, phi=phi, omega=omega)
    rows = [0, 1, 17, 63]
    got = ora.causal_rows(q[0, 0], k[0, 0], v[0, 0], rows, phi=phi, omega=omega)
    np.testing.assert_allclose(got, rec[0, 0, rows], rtol=1e-12, atol=1e-13)
    nc, _, _ = ora.noncausal_attention(q, k, v, phi=phi, omega=omega)
    got = ora.noncausal_rows(q[0, 0], k[0, 0], v[0, 0], rows, phi=phi, omega=omega)
    np.testing.assert_allclose(got, nc[0, 0, rows], rtol=1e-12, atol=1e-13)
    # with an initial state: rows after a split equal the one-shot rows
    n1 = 20
    _, S1, z1 = ora.recurrent_attention(q[..., :n1, :], k[..., :n1, :], v[..., :n1, :], phi=phi, omega=omega)
    got = ora.causal_rows(q[0, 0, n1:], k[0, 0, n1:], v[0, 0, n1:], [0, 5, 43], phi=phi, omega=omega,
                          S0=S1[0, 0], z0=z1[0, 0])
    np.testing.assert_allclose(got, rec[0, 0, [n1, n1 + 5, n1 + 43]], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- invariants

def test_constant_values_give_constant_output():
    q, k, _ = synth.draw_qkv(1, 2, 33, 8, 4, std=1.0, io="f32")
    v = np.broadcast_to(np.array([0.5, -2.0, 3.0, 7.25]), (1, 2, 33, 4))
    for out in (ora.recurrent_attention(q, k, v)[0],
                ora.explicit_attention(q, k, v),
                ora.noncausal_attention(q, k, v)[0]):
        np.testing.assert_allclose(out, v, rtol=1e-14, atol=1e-14)


def test_outputs_are_convex_combinations_of_past_values():
    q, k, v = synth.draw_qkv(1, 1, 60, 8, 3, std=1.0, io="f32")
    out, _, _ = ora.recurrent_attention(q, k, v)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 0], rtol=1e-15, atol=1e-15)   # o_1 = v_1
    for t in range(60):
        lo = v[0, 0, : t + 1].min(axis=0)
        hi = v[0, 0, : t + 1].max(axis=0)
        assert np.all(out[0, 0, t] >= lo - 1e-12) and np.all(out[0, 0, t] <= hi + 1e-12)


def test_scale_and_affine_invariance():
    q, k, v = synth.draw_qkv(1, 1, 25, 6, 4, std=1.0, io="f32")
    q, k, v = (x.astype(np.float64) for x in (q, k, v))
    fq, fk = np.abs(q) + 0.1, np.abs(k) + 0.1    # positive features through the identity map
    base, _, _ = ora.recurrent_attention(fq, fk, v, phi="identity")
    scaled, _, _ = ora.recurrent_attention(fq, 3.7 * fk, v, phi="identity")
    np.testing.assert_allclose(scaled, base, rtol=1e-13, atol=1e-13)
    aff, _, _ = ora.recurrent_attention(fq, fk, -2.5 * v + 1.25, phi="identity")
    np.testing.assert_allclose(aff, -2.5 * base + 1.25, rtol=1e-13, atol=1e-13)


def test_heads_are_independent():
    q, k, v = synth.draw_qkv(2, 3, 20, 8, 4, std=1.0, io="f32")
    full, _, _ = ora.recurrent_attention(q, k, v)
    one, _, _ = ora.recurrent_attention(q[1, 2], k[1, 2], v[1, 2])
    np.testing.assert_array_equal(full[1, 2], one)


def test_noncausal_with_initial_state_equals_all_keys():
    """A state carried in from earlier keys acts as those keys: non-causal
    attention over all keys equals non-causal attention over the later keys
    started from the earlier keys' recurrent state."""
    q, k, v = synth.draw_qkv(1, 2, 30, 8, 5, std=1.0, io="f32")
    n1 = 12
    _, S1, z1 = ora.recurrent_attention(q[..., :n1, :], k[..., :n1, :], v[..., :n1, :])
    full, S_all, z_all = ora.noncausal_attention(q, k, v)
    part, S_p, z_p = ora.noncausal_attention(q, k[..., n1:, :], v[..., n1:, :], S0=S1, z0=z1)
    np.testing.assert_allclose(part, full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_p, S_all, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z_p, z_all, rtol=1e-12, atol=1e-12)
