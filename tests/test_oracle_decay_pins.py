"""Pins of the decayed-state oracle (oracle/decay.py) against what the pages
and the mathematics fix, independently of the oracle's own code:

* the page's illustration ("Efficient attention variants", sec. 7.1):
  gamma = 0.99 and a record 100 steps back weigh about 0.366
  (tests/golden/retnet_decay.txt);
* gamma = 1 gives the plain causal linear attention of sec. 5 (the pinned
  oracle.linear_attention);
* closed forms: constant keys and values give a geometric series; one
  impulse key with normalisation gives gamma^t (1 - gamma) / (1 - gamma^(t+1)),
  which fails if z is not decayed;
* the explicit weight form and the token recurrence (independent algorithms)
  agree, normalised or not, with an initial state;
* decode chain, split prefill and sampled rows agree with the recurrence;
* per-head gammas act on their own heads only; normalised outputs stay in
  the range of the values.

A planted mistake (decay after the write, decay of the read, an exponent off
by one, z left undecayed) fails at least one pin (test_pins_catch_mistakes).
"""

import numpy as np
import pytest

from oracle import decay as dec
from oracle import linear_attention as ora
from tests.golden import load

TOL = 1e-12


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _impulse(n, lag_gamma):
    """d = d_v = 1, identity features: k_0 = v_0 = 1, every later k, v = 0,
    q = 1 everywhere; o_t (unnormalised) is the weight of record 0 at lag t."""
    q = np.ones((n, 1))
    k = np.zeros((n, 1)); k[0] = 1.0
    v = np.zeros((n, 1)); v[0] = 1.0
    return q, k, v


def test_page_illustration_gamma_099_lag_100():
    g = load("retnet_decay.txt")
    lag = int(g["lag"])
    q, k, v = _impulse(lag + 1, g["gamma"])
    o_rec, _, _ = dec.recurrent_decay(q, k, v, g["gamma"], phi="identity", normalize=False)
    o_exp = dec.explicit_decay(q, k, v, g["gamma"], phi="identity", normalize=False)
    w = o_rec[lag, 0]
    assert round(w, 3) == g["weight"]
    assert abs(w - g["gamma"] ** lag) < TOL
    assert abs(o_exp[lag, 0] - w) < TOL
    # every lag, not only the printed one
    np.testing.assert_allclose(o_rec[:, 0], g["gamma"] ** np.arange(lag + 1), rtol=0, atol=TOL)


@pytest.mark.parametrize("phi", ["elu1", "identity"])
def test_gamma_one_is_plain_linear_attention(phi):
    q, k, v = _rand((2, 3, 40, 5), 1), _rand((2, 3, 40, 5), 2), _rand((2, 3, 40, 4), 3)
    if phi == "identity":  # positive features keep the denominator away from zero
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    ref, S_ref, z_ref = ora.recurrent_attention(q, k, v, phi=phi)
    out, S, z = dec.recurrent_decay(q, k, v, np.ones(3), phi=phi)
    np.testing.assert_allclose(out, ref, rtol=0, atol=TOL)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=TOL)
    np.testing.assert_allclose(z, z_ref, rtol=0, atol=TOL)
    # unnormalised with gamma = 1: phi(q_t)^T S_t of the plain recurrence
    raw = dec.explicit_decay(q, k, v, 1.0, phi=phi, normalize=False)
    fq = ora.feature_map(phi, q)
    fk = ora.feature_map(phi, k)
    plain = np.tril(fq @ np.swapaxes(fk, -1, -2)) @ v
    np.testing.assert_allclose(raw, plain, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gamma", [0.5, 0.9, 0.99])
def test_geometric_series(gamma):
    n = 50
    q = np.ones((n, 1)); k = np.ones((n, 1)); v = np.ones((n, 1))
    t = np.arange(n)
    o, S, z = dec.recurrent_decay(q, k, v, gamma, phi="identity", normalize=False)
    geo = (1 - gamma ** (t + 1)) / (1 - gamma)
    np.testing.assert_allclose(o[:, 0], geo, rtol=1e-13)
    assert abs(S[0, 0] - geo[-1]) < 1e-12 and abs(z[0] - geo[-1]) < 1e-12
    on, _, _ = dec.recurrent_decay(q, k, v, gamma, phi="identity")  # constant V: the mean is 1
    np.testing.assert_allclose(on[:, 0], 1.0, rtol=0, atol=TOL)


@pytest.mark.parametrize("gamma", [0.5, 0.9])
def test_normalised_impulse_decays_the_denominator(gamma):
    """k_0 = v_0 = 1, later k_t = 1 with v_t = 0: o_t = gamma^t / sum_{j<=t} gamma^j."""
    n = 30
    q = np.ones((n, 1)); k = np.ones((n, 1)); v = np.zeros((n, 1)); v[0] = 1.0
    t = np.arange(n)
    o, _, _ = dec.recurrent_decay(q, k, v, gamma, phi="identity")
    closed = gamma ** t * (1 - gamma) / (1 - gamma ** (t + 1))
    np.testing.assert_allclose(o[:, 0], closed, rtol=1e-12)
    oe = dec.explicit_decay(q, k, v, gamma, phi="identity")
    np.testing.assert_allclose(oe[:, 0], closed, rtol=1e-12)


@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("phi", ["elu1", "identity"])
def test_explicit_equals_recurrent_with_state(phi, normalize):
    B, H, N, d, dv = 2, 3, 37, 6, 5
    q, k, v = _rand((B, H, N, d), 4, 0.5), _rand((B, H, N, d), 5, 0.5), _rand((B, H, N, dv), 6)
    if phi == "identity":
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    gamma = np.array([0.5, 0.9, 0.999])
    r = d
    S0 = np.abs(_rand((B, H, r, dv), 7))
    z0 = np.abs(_rand((B, H, r), 8)) + 1.0
    o_rec, S, z = dec.recurrent_decay(q, k, v, gamma, phi=phi, normalize=normalize, S0=S0, z0=z0)
    o_exp = dec.explicit_decay(q, k, v, gamma, phi=phi, normalize=normalize, S0=S0, z0=z0)
    np.testing.assert_allclose(o_exp, o_rec, rtol=1e-11, atol=1e-12)
    # final state: the decayed sum written out
    fk = ora.feature_map(phi, k)
    w = gamma[None, :, None] ** (N - 1 - np.arange(N))[None, None, :]       # [1, H, N]
    S_def = np.einsum("bhn,bhnr,bhnc->bhrc", np.broadcast_to(w, (B, H, N)), fk, v) + \
        gamma[None, :, None, None] ** N * S0
    np.testing.assert_allclose(S, S_def, rtol=1e-12, atol=1e-12)


def test_decode_chain_and_split_prefill():
    B, H, N, d, dv = 1, 2, 25, 4, 3
    q, k, v = _rand((B, H, N, d), 9), _rand((B, H, N, d), 10), _rand((B, H, N, dv), 11)
    gamma = np.array([0.8, 0.95])
    ref, S_ref, z_ref = dec.recurrent_decay(q, k, v, gamma)
    S = np.zeros((B, H, d, dv)); z = np.zeros((B, H, d))
    for t in range(N):
        o, S, z = dec.decode_step_decay(S, z, q[:, :, t], k[:, :, t], v[:, :, t], gamma)
        np.testing.assert_allclose(o, ref[:, :, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)
    cut = 11
    o1, S1, z1 = dec.recurrent_decay(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], gamma)
    o2, S2, z2 = dec.recurrent_decay(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], gamma, S0=S1, z0=z1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), ref, rtol=1e-12, atol=1e-12)
    o2e = dec.explicit_decay(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], gamma, S0=S1, z0=z1)
    np.testing.assert_allclose(o2e, ref[:, :, cut:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("normalize", [True, False])
def test_sampled_rows_and_head_independence(normalize):
    H, N, d, dv = 3, 60, 5, 4
    q, k, v = _rand((H, N, d), 12, 0.5), _rand((H, N, d), 13, 0.5), _rand((H, N, dv), 14)
    gamma = np.array([0.3, 0.9, 1.0])
    full, _, _ = dec.recurrent_decay(q, k, v, gamma, normalize=normalize)
    for h in range(H):
        rows = [0, 1, 17, 59]
        got = dec.causal_rows_decay(q[h], k[h], v[h], rows, gamma[h], normalize=normalize)
        np.testing.assert_allclose(got, full[h, rows], rtol=1e-12, atol=1e-12)
        alone, _, _ = dec.recurrent_decay(q[h], k[h], v[h], gamma[h], normalize=normalize)
        np.testing.assert_allclose(alone, full[h], rtol=0, atol=TOL)


def test_normalised_output_is_a_weighted_mean():
    N = 80
    q, k, v = _rand((N, 8), 15, 0.4), _rand((N, 8), 16, 0.4), _rand((N, 3), 17)
    o, _, _ = dec.recurrent_decay(q, k, v, 0.7)
    for t in range(N):
        assert np.all(o[t] >= v[: t + 1].min(axis=0) - 1e-12)
        assert np.all(o[t] <= v[: t + 1].max(axis=0) + 1e-12)


def _mutant(kind):
    """A copy of the recurrence with one plausible mistake planted (used only
    to check that the pins above would catch it)."""
    def run(q, k, v, gamma, normalize=True):
        q = np.asarray(q, float); k = np.asarray(k, float); v = np.asarray(v, float)
        n = q.shape[0]
        S = np.zeros((q.shape[1], v.shape[1])); z = np.zeros(q.shape[1])
        out = np.empty((n, v.shape[1]))
        for t in range(n):
            if kind == "decay_after_write":
                S = gamma * (S + np.outer(k[t], v[t])); z = gamma * (z + k[t])
            else:
                S = gamma * S + np.outer(k[t], v[t])
                z = (z + k[t]) if kind == "z_not_decayed" else gamma * z + k[t]
            num = q[t] @ S
            if kind == "decay_read":
                num = gamma * num
            out[t] = num / (q[t] @ z) if normalize else num
        return out
    return run


@pytest.mark.parametrize("kind", ["decay_after_write", "decay_read", "z_not_decayed"])
def test_pins_catch_mistakes(kind):
    bad = _mutant(kind)
    g = load("retnet_decay.txt")
    q, k, v = _impulse(101, g["gamma"])
    page_ok = round(bad(q, k, v, g["gamma"], normalize=False)[100, 0], 3) == g["weight"] and \
        abs(bad(q, k, v, g["gamma"], normalize=False)[100, 0] - g["gamma"] ** 100) < TOL
    n = 30
    q2 = np.ones((n, 1)); k2 = np.ones((n, 1)); v2 = np.zeros((n, 1)); v2[0] = 1.0
    t = np.arange(n)
    closed = 0.5 ** t * 0.5 / (1 - 0.5 ** (t + 1))
    impulse_ok = np.allclose(bad(q2, k2, v2, 0.5)[:, 0], closed, rtol=1e-12)
    assert not (page_ok and impulse_ok), f"mistake {kind} passes every pin"
