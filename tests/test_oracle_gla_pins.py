"""Pins of the per-channel gated (GLA form) oracle (oracle/gla.py) against
what the pages and the mathematics fix, independently of its own code:

* all gates one: plain causal linear attention ("Efficient attention
  variants" sec. 5, the pinned oracle.linear_attention);
* the same gate on every channel: the per-token scalar gate (the pinned
  oracle.gated), and through a constant gate the fixed decay figure of
  sec. 7.1 (gamma = 0.99 weighs 0.366 at lag 100, tests/golden/retnet_decay.txt);
* sec. 7.2's reading of the gate: entry f of alpha_t keeps row f of the
  state (key channel f), broadcast over the value columns: with one-hot keys
  and queries and d != d_v, o_t reads the product of channel f's gates only;
* a zero gate on channel f forgets that channel only: outputs through other
  channels are unchanged, channel f restarts;
* the explicit weight form and the token recurrence (independent
  algorithms) agree, normalised or not, with an initial state; decode chain,
  split prefill and sampled rows agree with the recurrence.

A planted mistake (gate on the value columns, gate after the write, the
previous token's gate, z ungated, channels reversed) fails at least one pin
(test_pins_catch_mistakes).
"""

import numpy as np
import pytest

from oracle import gated as gat
from oracle import gla
from oracle import linear_attention as ora
from tests.golden import load

TOL = 1e-12


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _gates(shape, seed):
    """GLA-like gates sigmoid(x)^(1/16), x ~ N(0, 2): values in about (0.6, 1)."""
    x = np.random.default_rng(seed).standard_normal(shape) * 2.0
    return (1.0 / (1.0 + np.exp(-x))) ** (1.0 / 16.0)


@pytest.mark.parametrize("phi", ["elu1", "identity"])
def test_unit_gates_are_plain_linear_attention(phi):
    q, k, v = _rand((2, 3, 30, 5), 1), _rand((2, 3, 30, 5), 2), _rand((2, 3, 30, 4), 3)
    if phi == "identity":
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    al = np.ones((2, 3, 30, 5))
    ref, S_ref, z_ref = ora.recurrent_attention(q, k, v, phi=phi)
    out, S, z = gla.recurrent_gla(q, k, v, al, phi=phi)
    np.testing.assert_allclose(out, ref, rtol=0, atol=TOL)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=TOL)
    np.testing.assert_allclose(z, z_ref, rtol=0, atol=TOL)
    np.testing.assert_allclose(gla.explicit_gla(q, k, v, al, phi=phi), ref, rtol=1e-12, atol=1e-12)


def test_channel_constant_gates_are_the_scalar_gate_and_the_page_figure():
    B, H, N, d, dv = 2, 2, 25, 6, 3
    q, k, v = _rand((B, H, N, d), 4, 0.5), _rand((B, H, N, d), 5, 0.5), _rand((B, H, N, dv), 6)
    a = _gates((B, H, N), 7)
    al = np.repeat(a[..., None], d, axis=-1)
    S0 = np.abs(_rand((B, H, d, dv), 8)); z0 = np.abs(_rand((B, H, d), 9)) + 1.0
    for normalize in (True, False):
        ref, S_ref, z_ref = gat.recurrent_gated(q, k, v, a, normalize=normalize, S0=S0, z0=z0)
        out, S, z = gla.recurrent_gla(q, k, v, al, normalize=normalize, S0=S0, z0=z0)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)
    g = load("retnet_decay.txt")
    n = int(g["lag"]) + 1
    q1 = np.ones((n, 1)); k1 = np.zeros((n, 1)); k1[0] = 1.0; v1 = np.zeros((n, 1)); v1[0] = 1.0
    o, _, _ = gla.recurrent_gla(q1, k1, v1, np.full((n, 1), g["gamma"]), phi="identity", normalize=False)
    assert round(o[-1, 0], 3) == g["weight"]


def test_gate_keeps_key_rows_broadcast_over_values():
    """d = 3 key channels, d_v = 2: write v_0 = (1, 2) under key e_f at t = 0,
    read with q = e_f: o_t = (prod_{l=1..t} alpha_{l,f}) (1, 2)."""
    N, d = 12, 3
    al = _gates((N, d), 10)
    for f in range(d):
        q = np.zeros((N, d)); q[:, f] = 1.0
        k = np.zeros((N, d)); k[0, f] = 1.0
        v = np.zeros((N, 2)); v[0] = (1.0, 2.0)
        o, S, _ = gla.recurrent_gla(q, k, v, al, phi="identity", normalize=False)
        prod = np.concatenate([[1.0], np.cumprod(al[1:, f])])
        np.testing.assert_allclose(o[:, 0], prod, rtol=1e-13, atol=0)
        np.testing.assert_allclose(o[:, 1], 2 * prod, rtol=1e-13, atol=0)
        assert np.all(S[[c for c in range(d) if c != f]] == 0.0)
        oe = gla.explicit_gla(q, k, v, al, phi="identity", normalize=False)
        np.testing.assert_allclose(oe, o, rtol=1e-13, atol=1e-15)


def test_zero_gate_forgets_one_channel():
    """Identity features, positive keys: a zero gate on channel f at t0 leaves
    the other channels' state as without it and restarts channel f."""
    N, d, dv, t0, f = 20, 4, 3, 8, 2
    q, k, v = np.abs(_rand((N, d), 11)) + 0.1, np.abs(_rand((N, d), 12)) + 0.1, _rand((N, dv), 13)
    al = _gates((N, d), 14)
    al0 = al.copy(); al0[t0, f] = 0.0
    _, S, _ = gla.recurrent_gla(q, k, v, al, phi="identity", normalize=False)
    _, S0, _ = gla.recurrent_gla(q, k, v, al0, phi="identity", normalize=False)
    others = [c for c in range(d) if c != f]
    np.testing.assert_allclose(S0[others], S[others], rtol=0, atol=TOL)
    _, Sf, _ = gla.recurrent_gla(q[t0:], k[t0:], v[t0:], al0[t0:], phi="identity", normalize=False)
    np.testing.assert_allclose(S0[f], Sf[f], rtol=1e-12, atol=1e-12)
    oe = gla.explicit_gla(q, k, v, al0, phi="identity", normalize=False)
    o0, _, _ = gla.recurrent_gla(q, k, v, al0, phi="identity", normalize=False)
    np.testing.assert_allclose(oe, o0, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("normalize", [True, False])
def test_explicit_equals_recurrent_with_state(normalize):
    B, H, N, d, dv = 2, 2, 23, 5, 4
    q, k, v = _rand((B, H, N, d), 15, 0.5), _rand((B, H, N, d), 16, 0.5), _rand((B, H, N, dv), 17)
    al = _gates((B, H, N, d), 18)
    S0 = np.abs(_rand((B, H, d, dv), 19)); z0 = np.abs(_rand((B, H, d), 20)) + 1.0
    o_rec, S, z = gla.recurrent_gla(q, k, v, al, normalize=normalize, S0=S0, z0=z0)
    o_exp = gla.explicit_gla(q, k, v, al, normalize=normalize, S0=S0, z0=z0)
    np.testing.assert_allclose(o_exp, o_rec, rtol=1e-11, atol=1e-12)
    # final state written out per channel: sum_j (alpha_{j+1} ... alpha_{N-1}) phi(k_j) v_j^T + (alpha_0 ...) S0
    fk = ora.phi_elu1(k)
    tail = np.flip(np.cumprod(np.flip(al, -2), -2), -2)            # alpha_j ... alpha_{N-1}
    w = np.concatenate([tail[..., 1:, :], np.ones((B, H, 1, d))], axis=-2)
    S_def = np.einsum("bhnr,bhnc->bhrc", w * fk, v) + tail[..., 0, :, None] * S0
    np.testing.assert_allclose(S, S_def, rtol=1e-12, atol=1e-12)


def test_decode_chain_split_prefill_and_rows():
    B, H, N, d, dv = 1, 2, 21, 4, 3
    q, k, v = _rand((B, H, N, d), 21), _rand((B, H, N, d), 22), _rand((B, H, N, dv), 23)
    al = _gates((B, H, N, d), 24)
    al[0, 1, 6, 2] = 0.0
    ref, S_ref, _ = gla.recurrent_gla(q, k, v, al)
    S = np.zeros((B, H, d, dv)); z = np.zeros((B, H, d))
    for t in range(N):
        o, S, z = gla.decode_step_gla(S, z, q[:, :, t], k[:, :, t], v[:, :, t], al[:, :, t])
        np.testing.assert_allclose(o, ref[:, :, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)
    cut = 9
    o1, S1, z1 = gla.recurrent_gla(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], al[:, :, :cut])
    o2, S2, _ = gla.recurrent_gla(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], al[:, :, cut:], S0=S1, z0=z1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S_ref, rtol=1e-12, atol=1e-12)
    for normalize in (True, False):
        full, _, _ = gla.recurrent_gla(q, k, v, al, normalize=normalize)
        for h in range(H):
            rows = [0, 1, 6, 7, 20]
            got = gla.causal_rows_gla(q[0, h], k[0, h], v[0, h], al[0, h], rows, normalize=normalize)
            np.testing.assert_allclose(got, full[0, h, rows], rtol=1e-12, atol=1e-12)


def _mutant(kind):
    """Single-head recurrence with one plausible mistake planted (used only to
    check that the pins above would catch it)."""
    def run(q, k, v, al, normalize=True):
        q = np.asarray(q, float); k = np.asarray(k, float); v = np.asarray(v, float); al = np.asarray(al, float)
        n = q.shape[0]
        if kind == "channels_reversed":
            al = al[:, ::-1]
        S = np.zeros((q.shape[1], v.shape[1])); z = np.zeros(q.shape[1])
        out = np.empty((n, v.shape[1]))
        for t in range(n):
            a = al[t - 1] if kind == "previous_gate" and t > 0 else (np.ones_like(al[0]) if kind == "previous_gate"
                                                                       else al[t])
            if kind == "value_columns":                  # (d_v <= d here)
                S = S * a[None, : S.shape[1]] + np.outer(k[t], v[t]); z = a * z + k[t]
            elif kind == "gate_after_write":
                S = a[:, None] * (S + np.outer(k[t], v[t])); z = a * (z + k[t])
            else:
                S = a[:, None] * S + np.outer(k[t], v[t])
                z = (z + k[t]) if kind == "z_not_gated" else a * z + k[t]
            num = q[t] @ S
            out[t] = num / (q[t] @ z) if normalize else num
        return out
    return run


@pytest.mark.parametrize("kind", ["value_columns", "gate_after_write", "previous_gate", "z_not_gated",
                                  "channels_reversed"])
def test_pins_catch_mistakes(kind):
    bad = _mutant(kind)
    ok = []
    # pin: one-hot rows, d = 3, d_v = 2 (gate keeps key rows)
    N, d = 12, 3
    al = _gates((N, d), 10)
    good = True
    for f in range(d):
        q = np.zeros((N, d)); q[:, f] = 1.0
        k = np.zeros((N, d)); k[0, f] = 1.0
        v = np.zeros((N, 2)); v[0] = (1.0, 2.0)
        prod = np.concatenate([[1.0], np.cumprod(al[1:, f])])
        o = bad(q, k, v, al, normalize=False)
        good &= np.allclose(o[:, 0], prod, rtol=1e-13) and np.allclose(o[:, 1], 2 * prod, rtol=1e-13)
    ok.append(good)
    # pin: channel-constant gates equal the scalar-gate oracle (normalised)
    n = 20
    q, k, v = _rand((n, 4), 30, 0.5), _rand((n, 4), 31, 0.5), _rand((n, 4), 32)
    a = _gates((n,), 33)
    ref, _, _ = gat.recurrent_gated(q, k, v, a)
    fq, fk = ora.phi_elu1(q), ora.phi_elu1(k)
    ok.append(np.allclose(bad(fq, fk, v, np.repeat(a[:, None], 4, 1)), ref, rtol=1e-12, atol=1e-12))
    assert not all(ok), f"mistake {kind} passes every pin"
