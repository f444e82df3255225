"""Pins of the per-token gated oracle (oracle/gated.py) against what the pages
and the mathematics fix, independently of the oracle's own code:

* every gate 1 gives plain causal linear attention: the "Linear attention and
  SSM" page states that linear attention is the special case of structured
  masked attention whose mask is the causal lower-triangular one (checked
  against the pinned oracle.linear_attention, and unnormalised against
  tril(phi(Q) phi(K)^T) V);
* a constant gate per head is the fixed decay of "Efficient attention
  variants" sec. 7.1 (the pinned oracle.decay), including that page's figure
  gamma = 0.99 -> weight 0.366 at lag 100 (tests/golden/retnet_decay.txt);
* the mask L is 1-semiseparable, as the page states: every submatrix taken
  wholly below the diagonal has rank at most one; and L_ii = 1, which the
  discrete SSM recurrence h_t = a_t h_{t-1} + B x_t, y_t = C h_t fixes;
* a zero gate (the page's "large Delta forgets the history") is a reset: the
  outputs from that token on equal a fresh run started there;
* the explicit mask form, the token recurrence and a chunked evaluation (the
  page's "matrix products inside a chunk, recurrence across chunks") agree,
  normalised or not, with an initial state;
* decode chain, split prefill and sampled rows agree with the recurrence.

A planted mistake (gate applied after the write, the previous token's gate,
z left ungated, a gated read-out, gates in reverse order) fails at least one
pin (test_pins_catch_mistakes).
"""

import numpy as np
import pytest

from oracle import decay as dec
from oracle import gated as gat
from oracle import linear_attention as ora
from tests.golden import load

TOL = 1e-12


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _gates(shape, seed):
    """Mamba-2-like gates exp(-dt * A): dt log-uniform in [1e-3, 1e-1], A in [1, 16]."""
    rng = np.random.default_rng(seed)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=shape))
    return np.exp(-dt * rng.uniform(1.0, 16.0, size=shape[:-1] + (1,)))


@pytest.mark.parametrize("phi", ["elu1", "identity"])
def test_unit_gates_are_plain_linear_attention(phi):
    q, k, v = _rand((2, 3, 40, 5), 1), _rand((2, 3, 40, 5), 2), _rand((2, 3, 40, 4), 3)
    if phi == "identity":
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    a = np.ones((2, 3, 40))
    ref, S_ref, z_ref = ora.recurrent_attention(q, k, v, phi=phi)
    out, S, z = gat.recurrent_gated(q, k, v, a, phi=phi)
    np.testing.assert_allclose(out, ref, rtol=0, atol=TOL)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=TOL)
    np.testing.assert_allclose(z, z_ref, rtol=0, atol=TOL)
    np.testing.assert_allclose(gat.explicit_gated(q, k, v, a, phi=phi), ref, rtol=1e-12, atol=1e-12)
    raw = gat.explicit_gated(q, k, v, a, phi=phi, normalize=False)
    fq, fk = ora.feature_map(phi, q), ora.feature_map(phi, k)
    np.testing.assert_allclose(raw, np.tril(fq @ np.swapaxes(fk, -1, -2)) @ v, rtol=1e-12, atol=1e-12)
    assert np.array_equal(gat.gate_mask(np.ones(7)), np.tril(np.ones((7, 7))))


def test_constant_gate_is_the_fixed_decay_and_the_page_figure():
    g = load("retnet_decay.txt")
    lag = int(g["lag"])
    q = np.ones((lag + 1, 1)); k = np.zeros((lag + 1, 1)); k[0] = 1.0
    v = np.zeros((lag + 1, 1)); v[0] = 1.0
    a = np.full(lag + 1, g["gamma"])
    o, _, _ = gat.recurrent_gated(q, k, v, a, phi="identity", normalize=False)
    assert round(o[lag, 0], 3) == g["weight"]
    np.testing.assert_allclose(o[:, 0], g["gamma"] ** np.arange(lag + 1), rtol=1e-13, atol=0)
    B, H, N = 2, 3, 33
    q, k, v = _rand((B, H, N, 6), 4, 0.5), _rand((B, H, N, 6), 5, 0.5), _rand((B, H, N, 3), 6)
    gam = np.array([0.5, 0.9, 0.999])
    a = np.broadcast_to(gam[None, :, None], (B, H, N))
    S0 = np.abs(_rand((B, H, 6, 3), 7)); z0 = np.abs(_rand((B, H, 6), 8)) + 1.0
    for normalize in (True, False):
        ref, S_ref, z_ref = dec.recurrent_decay(q, k, v, gam, normalize=normalize, S0=S0, z0=z0)
        out, S, z = gat.recurrent_gated(q, k, v, a, normalize=normalize, S0=S0, z0=z0)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(z, z_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(gat.explicit_gated(q, k, v, a, normalize=normalize, S0=S0, z0=z0), ref,
                                   rtol=1e-11, atol=1e-12)


def test_mask_is_one_semiseparable_with_unit_diagonal():
    a = _gates((24,), 9)
    L = gat.gate_mask(a)
    assert np.all(np.diag(L) == 1.0)
    assert np.all(np.triu(L, 1) == 0.0)
    for i0 in range(1, 24):
        for j1 in range(1, i0 + 1):
            sub = L[i0:, :j1]                          # rows >= i0, columns < j1 <= i0: below the diagonal
            sv = np.linalg.svd(sub, compute_uv=False)
            assert sv[0] > 0 and (len(sv) == 1 or sv[1] <= 1e-13 * sv[0])
    # one rank-one factor: L_ij = P_i / P_j with P the running product
    P = np.cumprod(a)
    np.testing.assert_allclose(np.tril(L, -1), np.tril(P[:, None] / P[None, :], -1), rtol=1e-12, atol=0)


@pytest.mark.parametrize("normalize", [True, False])
def test_zero_gate_resets(normalize):
    B, H, N, t0 = 1, 2, 30, 13
    q, k, v = _rand((B, H, N, 4), 10, 0.5), _rand((B, H, N, 4), 11, 0.5), _rand((B, H, N, 3), 12)
    a = _gates((B, H, N), 13)
    a[..., t0] = 0.0
    full, S, z = gat.recurrent_gated(q, k, v, a, normalize=normalize)
    fresh, S2, z2 = gat.recurrent_gated(q[:, :, t0:], k[:, :, t0:], v[:, :, t0:], a[:, :, t0:], normalize=normalize)
    np.testing.assert_allclose(full[:, :, t0:], fresh, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S2, rtol=1e-12, atol=1e-12)
    ex = gat.explicit_gated(q, k, v, a, normalize=normalize)
    np.testing.assert_allclose(ex, full, rtol=1e-11, atol=1e-12)


def _chunked(q, k, v, a, C, normalize):
    """The page's chunked evaluation for one head: inside a chunk the masked
    products ((phi(Q) phi(K)^T) o L) V; across chunks a carried state,
    read with the running product of the chunk's gates and advanced by the
    chunk's total product."""
    fq, fk = ora.phi_elu1(q), ora.phi_elu1(k)
    n = q.shape[0]
    S = np.zeros((fq.shape[1], v.shape[1])); z = np.zeros(fq.shape[1])
    out = np.empty((n, v.shape[1]))
    for c0 in range(0, n, C):
        sl = slice(c0, min(n, c0 + C))
        ac = a[sl]
        P = np.cumprod(ac)                                   # a_c0 ... a_i
        L = np.tril(P[:, None] / P[None, :])
        A = (fq[sl] @ fk[sl].T) * L
        num = A @ v[sl] + P[:, None] * (fq[sl] @ S)
        den = A.sum(axis=1) + P * (fq[sl] @ z)
        out[sl] = num / den[:, None] if normalize else num
        w = P[-1] / P                                       # a_{j+1} ... a_end
        S = P[-1] * S + (fk[sl] * w[:, None]).T @ v[sl]
        z = P[-1] * z + (fk[sl] * w[:, None]).sum(axis=0)
    return out, S, z


@pytest.mark.parametrize("normalize", [True, False])
def test_explicit_recurrent_and_chunked_agree_with_state(normalize):
    B, H, N, d, dv = 2, 3, 37, 6, 5
    q, k, v = _rand((B, H, N, d), 14, 0.5), _rand((B, H, N, d), 15, 0.5), _rand((B, H, N, dv), 16)
    a = _gates((B, H, N), 17)
    S0 = np.abs(_rand((B, H, d, dv), 18)); z0 = np.abs(_rand((B, H, d), 19)) + 1.0
    o_rec, S, z = gat.recurrent_gated(q, k, v, a, normalize=normalize, S0=S0, z0=z0)
    o_exp = gat.explicit_gated(q, k, v, a, normalize=normalize, S0=S0, z0=z0)
    np.testing.assert_allclose(o_exp, o_rec, rtol=1e-11, atol=1e-12)
    # final state written out: sum_j (a_{j+1} ... a_{N-1}) phi(k_j) v_j^T + (a_0 ... a_{N-1}) S0
    fk = ora.phi_elu1(k)
    tail = np.flip(np.cumprod(np.flip(a, -1), -1), -1)      # a_j ... a_{N-1}
    w = np.concatenate([tail[..., 1:], np.ones((B, H, 1))], axis=-1)
    S_def = np.einsum("bhn,bhnr,bhnc->bhrc", w, fk, v) + tail[..., 0, None, None] * S0
    np.testing.assert_allclose(S, S_def, rtol=1e-12, atol=1e-12)
    for C in (4, 16):
        o_c, S_c, z_c = _chunked(q[1, 2], k[1, 2], v[1, 2], a[1, 2], C, normalize)
        r1, _, _ = gat.recurrent_gated(q[1, 2], k[1, 2], v[1, 2], a[1, 2], normalize=normalize)
        np.testing.assert_allclose(o_c, r1, rtol=1e-11, atol=1e-12)


def test_decode_chain_split_prefill_and_rows():
    B, H, N, d, dv = 1, 2, 25, 4, 3
    q, k, v = _rand((B, H, N, d), 20), _rand((B, H, N, d), 21), _rand((B, H, N, dv), 22)
    a = _gates((B, H, N), 23)
    a[0, 1, 7] = 0.0
    ref, S_ref, z_ref = gat.recurrent_gated(q, k, v, a)
    S = np.zeros((B, H, d, dv)); z = np.zeros((B, H, d))
    for t in range(N):
        o, S, z = gat.decode_step_gated(S, z, q[:, :, t], k[:, :, t], v[:, :, t], a[:, :, t])
        np.testing.assert_allclose(o, ref[:, :, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)
    cut = 11
    o1, S1, z1 = gat.recurrent_gated(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], a[:, :, :cut])
    o2, S2, _ = gat.recurrent_gated(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], a[:, :, cut:], S0=S1, z0=z1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S_ref, rtol=1e-12, atol=1e-12)
    for normalize in (True, False):
        full, _, _ = gat.recurrent_gated(q, k, v, a, normalize=normalize)
        for h in range(H):
            rows = [0, 1, 7, 8, 24]
            got = gat.causal_rows_gated(q[0, h], k[0, h], v[0, h], a[0, h], rows, normalize=normalize)
            np.testing.assert_allclose(got, full[0, h, rows], rtol=1e-12, atol=1e-12)


def _mutant(kind):
    """A copy of the single-head recurrence with one plausible mistake planted
    (used only to check that the pins above would catch it)."""
    def run(q, k, v, a, normalize=True):
        q = np.asarray(q, float); k = np.asarray(k, float); v = np.asarray(v, float); a = np.asarray(a, float)
        n = q.shape[0]
        if kind == "reversed_gates":
            a = a[::-1]
        S = np.zeros((q.shape[1], v.shape[1])); z = np.zeros(q.shape[1])
        out = np.empty((n, v.shape[1]))
        for t in range(n):
            at = a[t - 1] if kind == "previous_gate" and t > 0 else (1.0 if kind == "previous_gate" else a[t])
            if kind == "gate_after_write":
                S = at * (S + np.outer(k[t], v[t])); z = at * (z + k[t])
            else:
                S = at * S + np.outer(k[t], v[t])
                z = (z + k[t]) if kind == "z_not_gated" else at * z + k[t]
            num = q[t] @ S
            if kind == "read_gated":
                num = at * num
            out[t] = num / (q[t] @ z) if normalize else num
        return out
    return run


@pytest.mark.parametrize("kind", ["gate_after_write", "previous_gate", "z_not_gated", "read_gated", "reversed_gates"])
def test_pins_catch_mistakes(kind):
    bad = _mutant(kind)
    g = load("retnet_decay.txt")
    # pin 1: the page's figure through constant gates
    n = 101
    q = np.ones((n, 1)); k = np.zeros((n, 1)); k[0] = 1.0; v = np.zeros((n, 1)); v[0] = 1.0
    o = bad(q, k, v, np.full(n, g["gamma"]), normalize=False)
    page_ok = round(o[100, 0], 3) == g["weight"] and abs(o[100, 0] - g["gamma"] ** 100) < TOL
    # pin 2: constant gate 0.5 with normalisation (the fixed decay's impulse closed form)
    m = 30
    q2 = np.ones((m, 1)); k2 = np.ones((m, 1)); v2 = np.zeros((m, 1)); v2[0] = 1.0
    t = np.arange(m)
    closed = 0.5 ** t * 0.5 / (1 - 0.5 ** (t + 1))
    impulse_ok = np.allclose(bad(q2, k2, v2, np.full(m, 0.5))[:, 0], closed, rtol=1e-12)
    # pin 3: a zero gate at t0 resets
    N, t0 = 30, 9
    q3, k3, v3 = np.abs(_rand((N, 4), 24)) + 0.1, np.abs(_rand((N, 4), 25)) + 0.1, _rand((N, 3), 26)
    a3 = _gates((N,), 27)
    a3[t0] = 0.0
    full = bad(q3, k3, v3, a3)
    fresh = bad(q3[t0:], k3[t0:], v3[t0:], a3[t0:])
    reset_ok = np.allclose(full[t0:], fresh, rtol=1e-12, atol=1e-12)
    assert not (page_ok and impulse_ok and reset_ok), f"mistake {kind} passes every pin"
