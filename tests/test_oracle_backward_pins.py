"""Pins of the gradient oracle (oracle/backward.py) against what fixes the
gradients independently of its code:

* central finite differences of the pinned forward oracle
  (oracle.linear_attention.recurrent_attention, the token recurrence: a
  different algorithm from the explicit form the gradients are written on),
  in fp64, for every entry of Q, K and V at a tiny size and for random
  directions at a larger one;
* closed forms: with all value rows equal, O does not depend on Q or K, so
  dQ = dK = 0; with dO = 1 everywhere, dV_j is the column sum of the
  normalised causal attention, sum_{i>=j} A_ij / D_i; for one token,
  dV = dO and dQ = dK = 0;
* the identity map's gradient is the ELU+1 one with phi' = 1;
* the sampled-row form (prefix and suffix states, for long sequences)
  equals the explicit form at every sampled row.

Planted mistakes (the rowsum(dO*O) term dropped, the mask transposed, phi'
left out, dV from the unnormalised weights) each fail a pin
(test_pins_catch_mistakes).
"""

import numpy as np
import pytest

from oracle import backward as bwd
from oracle import linear_attention as ora


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, dO, phi="elu1"):
    out, _, _ = ora.recurrent_attention(q, k, v, phi=phi)
    return float(np.sum(out * dO))


def _fd(q, k, v, dO, phi="elu1", eps=1e-6):
    """Central differences of sum(dO * O) for every entry of q, k, v."""
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(g.shape):
            up = [a.copy() for a in args]
            dn = [a.copy() for a in args]
            up[which][idx] += eps
            dn[which][idx] -= eps
            g[idx] = (_loss(*up, dO, phi) - _loss(*dn, dO, phi)) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("phi", ["elu1", "identity"])
def test_every_entry_against_finite_differences(phi):
    N, d, dv = 6, 3, 2
    q, k, v = _rand((N, d), 1, 0.7), _rand((N, d), 2, 0.7), _rand((N, dv), 3)
    if phi == "identity":
        q, k = np.abs(q) + 0.2, np.abs(k) + 0.2
    dO = _rand((N, dv), 4)
    dq, dk, dvv = bwd.grad_causal(q, k, v, dO, phi=phi)
    fq, fk, fv = _fd(q, k, v, dO, phi=phi)
    np.testing.assert_allclose(dq, fq, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dk, fk, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dvv, fv, rtol=1e-6, atol=1e-8)


def test_random_directions_against_finite_differences():
    """Directional derivatives at B=1, H=2, N=40, d=5, dv=4."""
    shape_qk, shape_v = (1, 2, 40, 5), (1, 2, 40, 4)
    q, k, v = _rand(shape_qk, 5, 0.6), _rand(shape_qk, 6, 0.6), _rand(shape_v, 7)
    dO = _rand(shape_v, 8)
    dq, dk, dvv = bwd.grad_causal(q, k, v, dO)
    rng = np.random.default_rng(9)
    for _ in range(4):
        uq, uk, uv = rng.standard_normal(shape_qk), rng.standard_normal(shape_qk), rng.standard_normal(shape_v)
        eps = 1e-6
        fd = (_loss(q + eps * uq, k + eps * uk, v + eps * uv, dO)
              - _loss(q - eps * uq, k - eps * uk, v - eps * uv, dO)) / (2 * eps)
        an = np.sum(dq * uq) + np.sum(dk * uk) + np.sum(dvv * uv)
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an))


def test_closed_forms():
    N, d, dv = 9, 4, 3
    q, k = _rand((N, d), 10), _rand((N, d), 11)
    # equal value rows: O = v for every row, independent of q and k
    v = np.tile(_rand((1, dv), 12), (N, 1))
    dq, dk, _ = bwd.grad_causal(q, k, v, _rand((N, dv), 13))
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    # dO = 1: dV_j = sum_{i >= j} A_ij / D_i
    v = _rand((N, dv), 14)
    _, _, dvv = bwd.grad_causal(q, k, v, np.ones((N, dv)))
    fq, fk = ora.phi_elu1(q), ora.phi_elu1(k)
    A = np.tril(fq @ fk.T)
    col = (A / A.sum(axis=1, keepdims=True)).sum(axis=0)
    np.testing.assert_allclose(dvv, np.repeat(col[:, None], dv, axis=1), rtol=1e-13)
    # one token: O = v, so dV = dO and dQ = dK = 0
    dq1, dk1, dv1 = bwd.grad_causal(q[:1], k[:1], v[:1], np.ones((1, dv)) * 0.3)
    np.testing.assert_allclose(dv1, 0.3 * np.ones((1, dv)), rtol=0, atol=1e-15)
    assert np.all(np.abs(dq1) < 1e-15) and np.all(np.abs(dk1) < 1e-15)


def test_identity_is_elu_path_with_unit_derivative():
    N, d, dv = 12, 3, 2
    q, k = np.abs(_rand((N, d), 15)) + 0.1, np.abs(_rand((N, d), 16)) + 0.1   # x > 0: phi = x + 1
    v, dO = _rand((N, dv), 17), _rand((N, dv), 18)
    g_elu = bwd.grad_causal(q, k, v, dO, phi="elu1")
    g_id = bwd.grad_causal(q + 1.0, k + 1.0, v, dO, phi="identity")
    for a, b in zip(g_elu, g_id):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("phi", ["elu1", "identity"])
def test_sampled_rows_equal_the_explicit_form(phi):
    shape_qk, shape_v = (2, 2, 45, 5), (2, 2, 45, 3)
    q, k, v = _rand(shape_qk, 19, 0.6), _rand(shape_qk, 20, 0.6), _rand(shape_v, 21)
    if phi == "identity":
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    dO = _rand(shape_v, 22)
    full = bwd.grad_causal(q, k, v, dO, phi=phi)
    rows = [0, 1, 17, 30, 44]
    part = bwd.grad_rows(q, k, v, dO, rows, phi=phi)
    for a, b in zip(part, full):
        np.testing.assert_allclose(a, b[..., rows, :], rtol=1e-11, atol=1e-12)


def _mutant(kind):
    def run(q, k, v, dO):
        fq, fk = ora.phi_elu1(q), ora.phi_elu1(k)
        n = q.shape[0]
        mask = np.tril(np.ones((n, n)))
        if kind == "mask_transposed":
            mask = mask.T
        A = fq @ fk.T * np.tril(np.ones((n, n)))
        D = A.sum(axis=1)
        O = A @ v / D[:, None]
        rho = np.sum(dO * O, axis=1)
        if kind == "no_rowsum_term":
            rho = 0 * rho
        dA = ((dO @ v.T) - rho[:, None]) / D[:, None] * mask
        dfq, dfk = dA @ fk, dA.T @ fq
        W = A if kind == "dv_unnormalised" else A / D[:, None]
        dvv = W.T @ dO
        pq = np.ones_like(q) if kind == "no_phi_prime" else bwd.phi_prime("elu1", q)
        pk = np.ones_like(k) if kind == "no_phi_prime" else bwd.phi_prime("elu1", k)
        return dfq * pq, dfk * pk, dvv
    return run


@pytest.mark.parametrize("kind", ["no_rowsum_term", "mask_transposed", "no_phi_prime", "dv_unnormalised"])
def test_pins_catch_mistakes(kind):
    N, d, dv = 6, 3, 2
    q, k, v = _rand((N, d), 1, 0.7), _rand((N, d), 2, 0.7), _rand((N, dv), 3)
    dO = _rand((N, dv), 4)
    got = _mutant(kind)(q, k, v, dO)
    ref = _fd(q, k, v, dO)
    ok = all(np.allclose(a, b, rtol=1e-6, atol=1e-8) for a, b in zip(got, ref))
    assert not ok, f"mistake {kind} passes the finite-difference pin"
