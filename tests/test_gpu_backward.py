"""GPU parity of the backward pass (la_backward) against the fp64 gradient
oracle (oracle/backward.py): dQ, dK, dV of sum(dO * O), with O the
library's own forward output for the same bf16 Q, K, V (as a training step
would pass it).

Tolerance.  Each gradient entry is a sum of terms of mixed sign (for dQ:
(v_j.g_i + h_i) phi(k_j) over j <= i), and every term passes through a few
bf16 roundings (phi, g = dO / D, the weights, the bf16 state tiles), each
within 2^-9 of its value.  The bound is therefore taken against the sum of
the terms' magnitudes, computed in fp64 from the same inputs:
    |err| <= 2e-2 |ref| + 2e-2 scale,
    scale(dQ_i) = sum_{j<=i} (|dO_i|.|v_j| + |rho_i|) / D_i |phi(k_j)| |phi'(q_i)|,
    scale(dK_j) = sum_{i>=j} (|dO_i|.|v_j| + |rho_i|) / D_i |phi(q_i)| |phi'(k_j)|,
    scale(dV_j) = sum_{i>=j} A_ij / D_i |dO_i|,
with rho_i = dO_i . O_i: several times the worst bf16 accumulation.
"""

import numpy as np
import pytest

from oracle import backward as bwd
from oracle import linear_attention as ora
from kernelized_linear_attention_elu_amd import synth
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture
def span(monkeypatch):
    def _set(tokens):
        if tokens is None:
            monkeypatch.delenv("LA_SPAN", raising=False)
        else:
            monkeypatch.setenv("LA_SPAN", str(tokens))
    _set(None)
    return _set


def _draw(B, H, N, seed, phi="elu1", d=64):
    q, k, v = synth.draw_qkv(B, H, N, d, d, seed=seed)
    if phi == "identity":  # positive features keep the denominators positive
        q = synth.round_to_io(np.abs(q) + 0.25, "bf16")
        k = synth.round_to_io(np.abs(k) + 0.25, "bf16")
    rng = np.random.default_rng(seed + 1000)
    dO = synth.round_to_io(rng.standard_normal((B, H, N, d), dtype=np.float32), "bf16")
    return q, k, v, dO


def _run(lib, q, k, v, dO, phi="elu1"):
    import torch
    Q, K, V, G = (to_dev(x, "bf16") for x in (q, k, v, dO))
    O = lib.forward(Q, K, V, phi=phi)
    dQ, dK, dV = lib.backward(Q, K, V, O, G, phi=phi)
    torch.cuda.synchronize()
    return to_host(dQ), to_host(dK), to_host(dV)


def _scales(q, k, v, dO, phi="elu1"):
    fq = ora.feature_map(phi, q)
    fk = ora.feature_map(phi, k)
    v = np.asarray(v, np.float64)
    dO = np.asarray(dO, np.float64)
    n = fq.shape[-2]
    mask = np.tril(np.ones((n, n)))
    A = (fq @ np.swapaxes(fk, -1, -2)) * mask
    D = A.sum(-1)
    O = (A @ v) / D[..., None]
    rho = np.abs(np.sum(dO * O, -1))
    M = ((np.abs(dO) @ np.swapaxes(np.abs(v), -1, -2)) + rho[..., None]) / D[..., None] * mask
    sq = (M @ np.abs(fk)) * np.abs(bwd.phi_prime(phi, q))
    sk = (np.swapaxes(M, -1, -2) @ np.abs(fq)) * np.abs(bwd.phi_prime(phi, k))
    sv = np.swapaxes(A / D[..., None], -1, -2) @ np.abs(dO)
    return sq, sk, sv


def _check(got, ref, scale, what):
    err = np.abs(got - ref)
    bound = 2e-2 * np.abs(ref) + 2e-2 * scale
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (f"{what}: worst at {worst}: got {got[worst]!r} ref {ref[worst]!r} "
                                  f"bound {bound[worst]:.3e}")


@pytest.mark.parametrize("phi", ["elu1", "identity"])
@pytest.mark.parametrize("B,H,N,tokens", [
    (1, 3, 1, None), (1, 3, 17, None), (1, 3, 64, None), (2, 2, 100, None), (1, 3, 300, None),
    (1, 3, 300, 128), (1, 2, 517, 64),
])
def test_backward_small(lib, span, B, H, N, tokens, phi):
    """Ragged tails, several chunks and (with the span override) several
    spans per head, so that the forward prefix, the reverse suffix and both
    in-span carries are exercised."""
    span(tokens)
    q, k, v, dO = _draw(B, H, N, 81 + N, phi)
    dq, dk, dv = _run(lib, q, k, v, dO, phi)
    rq, rk, rv = bwd.grad_causal(q, k, v, dO, phi=phi)
    sq, sk, sv = _scales(q, k, v, dO, phi)
    _check(dq, rq, sq, "dQ")
    _check(dk, rk, sk, "dK")
    _check(dv, rv, sv, "dV")


@pytest.mark.parametrize("phi", ["elu1", "identity"])
@pytest.mark.parametrize("N,tokens", [(17, None), (300, None), (333, 128)])
def test_backward_wide_heads(lib, span, N, tokens, phi):
    """d = d_v = 128: eight waves, two per 16-row block, each with half of the
    feature and value tiles."""
    span(tokens)
    q, k, v, dO = _draw(2, 2, N, 95 + N, phi, d=128)
    dq, dk, dv = _run(lib, q, k, v, dO, phi)
    rq, rk, rv = bwd.grad_causal(q, k, v, dO, phi=phi)
    sq, sk, sv = _scales(q, k, v, dO, phi)
    _check(dq, rq, sq, "dQ")
    _check(dk, rk, sk, "dK")
    _check(dv, rv, sv, "dV")


def test_backward_no_future_leakage_in_dq_bitwise(lib, span):
    """dQ_i depends on tokens up to i only: changing keys, values and the
    upstream gradient from t0 on leaves dQ before t0 bit-identical (dK and
    dV, which depend on later tokens, change)."""
    import torch
    span(128)
    q, k, v, dO = _draw(1, 2, 400, 90)
    base = _run(lib, q, k, v, dO)
    for t0 in (256, 200, 37):
        k2, v2, d2 = k.copy(), v.copy(), dO.copy()
        k2[..., t0:, :] = synth.round_to_io(k2[..., t0:, :] + 0.5, "bf16")
        v2[..., t0:, :] = synth.round_to_io(v2[..., t0:, :] - 1.0, "bf16")
        d2[..., t0:, :] = synth.round_to_io(d2[..., t0:, :] * 2.0, "bf16")
        out = _run(lib, q, k2, v2, d2)
        np.testing.assert_array_equal(out[0][..., :t0, :], base[0][..., :t0, :])
        assert np.max(np.abs(out[1][..., :t0, :] - base[1][..., :t0, :])) > 0
    torch.cuda.synchronize()


def test_backward_long_workload_sampled(lib):
    """The long workload (B1 H32 N32768 d64 bf16) in the bench's launch
    configuration: dQ, dK, dV at sampled rows of every head from the
    sampled-row oracle (prefix and suffix sums in fp64)."""
    w = synth.WORKLOADS["long"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    rng = np.random.default_rng(91)
    dO = synth.round_to_io(rng.standard_normal((w.B, w.H, w.N, w.dv), dtype=np.float32), "bf16")
    dq, dk, dv = _run(lib, q, k, v, dO)
    rows = sorted({0, 1, 63, 64, 2047, 2048, 2049, 17000, w.N - 2, w.N - 1})   # 2048-token spans
    rq, rk, rv = bwd.grad_rows(q, k, v, dO, rows)
    # the magnitude scales at the sampled rows, from the same sums with |.|
    fq, fk = ora.phi_elu1(q), ora.phi_elu1(k)
    scale_q = np.zeros_like(rq)
    scale_k = np.zeros_like(rk)
    scale_v = np.zeros_like(rv)
    for h in range(w.H):
        z = np.cumsum(fk[0, h], axis=0)
        D = np.sum(fq[0, h] * z, axis=1)                              # [N]
        # O_i from the same sums (fp64): only |rho| enters the scale
        S_rows = {}
        for t in rows:
            S_rows[t] = fk[0, h, : t + 1].T @ v[0, h, : t + 1].astype(np.float64)
        for n_, t in enumerate(rows):
            Ot = fq[0, h, t] @ S_rows[t] / D[t]
            rho = abs(float(np.dot(dO[0, h, t], Ot)))
            wts = (np.abs(v[0, h, : t + 1]) @ np.abs(dO[0, h, t]) + rho) / D[t]
            scale_q[0, h, n_] = (wts @ np.abs(fk[0, h, : t + 1])) * np.abs(bwd.phi_prime("elu1", q[0, h, t]))
        # dK, dV scales need all later rows' rho_i: bound |rho_i| by |dO_i|.max|v| (a looser scale)
        vmax = np.max(np.abs(v[0, h]))
        rho_b = np.sum(np.abs(dO[0, h]), axis=1) * vmax
        for n_, t in enumerate(rows):
            a = fq[0, h, t:] @ fk[0, h, t] / D[t:]                      # A_it / D_i, i >= t
            wts = (np.abs(dO[0, h, t:]) @ np.abs(v[0, h, t]) + rho_b[t:]) / D[t:]
            scale_k[0, h, n_] = (wts @ np.abs(fq[0, h, t:])) * np.abs(bwd.phi_prime("elu1", k[0, h, t]))
            scale_v[0, h, n_] = a @ np.abs(dO[0, h, t:])
    _check(dq[:, :, rows], rq, scale_q, "dQ")
    _check(dk[:, :, rows], rk, scale_k, "dK")
    _check(dv[:, :, rows], rv, scale_v, "dV")
