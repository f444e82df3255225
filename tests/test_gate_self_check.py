"""The parity gates of tests/gates.py reject plausible wrong results (CPU).

Each case takes the oracle's own result for a seeded input, plants a
mistake a kernel could plausibly make (nothing here comes from the GPU), and
checks that the gates the GPU tests use reject it.  A rounding model of the
kernels (the same arithmetic in fp64 with every operand the kernels round
to bf16 rounded to bf16) must pass, so the gates are not tighter than the
arithmetic allows.
"""

import numpy as np
import pytest

from oracle import backward as bwd
from oracle import linear_attention as ora
from kernelized_linear_attention_elu_amd import synth
from tests.gates import check_close, check_grad
from tests.grad_scales import grad_scales

N_LONG = 32768
SPAN = 1366          # about the library's span at the long workload (24 per head)


def _bf(x):
    return synth.round_to_io(np.asarray(x, np.float32), "bf16").astype(np.float64)


def _rejected(fn, *args, **kw):
    with pytest.raises(AssertionError):
        fn(*args, **kw)


def _bf16_chunked(q, k, v, C=64):
    """Rounding model of the bf16 prefill: chunks of C tokens, phi(Q) and
    phi(K) rounded to bf16, the carried state rounded to bf16 where it is
    read out, the masked weights rounded to bf16 before they meet V, the
    denominator in full precision, the output rounded to bf16."""
    fq, fk = _bf(ora.phi_elu1(q)), _bf(ora.phi_elu1(k))
    v = np.asarray(v, np.float64)
    out = np.empty(v.shape)
    lead = v.shape[:-2]
    S = np.zeros(lead + (fq.shape[-1], v.shape[-1]))
    z = np.zeros(lead + (fq.shape[-1],))
    for c0 in range(0, v.shape[-2], C):
        Q, K, Vc = fq[..., c0:c0 + C, :], fk[..., c0:c0 + C, :], v[..., c0:c0 + C, :]
        n = Q.shape[-2]
        P = _bf((Q @ np.swapaxes(K, -1, -2)) * np.tril(np.ones((n, n))))
        num = Q @ _bf(S) + P @ Vc
        den = Q @ z[..., None] + P.sum(-1, keepdims=True)
        out[..., c0:c0 + C, :] = _bf(num / den)
        S = S + np.swapaxes(K, -1, -2) @ Vc
        z = z + K.sum(-2)
    return out


@pytest.fixture(scope="module")
def long2():
    """Two heads shaped like the long workload (N = 32768, d = 64, bf16)."""
    q, k, v = synth.draw_qkv(1, 2, N_LONG, 64, 64)
    O, S, z = ora.recurrent_attention(q, k, v)
    return q, k, v, O


def test_zero_rows_pass_the_elementwise_rule_alone(long2):
    """Why the row gate exists: the late rows are below the 2e-2 floor."""
    q, k, v, O = long2
    late = O[..., N_LONG // 2:, :]
    assert np.all(np.abs(late) <= 2e-2)
    check_close(np.zeros_like(late), late, "bf16", rows=False)      # accepted by rule 1 ...
    _rejected(check_close, np.zeros_like(late), late, "bf16")         # ... not by rule 2


def test_half_output_rejected(long2):
    O = long2[3]
    _rejected(check_close, 0.5 * O, O, "bf16")
    _rejected(check_close, 0.9 * O, O, "bf16")


def test_dropped_span_prefix_rejected(long2):
    """Every span restarted from the zero state (the span scan left out)."""
    q, k, v, O = long2
    bad = np.empty_like(O)
    for t0 in range(0, N_LONG, SPAN):
        sl = slice(t0, min(t0 + SPAN, N_LONG))
        bad[..., sl, :] = ora.recurrent_attention(q[..., sl, :], k[..., sl, :], v[..., sl, :])[0]
    late = slice(N_LONG - SPAN, N_LONG)
    _rejected(check_close, bad[..., late, :], O[..., late, :], "bf16")


def test_one_span_missing_from_the_prefix_rejected(long2):
    """The last span read out against a prefix that lacks one earlier span
    (span 10 of 24): a scan that skips a slot."""
    q, k, v, O = long2
    t_last = N_LONG - SPAN
    _, S_pre, z_pre = ora.noncausal_attention(q[..., :t_last, :], k[..., :t_last, :], v[..., :t_last, :])
    sl = slice(10 * SPAN, 11 * SPAN)
    _, dS, dz = ora.noncausal_attention(q[..., sl, :], k[..., sl, :], v[..., sl, :])
    bad = ora.recurrent_attention(q[..., t_last:, :], k[..., t_last:, :], v[..., t_last:, :],
                                  S0=S_pre - dS, z0=z_pre - dz)[0]
    _rejected(check_close, bad, O[..., t_last:, :], "bf16")


def test_off_by_one_and_missing_diagonal_rejected():
    q, k, v = synth.draw_qkv(1, 2, 2048, 64, 64, seed=3)
    O = ora.explicit_attention(q, k, v)
    shifted = np.concatenate([O[..., :1, :], O[..., :-1, :]], axis=-2)
    _rejected(check_close, shifted, O, "bf16")
    fq, fk = ora.phi_elu1(q), ora.phi_elu1(k)
    A = np.tril(fq @ np.swapaxes(fk, -1, -2), -1)                      # j < i only
    A[..., 0, 0] = 1.0
    strict = (A @ v) / A.sum(-1, keepdims=True)
    _rejected(check_close, strict, O, "bf16")


def test_rounding_model_passes():
    """The kernels' roundings stay inside the gates (prefill shapes)."""
    q, k, v = synth.draw_qkv(1, 3, 4096, 64, 64, seed=5)
    O = ora.recurrent_attention(q, k, v)[0]
    _, _, worst_row = check_close(_bf16_chunked(q, k, v), O, "bf16")
    assert worst_row < 0.5e-2                                           # half the gate


def test_noncausal_planted_mistakes_rejected(long2):
    q, k, v, _ = long2
    O = ora.noncausal_attention(q, k, v)[0]
    assert np.all(np.abs(O) < 2e-2)                                     # all below the floor
    _rejected(check_close, np.zeros_like(O), O, "bf16")
    _rejected(check_close, 0.5 * O, O, "bf16")
    _rejected(check_close, long2[3], O, "bf16")                         # the causal rows instead


# ---------------------------------------------------------------- gradients

def _chunk_mask(n, C=64):
    i = np.arange(n)
    return (i[None, :] <= i[:, None]) & (i[None, :] // C == i[:, None] // C)


def _grads_masked(q, k, v, dO, mask):
    """The chain rule of oracle.backward with the weights' gradient kept only
    where ``mask`` holds (a kernel that loses the history or the suffix)."""
    fq, fk = ora.phi_elu1(q), ora.phi_elu1(k)
    n = q.shape[-2]
    A = (fq @ np.swapaxes(fk, -1, -2)) * np.tril(np.ones((n, n)))
    D = A.sum(-1)
    O = (A @ v) / D[..., None]
    rho = np.sum(dO * O, -1)
    dA = ((dO @ np.swapaxes(v, -1, -2)) - rho[..., None]) / D[..., None] * mask
    dq = (dA @ fk) * bwd.phi_prime("elu1", q)
    dk = (np.swapaxes(dA, -1, -2) @ fq) * bwd.phi_prime("elu1", k)
    return dq, dk


def _bwd_dq_rounding_model(q, k, v, dO, C=64):
    """Rounding model of the dQ pass: phi, g = dO / D, the masked W, the
    carried state and the forward output in bf16, the result rounded to bf16."""
    O = _bf(ora.recurrent_attention(q, k, v)[0])
    fq, fk = _bf(ora.phi_elu1(q)), _bf(ora.phi_elu1(k))
    v = np.asarray(v, np.float64)
    dO = np.asarray(dO, np.float64)
    lead = v.shape[:-2]
    S = np.zeros(lead + (64, 64))
    z = np.zeros(lead + (64,))
    dq = np.empty(v.shape)
    for c0 in range(0, v.shape[-2], C):
        sl = slice(c0, c0 + C)
        Q, K, Vc, G, o = fq[..., sl, :], fk[..., sl, :], v[..., sl, :], dO[..., sl, :], O[..., sl, :]
        n = Q.shape[-2]
        tri = np.tril(np.ones((n, n)))
        P = _bf((Q @ np.swapaxes(K, -1, -2)) * tri)
        D = (Q @ z[..., None])[..., 0] + P.sum(-1)
        g = G / D[..., None]
        h = -np.sum(G * o, -1) / D
        W = _bf((_bf(g) @ np.swapaxes(Vc, -1, -2) + h[..., None]) * tri)
        dphi = W @ K + _bf(g) @ np.swapaxes(_bf(S), -1, -2) + h[..., None] * z[..., None, :]
        dq[..., sl, :] = _bf(dphi * np.minimum(1.0, ora.phi_elu1(q[..., sl, :])))
        S = S + np.swapaxes(K, -1, -2) @ Vc
        z = z + K.sum(-2)
    return dq


@pytest.fixture(scope="module")
def grad_case():
    q, k, v = synth.draw_qkv(1, 3, 640, 64, 64, seed=81)
    dO = synth.round_to_io(np.random.default_rng(1081).standard_normal(q.shape, dtype=np.float32), "bf16")
    return q, k, v, dO, bwd.grad_causal(q, k, v, dO), grad_scales(q, k, v, dO)


def test_grad_scaled_rejected(grad_case):
    *_, (rq, rk, rv), (sq, sk, sv) = grad_case
    for f in (0.5, 0.9):
        _rejected(check_grad, f * rq, rq, sq, "dQ")
        _rejected(check_grad, f * rk, rk, sk, "dK")
        _rejected(check_grad, f * rv, rv, sv, "dV")


def test_grad_without_history_or_suffix_rejected(grad_case):
    """dQ from the in-chunk terms only (no S g + h z from earlier chunks), and
    dK with the later chunks' suffix sums dropped."""
    q, k, v, dO, (rq, rk, rv), (sq, sk, sv) = grad_case
    dq_in, dk_in = _grads_masked(q, k, v, dO, _chunk_mask(q.shape[-2]))
    _rejected(check_grad, dq_in, rq, sq, "dQ")
    _rejected(check_grad, dk_in, rk, sk, "dK")


def test_grad_unnormalised_dv_rejected(grad_case):
    q, k, v, dO, (rq, rk, rv), (sq, sk, sv) = grad_case
    fq, fk = ora.phi_elu1(q), ora.phi_elu1(k)
    A = np.tril(fq @ np.swapaxes(fk, -1, -2))
    _rejected(check_grad, np.swapaxes(A, -1, -2) @ dO, rv, sv, "dV")


def test_grad_rounding_model_passes(grad_case):
    q, k, v, dO, (rq, _, _), (sq, _, _) = grad_case
    head, block, row = check_grad(_bwd_dq_rounding_model(q, k, v, dO), rq, sq, "dQ")
    assert head < 0.6 * 3e-2 and block < 0.6 * 5e-2 and row < 0.6
