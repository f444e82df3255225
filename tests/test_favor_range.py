"""Numeric range of FAVOR+ at large input norms ("Efficient attention
variants", sec. 6: the estimator's quality depends on its numerical
stability).  CPU only: the fp64 oracle and plain float32 arithmetic written
here, nothing of the HIP path.

1. The shifts the kernels apply cancel: multiplying every feature of query
   row i by one constant c_i, and every key feature of a head by one
   constant c_h, leaves the normalised outputs unchanged (checked in fp64
   with the oracle's features, with the kernels' choice of constants and with
   arbitrary ones).
2. Without them, float32 features at 14 times the workload's norms make most
   rows 0/0: the reason the GPU test at that scale (tests/test_gpu_favor.py)
   is a test of the shifts and not of ordinary rounding.
"""

import numpy as np
import pytest

from oracle import linear_attention as ora
from kernelized_linear_attention_elu_amd import synth


def _inputs(scale, N=200, seed=21):
    q, k, v = synth.draw_qkv(1, 1, N, 64, 64, seed=seed)
    q = synth.round_to_io(q * scale, "bf16").astype(np.float64)
    k = synth.round_to_io(k * scale, "bf16").astype(np.float64)
    return q[0, 0], k[0, 0], v[0, 0].astype(np.float64)


def _causal_from_features(fq, fk, v):
    A = np.tril(fq @ fk.T)
    return (A @ v) / A.sum(-1, keepdims=True)


@pytest.mark.parametrize("scale", [1.0, 6.0])
def test_row_and_head_constants_cancel(scale):
    omega = synth.draw_omega(256, 64)
    q, k, v = _inputs(scale)
    fq, fk = ora.phi_favor(q, omega), ora.phi_favor(k, omega)
    base = _causal_from_features(fq, fk, v)
    np.testing.assert_allclose(base, ora.recurrent_attention(q[None, None], k[None, None], v[None, None],
                                                             phi="favor", omega=omega)[0][0, 0], rtol=1e-9, atol=1e-12)
    # the kernels' constants: exp(|x|^2 / 2 - 4 |x|) per query row, and per head
    # the first key's exp(|x_0|^2 / 2 - 4 |x_0|)
    xq = q / 64 ** 0.25
    xk0 = k[0] / 64 ** 0.25
    cq = np.exp(0.5 * np.sum(xq * xq, -1, keepdims=True) - 4 * np.linalg.norm(xq, axis=-1, keepdims=True))
    ch = np.exp(0.5 * xk0 @ xk0 - 4 * np.linalg.norm(xk0))
    np.testing.assert_allclose(_causal_from_features(fq * cq, fk * ch, v), base, rtol=1e-9, atol=1e-12)
    rng = np.random.default_rng(5)
    cr = np.exp(rng.uniform(-20, 20, size=(q.shape[0], 1)))
    np.testing.assert_allclose(_causal_from_features(fq * cr, fk * np.exp(7.5), v), base, rtol=1e-9, atol=1e-12)
    # a constant per key token does not cancel (the reason none is used)
    ck = np.exp(rng.uniform(-1, 1, size=(k.shape[0], 1)))
    assert np.max(np.abs(_causal_from_features(fq, fk * ck, v) - base)) > 1e-3


def test_unshifted_float32_features_fail_at_fourteen_times_the_norm():
    omega = synth.draw_omega(256, 64)
    q, k, v = _inputs(14.0)
    ref = ora.recurrent_attention(q[None, None], k[None, None], v[None, None], phi="favor", omega=omega)[0][0, 0]
    assert np.all(np.isfinite(ref))

    def phi32(u):
        x = (u / 64 ** 0.25).astype(np.float32)
        a = x @ omega.astype(np.float32).T - np.float32(0.5) * np.sum(x * x, -1, keepdims=True)
        return np.exp(a) / np.float32(16.0)

    with np.errstate(all="ignore"):
        A = np.tril(phi32(q) @ phi32(k).T)
        den = A.sum(-1)
    assert np.mean(den == 0) > 0.5  # most rows have no representable weight left


def test_shifted_float32_features_stay_in_range_at_fourteen_times_the_norm():
    omega = synth.draw_omega(256, 64)
    q, k, v = _inputs(14.0)
    ref = ora.recurrent_attention(q[None, None], k[None, None], v[None, None], phi="favor", omega=omega)[0][0, 0]
    om32 = omega.astype(np.float32)

    def x32(u):
        return (u / 64 ** 0.25).astype(np.float32)

    xq, xk = x32(q), x32(k)
    fq = np.exp(xq @ om32.T - 4 * np.linalg.norm(xq, axis=-1, keepdims=True)) / np.float32(16.0)
    kap = np.float32(0.5) * xk[0] @ xk[0] - 4 * np.linalg.norm(xk[0])
    fk = np.exp(xk @ om32.T - np.float32(0.5) * np.sum(xk * xk, -1, keepdims=True) + kap) / np.float32(16.0)
    assert np.all(np.isfinite(fq)) and np.all(np.isfinite(fk))
    out = _causal_from_features(fq.astype(np.float64), fk.astype(np.float64), v)
    np.testing.assert_allclose(out, ref, rtol=1e-3, atol=1e-3)
