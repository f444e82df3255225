"""GPU parity of the backward pass (la_backward) against the fp64 gradient
oracle (oracle/backward.py): dQ, dK, dV of sum(dO * O), with O the
library's own forward output for the same bf16 Q, K, V (as a training step
would pass it).

Gates (tests/gates.py, check_grad): per head, the relative RMS error of the
whole gradient array <= 3e-2; per block of 64 rows <= 5e-2; per row, the
error <= 1e-1 of the row's norm or <= 2^-4 of the magnitude of the two sums
the kernels form for it (tests/grad_scales.py), whichever is larger.
Every row is compared, at the long workload too.
"""

import numpy as np
import pytest

from oracle import backward as bwd
from oracle import heads
from kernelized_linear_attention_elu_amd import synth
from tests.gates import check_grad
from tests.grad_scales import grad_scales
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


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


def _check_all(got, q, k, v, dO, phi="elu1"):
    refs = bwd.grad_causal(q, k, v, dO, phi=phi)
    scales = grad_scales(q, k, v, dO, phi=phi)
    worst = []
    for name, g, r, sc in zip(("dQ", "dK", "dV"), got, refs, scales):
        worst.append(check_grad(g, r, sc, name))
    return worst


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
    _check_all(_run(lib, q, k, v, dO, phi), q, k, v, dO, phi)


@pytest.mark.parametrize("phi", ["elu1", "identity"])
@pytest.mark.parametrize("N,tokens", [(17, None), (300, None), (333, 128)])
def test_backward_wide_heads(lib, span, N, tokens, phi):
    """d = d_v = 128: eight waves, two per 16-row block, each with half of the
    feature and value tiles."""
    span(tokens)
    q, k, v, dO = _draw(2, 2, N, 95 + N, phi, d=128)
    _check_all(_run(lib, q, k, v, dO, phi), q, k, v, dO, phi)


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


def _grad_rows_all(q, k, v, dO):
    return bwd.grad_rows(q, k, v, dO, range(q.shape[-2]))


def test_backward_long_workload_full(lib):
    """The long workload (B1 H32 N32768 d64 bf16) in the bench's launch
    configuration: dQ, dK, dV at every row of every head against the fp64
    prefix/suffix gradient loops."""
    w = synth.WORKLOADS["long"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    rng = np.random.default_rng(91)
    dO = synth.round_to_io(rng.standard_normal((w.B, w.H, w.N, w.dv), dtype=np.float32), "bf16")
    got = _run(lib, q, k, v, dO)
    refs = heads.map_heads(_grad_rows_all, q, k, v, dO)
    scales = heads.map_heads(grad_scales, q, k, v, dO)
    for name, g, r, sc in zip(("dQ", "dK", "dV"), got, refs, scales):
        head, block, row = check_grad(g, r, sc, name)
        print(f"backward long {name}: head RMS error {head:.3e}, block RMS error {block:.3e}, "
              f"worst row {row:.3f} of its bound", flush=True)


def test_backward_wide_workload_full(lib):
    """The wide workload (B2 H16 N65536 d128 bf16) in the bench's launch
    configuration (eight waves per workgroup, the reverse sums in a pass of
    their own): dQ, dK, dV at every row of every (batch, head) against the
    fp64 prefix/suffix gradient loops."""
    w = synth.WORKLOADS["wide"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    rng = np.random.default_rng(92)
    dO = synth.round_to_io(rng.standard_normal((w.B, w.H, w.N, w.dv), dtype=np.float32), "bf16")
    got = _run(lib, q, k, v, dO)
    refs = heads.map_heads(_grad_rows_all, q, k, v, dO)
    scales = heads.map_heads(grad_scales, q, k, v, dO)
    del q, k, v, dO
    for name, g, r, sc in zip(("dQ", "dK", "dV"), got, refs, scales):
        head, block, row = check_grad(g, r, sc, name)
        print(f"backward wide {name}: head RMS error {head:.3e}, block RMS error {block:.3e}, "
              f"worst row {row:.3f} of its bound", flush=True)
