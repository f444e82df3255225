"""The Python binding rejects mis-shaped outputs and feature matrices before
anything reaches the C ABI (a buffer smaller than the call's sizes would
otherwise be written or read past its end), and ``out=`` buffers are filled
exactly as freshly allocated ones."""

import numpy as np
import pytest

from kernelized_linear_attention_elu_amd import synth
from tests.gpu_util import f32_dev, to_dev, to_host

pytestmark = pytest.mark.gpu


def _qkv(B=1, H=2, N=100, d=64, dv=64):
    q, k, v = synth.draw_qkv(B, H, N, d, dv, seed=21)
    return tuple(to_dev(x, "bf16") for x in (q, k, v))


def test_forward_rejects_wrong_out_shape(lib):
    import torch
    Q, K, V = _qkv()
    bad = torch.empty((1, 2, 99, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="out has shape"):
        lib.forward(Q, K, V, out=bad)


def test_forward_rejects_wrong_omega_width(lib):
    Q, K, V = _qkv()
    om = f32_dev(synth.draw_omega(256, 32))
    with pytest.raises(ValueError, match="omega"):
        lib.forward(Q, K, V, phi="favor", omega=om)
    with pytest.raises(ValueError, match="omega"):
        lib.forward(Q, K, V, phi="favor", omega=None)


def test_decode_rejects_wrong_shapes(lib):
    import torch
    Q, K, V = _qkv(N=10)
    _, S, z = lib.forward(Q, K, V, return_state=True)
    q, k, v = (t[:, :, -1].contiguous() for t in (Q, K, V))
    with pytest.raises(ValueError, match="out has shape"):
        lib.decode_step(S, z, q, k, v, out=torch.empty((1, 2, 32), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="decode shapes"):
        lib.decode_step(S, z, q, k, v[..., :32].contiguous())
    om = f32_dev(synth.draw_omega(256, 64))
    with pytest.raises(ValueError, match="feature rows"):
        lib.decode_step(S, z, q, k, v, phi="favor", omega=om)


def test_feature_map_out_matches_fresh(lib):
    import torch
    x = synth.draw_qkv(1, 1, 300, 64, 64, seed=22)[0]
    X = to_dev(x, "bf16")
    fresh = lib.feature_map(X)
    Y = torch.full(tuple(X.shape), float("nan"), dtype=torch.float32, device="cuda")
    got = lib.feature_map(X, out=Y)
    torch.cuda.synchronize()
    assert got is Y
    np.testing.assert_array_equal(to_host(Y), to_host(fresh))
    with pytest.raises(ValueError, match="out has shape"):
        lib.feature_map(X, out=torch.empty((1, 1, 300, 32), dtype=torch.float32, device="cuda"))


def test_decay_and_gate_arguments_are_checked(lib):
    """gamma [H], log_gate [B,H,N], log_gate_ch [B,H,N,r]: wrong shapes, two
    decays at once, a non-causal decayed call and normalize=False without a
    decay are refused before the C ABI."""
    import torch
    Q, K, V = _qkv()
    with pytest.raises(ValueError, match="gamma must have shape"):
        lib.forward(Q, K, V, gamma=f32_dev(np.full(3, 0.9, np.float32)))
    with pytest.raises(ValueError, match="log_gate must have shape"):
        lib.forward(Q, K, V, log_gate=f32_dev(np.zeros((1, 2, 99), np.float32)))
    with pytest.raises(ValueError, match="log_gate_ch must have shape"):
        lib.forward(Q, K, V, log_gate_ch=f32_dev(np.zeros((1, 2, 100, 32), np.float32)))
    with pytest.raises(ValueError, match="at most one"):
        lib.forward(Q, K, V, gamma=f32_dev(np.full(2, 0.9, np.float32)),
                    log_gate=f32_dev(np.zeros((1, 2, 100), np.float32)))
    with pytest.raises(ValueError, match="causal"):
        lib.forward(Q, K, V, causal=False, log_gate=f32_dev(np.zeros((1, 2, 100), np.float32)))
    with pytest.raises(ValueError, match="normalize=False"):
        lib.forward(Q, K, V, normalize=False)
    with pytest.raises(TypeError, match="log_gate must be"):
        lib.forward(Q, K, V, log_gate=torch.zeros((1, 2, 100), dtype=torch.bfloat16, device="cuda"))
    _, S, z = lib.forward(Q, K, V, return_state=True)
    q, k, v = (t[:, :, -1].contiguous() for t in (Q, K, V))
    with pytest.raises(ValueError, match="log_gate_ch must have shape"):
        lib.decode_step(S, z, q, k, v, log_gate_ch=f32_dev(np.zeros((1, 2), np.float32)))


def test_backward_arguments_and_out(lib):
    """Mis-shaped O / dO / out tensors are refused; out= buffers are filled
    exactly as freshly allocated ones."""
    import torch
    Q, K, V = _qkv()
    O = lib.forward(Q, K, V)
    dO = to_dev(synth.round_to_io(np.random.default_rng(23).standard_normal((1, 2, 100, 64),
                                                                         dtype=np.float32), "bf16"), "bf16")
    with pytest.raises(ValueError, match="shape mismatch"):
        lib.backward(Q, K, V, O[:, :, :99].contiguous(), dO)
    with pytest.raises(ValueError, match="dK has shape"):
        lib.backward(Q, K, V, O, dO, out=(torch.empty_like(Q), torch.empty_like(Q[:, :1]), torch.empty_like(V)))
    fresh = lib.backward(Q, K, V, O, dO)
    outs = tuple(torch.full_like(t, float("nan")) for t in (Q, K, V))
    got = lib.backward(Q, K, V, O, dO, out=outs)
    torch.cuda.synchronize()
    for a, b, c in zip(got, outs, fresh):
        assert a is b
        np.testing.assert_array_equal(to_host(a), to_host(c))
