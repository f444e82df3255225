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
