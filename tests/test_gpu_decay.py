"""GPU parity of the decayed (RetNet-form) prefill and decode, la_forward_decay
and la_decode_step_decay, against the fp64 oracle (oracle/decay.py).

Tolerances.  Normalised outputs: the rule of the undecayed path (fp32 I/O
max |err| <= 1e-4; bf16 |err| <= 2e-2 + 2e-2 |ref|).  Unnormalised outputs
o_t = sum_j gamma^(t-j) w_j v_j are sums whose terms have random signs, so a
bound relative to |o_t| alone fails where they cancel; the bound is taken
relative to the row's scale instead: |err| <= 2e-2 |ref| + 2e-2 den_t max|v|
(bf16) or 1e-5 den_t max|v| (fp32), with den_t = sum_j gamma^(t-j) w_j > 0
(ELU+1 features).  The bf16 rounding of the features and of the carried
state contributes at most about 2^-9 den_t max|v|.
"""

import numpy as np
import pytest

from oracle import decay as dec
from oracle import heads
from oracle import linear_attention as ora
from kernelized_linear_attention_elu_amd import synth
from tests.gpu_util import check_close, check_rows, f32_dev, to_dev, to_host

pytestmark = pytest.mark.gpu

GAMMAS3 = np.array([0.5, 0.9, 0.999], dtype=np.float32)


def _run(lib, q, k, v, gamma, io="bf16", **kw):
    import torch
    Q, K, V = (to_dev(x, io) for x in (q, k, v))
    res = lib.forward(Q, K, V, gamma=f32_dev(gamma), **kw)
    torch.cuda.synchronize()
    return res


def _check_unnormalised(got, ref, den, v, io, what):
    got = np.asarray(got, dtype=np.float64)
    scale = den[..., None] * np.max(np.abs(v))
    if io == "f32":
        bound = 1e-5 * scale + 1e-5 * np.abs(ref)
    else:
        bound = 2e-2 * np.abs(ref) + 2e-2 * scale
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert np.all(err <= bound), (f"{what}: worst at {worst}: got {got[worst]!r} ref {ref[worst]!r} "
                                  f"bound {bound[worst]:.3e}")
    check_rows(got, ref, io, what)


def _den(q, k, gamma, phi="elu1"):
    """den_t = sum_j gamma^(t-j) phi(q_t).phi(k_j): the unnormalised output for V = 1."""
    ones = np.ones(q.shape[:-1] + (1,))
    return dec.explicit_decay(q, k, ones, gamma, phi=phi, normalize=False)[..., 0]


@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("N,chunk,io,tokens", [
    (1, 64, "bf16", None), (17, 64, "bf16", None), (300, 64, "bf16", None), (300, 64, "bf16", 128),
    (300, 16, "bf16", 64), (300, 32, "bf16", None), (300, 128, "bf16", None),
    (300, 64, "f32", 128), (100, 16, "f32", None),
])
def test_decay_small(lib, span, N, chunk, io, tokens, normalize):
    """Outputs and final state; ragged tails, several chunks and (with the
    span override) several spans per head, so that the span sums, their
    decayed scan and the in-span carry are all exercised."""
    span(tokens)
    q, k, v = synth.draw_qkv(1, 3, N, 64, 64, seed=31, io=io)
    O, S, z = _run(lib, q, k, v, GAMMAS3, io=io, chunk=chunk, normalize=normalize, return_state=True)
    ref, S_ref, z_ref = dec.recurrent_decay(q, k, v, GAMMAS3.astype(np.float64), normalize=normalize)
    if normalize:
        check_close(to_host(O), ref, io, "O")
    else:
        _check_unnormalised(to_host(O), ref, _den(q, k, GAMMAS3.astype(np.float64)), v, io, "O")
    check_close(to_host(S), S_ref, io, "S_N")
    check_close(to_host(z), z_ref, io, "z_N")


def test_decay_wide_heads(lib, span):
    """d = d_v = 128 (eight waves per workgroup)."""
    span(128)
    q, k, v = synth.draw_qkv(2, 2, 333, 128, 128, seed=32)
    g = np.array([0.7, 0.995], dtype=np.float32)
    O, S, z = _run(lib, q, k, v, g, return_state=True)
    ref, S_ref, z_ref = dec.recurrent_decay(q, k, v, g.astype(np.float64))
    check_close(to_host(O), ref, "bf16", "O")
    check_close(to_host(S), S_ref, "bf16", "S_N")
    check_close(to_host(z), z_ref, "bf16", "z_N")


def test_decay_gamma_one_is_the_plain_path(lib, span):
    span(128)
    q, k, v = synth.draw_qkv(1, 2, 400, 64, 64, seed=33)
    O1 = to_host(_run(lib, q, k, v, np.ones(2, dtype=np.float32)))
    import torch
    O0 = lib.forward(*(to_dev(x, "bf16") for x in (q, k, v)))
    torch.cuda.synchronize()
    ref, _, _ = ora.recurrent_attention(q, k, v)
    check_close(O1, ref, "bf16", "gamma = 1")
    check_close(to_host(O0), ref, "bf16", "plain")


def test_decay_page_illustration_on_gpu(lib):
    """The page's figure (gamma = 0.99: weight 0.366 at lag 100) through the
    library: identity features, the page's unnormalised read-out, d = 1
    zero-padded to 64 (exact), fp32 I/O."""
    N = 130
    q = np.zeros((1, 1, N, 64), np.float32); q[..., 0] = 1.0
    k = np.zeros_like(q); k[0, 0, 0, 0] = 1.0
    v = np.zeros_like(q); v[0, 0, 0, 0] = 1.0
    O = to_host(_run(lib, q, k, v, np.array([0.99], np.float32), io="f32", phi="identity", normalize=False))
    assert round(O[0, 0, 100, 0], 3) == 0.366
    np.testing.assert_allclose(O[0, 0, :, 0], 0.99 ** np.arange(N), rtol=0, atol=1e-5)
    assert np.all(O[..., 1:] == 0.0)


def test_decay_split_prefill_and_decode(lib, span):
    """Prefill, prefill from its state, then decode steps: all equal the one
    decayed recurrence (normalised and not)."""
    import torch
    span(128)
    q, k, v = synth.draw_qkv(1, 3, 520, 64, 64, seed=34)
    g = GAMMAS3.astype(np.float64)
    gd = f32_dev(GAMMAS3)
    for normalize in (True, False):
        ref, S_ref, z_ref = dec.recurrent_decay(q, k, v, g, normalize=normalize)
        den = _den(q, k, g)
        cut, end = 301, 517
        O1, S1, z1 = _run(lib, q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], GAMMAS3, normalize=normalize,
                          return_state=True)
        O2, S2, z2 = _run(lib, q[:, :, cut:end], k[:, :, cut:end], v[:, :, cut:end], GAMMAS3, normalize=normalize,
                          S0=S1, z0=z1, return_state=True)
        got = np.concatenate([to_host(O1), to_host(O2)], axis=2)
        if normalize:
            check_close(got, ref[:, :, :end], "bf16", "split prefill")
        else:
            _check_unnormalised(got, ref[:, :, :end], den[:, :, :end], v, "bf16", "split prefill")
        for t in range(end, 520):
            o = lib.decode_step(S2, z2, to_dev(q[:, :, t], "bf16"), to_dev(k[:, :, t], "bf16"),
                                to_dev(v[:, :, t], "bf16"), gamma=gd, normalize=normalize)
            torch.cuda.synchronize()
            if normalize:
                check_close(to_host(o), ref[:, :, t], "bf16", f"decode t={t}")
            else:
                _check_unnormalised(to_host(o), ref[:, :, t], den[:, :, t], v, "bf16", f"decode t={t}")
        check_close(to_host(S2), S_ref, "bf16", "S after decode")
        check_close(to_host(z2), z_ref, "bf16", "z after decode")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("normalize", [True, False])
def test_decode_decay_step(lib, io, normalize):
    """One decode step from a random state, d = 64 and 128, against the oracle."""
    import torch
    for d in (64, 128):
        rng = np.random.default_rng(35 + d)
        S = np.abs(rng.standard_normal((2, 3, d, d))).astype(np.float32)
        z = (np.abs(rng.standard_normal((2, 3, d))) + 1.0).astype(np.float32)
        q, k, v = synth.draw_decode_token(2, 3, d, d, seed=36, io=io)
        o_ref, S_ref, z_ref = dec.decode_step_decay(S, z, q, k, v, GAMMAS3.astype(np.float64), normalize=normalize)
        Sd, zd = f32_dev(S), f32_dev(z)
        o = lib.decode_step(Sd, zd, to_dev(q, io), to_dev(k, io), to_dev(v, io), gamma=f32_dev(GAMMAS3),
                            normalize=normalize)
        torch.cuda.synchronize()
        if normalize:
            check_close(to_host(o), o_ref, io, f"o d={d}")
        else:
            np.testing.assert_allclose(to_host(o), o_ref, rtol=2e-2 if io == "bf16" else 1e-5,
                                       atol=2e-2 * np.abs(o_ref).max())
            check_rows(to_host(o), o_ref, io, f"o d={d}")
        np.testing.assert_allclose(to_host(Sd), S_ref, rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(to_host(zd), z_ref, rtol=1e-6, atol=1e-6)


def test_decay_no_future_leakage_bitwise(lib, span):
    span(128)
    q, k, v = synth.draw_qkv(1, 3, 400, 64, 64, seed=37)
    base = to_host(_run(lib, q, k, v, GAMMAS3))
    for t0 in (256, 200, 37):
        k2, v2 = k.copy(), v.copy()
        k2[..., t0:, :] = synth.round_to_io(k2[..., t0:, :] + 1.0, "bf16")
        v2[..., t0:, :] = synth.round_to_io(v2[..., t0:, :] - 2.0, "bf16")
        out = to_host(_run(lib, q, k2, v2, GAMMAS3))
        np.testing.assert_array_equal(out[..., :t0, :], base[..., :t0, :])
        assert np.max(np.abs(out[..., t0:, :] - base[..., t0:, :])) > 1e-3


def _decay_head(q, k, v, gamma):
    return dec.recurrent_decay(q, k, v, gamma)


def test_decay_long_workload_full(lib):
    """The long workload (B1 H32 N32768 d64 bf16) with the per-head decays of
    synth.decay_gammas, in the bench's launch configuration: every output of
    every head against the fp64 decayed recurrence, and the final state."""
    w = synth.WORKLOADS["long"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    g = synth.decay_gammas(w.H)
    O, S, z = _run(lib, q, k, v, g, return_state=True)
    O, S, z = to_host(O), to_host(S), to_host(z)
    ref, S_ref, z_ref = heads.map_heads(_decay_head, q, k, v, head_kw=lambda b, h: {"gamma": float(g[h])})
    _, _, worst = check_close(O, ref, "bf16", "O")
    print(f"decay long: worst row relative error {worst:.3e}", flush=True)
    check_close(S, S_ref, "bf16", "S_N")
    check_close(z, z_ref, "bf16", "z_N")


def test_decay_wide_workload_full(lib):
    """The wide workload (B2 H16 N65536 d128 bf16) with the per-head decays of
    synth.decay_gammas, in the bench's launch configuration: every output of
    every (batch, head) against the fp64 decayed recurrence."""
    w = synth.WORKLOADS["wide"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    g = synth.decay_gammas(w.H)
    O = to_host(_run(lib, q, k, v, g))
    ref, _, _ = heads.map_heads(_decay_head, q, k, v, head_kw=lambda b, h: {"gamma": float(g[h])})
    _, _, worst = check_close(O, ref, "bf16", "O")
    print(f"decay wide: worst row relative error {worst:.3e}", flush=True)
