"""GPU parity of the per-token gated (SSD scalar-decay form) prefill and
decode, la_forward_gated and la_decode_step_gated, against the fp64 oracle
(oracle/gated.py), which is given the gates a_t = exp(log a_t) of exactly
the fp32 log gates the GPU reads.

Tolerances: normalised outputs follow the undecayed rule (fp32 I/O max
|err| <= 1e-4; bf16 |err| <= 2e-2 + 2e-2 |ref|).  Unnormalised outputs are
sums whose terms have random signs, so the bound is taken relative to the
row's scale: |err| <= 2e-2 |ref| + 2e-2 den_t max|v| (bf16) or
1e-5 (|ref| + den_t max|v|) (fp32), with den_t = sum_j L_tj w_j > 0 (ELU+1
features).  The library clamps each log2 gate at -126; a zero gate's
2^-126 leaves nothing an fp32 sum resolves, so resets are compared with the
oracle's exact zero.
"""

import numpy as np
import pytest

from oracle import decay as dec
from oracle import gated as gat
from oracle import heads
from oracle import linear_attention as ora
from kernelized_linear_attention_elu_amd import synth
from tests.gpu_util import check_close, check_rows, f32_dev, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(lib, q, k, v, log_a, io="bf16", **kw):
    import torch
    Q, K, V = (to_dev(x, io) for x in (q, k, v))
    res = lib.forward(Q, K, V, log_gate=f32_dev(log_a), **kw)
    torch.cuda.synchronize()
    return res


def _gates(log_a):
    return np.exp(np.asarray(log_a, dtype=np.float64))


def _den(q, k, a, phi="elu1"):
    """den_t = sum_j L_tj phi(q_t).phi(k_j): the unnormalised output for V = 1."""
    ones = np.ones(q.shape[:-1] + (1,))
    return gat.explicit_gated(q, k, ones, a, phi=phi, normalize=False)[..., 0]


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


def _check(got, ref, q, k, a, v, io, normalize, what):
    if normalize:
        check_close(got, ref, io, what)
    else:
        _check_unnormalised(got, ref, _den(q, k, a), v, io, what)


@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("N,chunk,io,tokens,resets", [
    (1, 64, "bf16", None, 0), (17, 64, "bf16", None, 0), (300, 64, "bf16", None, 0), (300, 64, "bf16", 128, 3),
    (300, 16, "bf16", 64, 0), (300, 32, "bf16", None, 2), (300, 128, "bf16", None, 0), (300, 128, "bf16", 128, 4),
    (300, 64, "f32", 128, 2), (100, 16, "f32", None, 0),
])
def test_gated_small(lib, span, N, chunk, io, tokens, resets, normalize):
    """Outputs and final state; ragged tails, several chunks and (with the
    span override) several spans per head, so that the chunk gates, the span
    totals, their scan and the in-span carry are all exercised; zero gates
    (resets) at seeded positions."""
    span(tokens)
    q, k, v = synth.draw_qkv(1, 3, N, 64, 64, seed=41, io=io)
    log_a = synth.draw_log_gates(1, 3, N, seed=42, resets=resets)
    a = _gates(log_a)
    O, S, z = _run(lib, q, k, v, log_a, io=io, chunk=chunk, normalize=normalize, return_state=True)
    ref, S_ref, z_ref = gat.recurrent_gated(q, k, v, a, normalize=normalize)
    _check(to_host(O), ref, q, k, a, v, io, normalize, "O")
    check_close(to_host(S), S_ref, io, "S_N")
    check_close(to_host(z), z_ref, io, "z_N")


def test_gated_wide_heads(lib, span):
    """d = d_v = 128 (eight waves per workgroup), two sequences."""
    span(128)
    q, k, v = synth.draw_qkv(2, 2, 333, 128, 128, seed=43)
    log_a = synth.draw_log_gates(2, 2, 333, seed=44, resets=1)
    O, S, z = _run(lib, q, k, v, log_a, return_state=True)
    ref, S_ref, z_ref = gat.recurrent_gated(q, k, v, _gates(log_a))
    check_close(to_host(O), ref, "bf16", "O")
    check_close(to_host(S), S_ref, "bf16", "S_N")
    check_close(to_host(z), z_ref, "bf16", "z_N")


def test_gated_unit_and_constant_gates(lib, span):
    """All gates one: the plain causal result; a constant gate per head: the
    fixed decay (against both oracles, and the two library paths against
    each other)."""
    import torch
    span(128)
    q, k, v = synth.draw_qkv(1, 3, 400, 64, 64, seed=45)
    O1 = to_host(_run(lib, q, k, v, np.zeros((1, 3, 400), np.float32)))
    ref, _, _ = ora.recurrent_attention(q, k, v)
    check_close(O1, ref, "bf16", "unit gates")
    gam = np.array([0.5, 0.9, 0.999], np.float32)
    log_a = np.broadcast_to(np.log(gam.astype(np.float64))[None, :, None], (1, 3, 400)).astype(np.float32)
    for normalize in (True, False):
        Og = to_host(_run(lib, q, k, v, log_a, normalize=normalize))
        a = _gates(log_a)
        ref, _, _ = dec.recurrent_decay(q, k, v, a[0, :, 0], normalize=normalize)
        _check(Og, ref, q, k, a, v, "bf16", normalize, f"constant gates normalize={normalize}")
        Od = lib.forward(*(to_dev(x, "bf16") for x in (q, k, v)), gamma=f32_dev(gam), normalize=normalize)
        torch.cuda.synchronize()
        _check(Og, to_host(Od), q, k, a, v, "bf16", normalize, "gated vs decay path")


def test_gated_page_illustration_on_gpu(lib):
    """The decay page's figure through constant gates (a = 0.99: weight 0.366
    at lag 100): identity features, unnormalised read-out, d = 1 zero-padded
    to 64, fp32 I/O."""
    N = 130
    q = np.zeros((1, 1, N, 64), np.float32); q[..., 0] = 1.0
    k = np.zeros_like(q); k[0, 0, 0, 0] = 1.0
    v = np.zeros_like(q); v[0, 0, 0, 0] = 1.0
    log_a = np.full((1, 1, N), np.log(0.99), np.float32)
    O = to_host(_run(lib, q, k, v, log_a, io="f32", phi="identity", normalize=False))
    assert round(O[0, 0, 100, 0], 3) == 0.366
    np.testing.assert_allclose(O[0, 0, :, 0], np.exp(np.arange(N) * np.float64(log_a[0, 0, 0])), rtol=1e-5, atol=0)
    assert np.all(O[..., 1:] == 0.0)


def test_gated_zero_gate_resets(lib, span):
    """A zero gate at a chunk start, inside a chunk, at a span start and at
    the last token: from there on the outputs equal a fresh run started at
    that token (within the tolerance: the library's 2^-126 for a zero gate
    leaves the earlier state in at that scale)."""
    span(128)
    N = 400
    q, k, v = synth.draw_qkv(1, 2, N, 64, 64, seed=46)
    base = synth.draw_log_gates(1, 2, N, seed=47)
    for t0 in (64, 77, 256, N - 1):
        log_a = base.copy()
        log_a[..., t0] = -np.inf
        O = to_host(_run(lib, q, k, v, log_a))
        ref, _, _ = gat.recurrent_gated(q, k, v, _gates(log_a))
        check_close(O, ref, "bf16", f"reset at {t0}")
        fresh = to_host(_run(lib, q[:, :, t0:], k[:, :, t0:], v[:, :, t0:], log_a[:, :, t0:]))
        check_close(O[:, :, t0:], fresh, "bf16", f"fresh run from {t0}")


def test_gated_split_prefill_and_decode(lib, span):
    """Prefill, prefill from its state, then decode steps: all equal the one
    gated recurrence (normalised and not)."""
    import torch
    span(128)
    B, H, N = 1, 3, 520
    q, k, v = synth.draw_qkv(B, H, N, 64, 64, seed=48)
    log_a = synth.draw_log_gates(B, H, N, seed=49, resets=1)
    a = _gates(log_a)
    for normalize in (True, False):
        ref, S_ref, z_ref = gat.recurrent_gated(q, k, v, a, normalize=normalize)
        den = _den(q, k, a)
        cut, end = 301, 517
        O1, S1, z1 = _run(lib, q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], log_a[:, :, :cut], normalize=normalize,
                          return_state=True)
        O2, S2, z2 = _run(lib, q[:, :, cut:end], k[:, :, cut:end], v[:, :, cut:end], log_a[:, :, cut:end],
                          normalize=normalize, S0=S1, z0=z1, return_state=True)
        got = np.concatenate([to_host(O1), to_host(O2)], axis=2)
        if normalize:
            check_close(got, ref[:, :, :end], "bf16", "split prefill")
        else:
            _check_unnormalised(got, ref[:, :, :end], den[:, :, :end], v, "bf16", "split prefill")
        for t in range(end, N):
            o = lib.decode_step(S2, z2, to_dev(q[:, :, t], "bf16"), to_dev(k[:, :, t], "bf16"),
                                to_dev(v[:, :, t], "bf16"), log_gate=f32_dev(np.ascontiguousarray(log_a[:, :, t])),
                                normalize=normalize)
            torch.cuda.synchronize()
            if normalize:
                check_close(to_host(o), ref[:, :, t], "bf16", f"decode t={t}")
            else:
                _check_unnormalised(to_host(o), ref[:, :, t], den[:, :, t], v, "bf16", f"decode t={t}")
        check_close(to_host(S2), S_ref, "bf16", "S after decode")
        check_close(to_host(z2), z_ref, "bf16", "z after decode")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("normalize", [True, False])
def test_decode_gated_step(lib, io, normalize):
    """One gated decode step from a random state, d = 64 and 128, one zero
    gate among the (batch, head) pairs."""
    import torch
    for d in (64, 128):
        rng = np.random.default_rng(50 + d)
        S = np.abs(rng.standard_normal((2, 3, d, d))).astype(np.float32)
        z = (np.abs(rng.standard_normal((2, 3, d))) + 1.0).astype(np.float32)
        q, k, v = synth.draw_decode_token(2, 3, d, d, seed=51, io=io)
        log_a = synth.draw_log_gates(2, 3, 1, seed=52)[..., 0]
        log_a[1, 2] = -np.inf
        o_ref, S_ref, z_ref = gat.decode_step_gated(S, z, q, k, v, _gates(log_a), normalize=normalize)
        Sd, zd = f32_dev(S), f32_dev(z)
        o = lib.decode_step(Sd, zd, to_dev(q, io), to_dev(k, io), to_dev(v, io), log_gate=f32_dev(log_a),
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


def test_gated_no_future_leakage_bitwise(lib, span):
    """Changing the keys, values and gates from t0 on leaves every output
    before t0 bit-identical."""
    span(128)
    q, k, v = synth.draw_qkv(1, 3, 400, 64, 64, seed=53)
    log_a = synth.draw_log_gates(1, 3, 400, seed=54)
    base = to_host(_run(lib, q, k, v, log_a))
    for t0 in (256, 200, 37):
        k2, v2, g2 = k.copy(), v.copy(), log_a.copy()
        k2[..., t0:, :] = synth.round_to_io(k2[..., t0:, :] + 1.0, "bf16")
        v2[..., t0:, :] = synth.round_to_io(v2[..., t0:, :] - 2.0, "bf16")
        g2[..., t0:] = -np.inf
        out = to_host(_run(lib, q, k2, v2, g2))
        np.testing.assert_array_equal(out[..., :t0, :], base[..., :t0, :])
        assert np.max(np.abs(out[..., t0:, :] - base[..., t0:, :])) > 1e-3


def _gated_head(q, k, v, a):
    return gat.recurrent_gated(q, k, v, a)


def test_gated_long_workload_full(lib):
    """The long workload (B1 H32 N32768 d64 bf16) with the seeded gates of
    synth.draw_log_gates, in the bench's launch configuration: every output of
    every head against the fp64 gated recurrence, and the final state."""
    w = synth.WORKLOADS["long"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    log_a = synth.draw_log_gates(w.B, w.H, w.N)
    O, S, z = _run(lib, q, k, v, log_a, return_state=True)
    O, S, z = to_host(O), to_host(S), to_host(z)
    ref, S_ref, z_ref = heads.map_heads(_gated_head, q, k, v, _gates(log_a))
    _, _, worst = check_close(O, ref, "bf16", "O")
    print(f"gated long: worst row relative error {worst:.3e}", flush=True)
    check_close(S, S_ref, "bf16", "S_N")
    check_close(z, z_ref, "bf16", "z_N")


def test_gated_wide_workload_full(lib):
    """The wide workload (B2 H16 N65536 d128 bf16) with the seeded per-token
    gates, in the bench's launch configuration: every output of every
    (batch, head) against the fp64 gated recurrence."""
    w = synth.WORKLOADS["wide"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    log_a = synth.draw_log_gates(w.B, w.H, w.N)
    O = to_host(_run(lib, q, k, v, log_a))
    ref, _, _ = heads.map_heads(_gated_head, q, k, v, _gates(log_a))
    _, _, worst = check_close(O, ref, "bf16", "O")
    print(f"gated wide: worst row relative error {worst:.3e}", flush=True)
