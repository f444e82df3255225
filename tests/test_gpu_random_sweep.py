"""Seeded random sweep over the prefill and backward entry points against
the fp64 oracle: plain causal and non-causal (bf16 and fp32), fixed decay,
per-token gates, per-channel gates, FAVOR+ and the backward, each at a
random size (B <= 2, H <= 3, N < 700), dimension, chunk and span split;
and single decode steps of every kind from random states.
Outputs use the tolerance rule of the other parity tests; final states
(fp32 sums over up to 700 tokens) are bounded as in the fp32 tiny test,
rtol 1e-5 + atol 1e-4, and by the bf16 rule for bf16 I/O."""

import numpy as np
import pytest

from oracle import backward as bwd
from oracle import decay as dec
from oracle import gated as gat
from oracle import gla as glo
from oracle import linear_attention as ora
from kernelized_linear_attention_elu_amd import synth
from tests.gates import check_grad
from tests.grad_scales import grad_scales
from tests.gpu_util import check_close, f32_dev, to_dev, to_host
from tests.test_gpu_gla import FLOOR

pytestmark = pytest.mark.gpu

KINDS = ["plain", "plain", "noncausal", "decay", "gated", "gla", "favor", "backward", "decode"]


def _check_state(got, ref, io, what):
    if io == "f32":
        np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-4, err_msg=what)
    else:
        check_close(got, ref, io, what)


def _case(lib, rng, om, span_set):
    import torch
    pick = lambda xs: xs[int(rng.integers(0, len(xs)))]
    kind = pick(KINDS)
    if kind == "decode":
        return _decode_case(lib, rng, pick)
    B, H, N = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 700))
    io, d, chunk = "bf16", 64, 64
    if kind in ("plain", "noncausal", "decay", "gated"):
        io = pick(["bf16", "bf16", "f32"])
        d = 64 if io == "f32" else pick([64, 64, 128])
        chunk = pick([16, 32, 64, 128] if (io == "bf16" and d == 64) else [16, 32, 64])
    elif kind == "gla":
        d = pick([64, 64, 128])
        chunk = pick([16, 32, 64, 128]) if d == 64 else pick([16, 32])
    elif kind == "backward":
        d = pick([64, 128])
    span = pick([None, None, chunk, 2 * chunk, 3 * chunk])
    seed = int(rng.integers(0, 2**31))
    what = f"{kind} B{B} H{H} N{N} d{d} {io} chunk {chunk} span {span} seed {seed}"
    span_set(span)
    q, k, v = synth.draw_qkv(B, H, N, d, d, seed=seed, io=io)
    Q, K, V = (to_dev(x, io) for x in (q, k, v))
    if kind in ("plain", "noncausal"):
        causal = kind == "plain"
        O, S, z = lib.forward(Q, K, V, chunk=chunk, causal=causal, return_state=True)
        torch.cuda.synchronize()
        ref, S_ref, z_ref = (ora.recurrent_attention if causal else ora.noncausal_attention)(q, k, v)
        check_close(to_host(O), ref, io, what + " O")
        _check_state(to_host(S), S_ref, io, what + " S")
        _check_state(to_host(z), z_ref, io, what + " z")
    elif kind == "decay":
        g = (np.float32(1.0) - np.float32(2.0) ** (-rng.uniform(3, 10, size=H)).astype(np.float32)).astype(np.float32)
        O = lib.forward(Q, K, V, chunk=chunk, gamma=f32_dev(g))
        torch.cuda.synchronize()
        check_close(to_host(O), dec.recurrent_decay(q, k, v, g.astype(np.float64))[0], io, what)
    elif kind == "gated":
        log_a = synth.draw_log_gates(B, H, N, seed=seed + 1)
        O = lib.forward(Q, K, V, chunk=chunk, log_gate=f32_dev(log_a))
        torch.cuda.synchronize()
        check_close(to_host(O), gat.recurrent_gated(q, k, v, np.exp(log_a.astype(np.float64)))[0], io, what)
    elif kind == "gla":
        log_a = synth.draw_log_gates_ch(B, H, N, d, seed=seed + 2)
        O = lib.forward(Q, K, V, chunk=chunk, log_gate_ch=f32_dev(log_a))
        torch.cuda.synchronize()
        al = np.maximum(np.exp(log_a.astype(np.float64)), FLOOR)
        check_close(to_host(O), glo.recurrent_gla(q, k, v, al)[0], io, what)
    elif kind == "favor":
        causal = bool(rng.integers(0, 2))
        O = lib.forward(Q, K, V, phi="favor", omega=f32_dev(om), causal=causal)
        torch.cuda.synchronize()
        ref = (ora.recurrent_attention if causal else ora.noncausal_attention)(q, k, v, phi="favor", omega=om)[0]
        check_close(to_host(O), ref, io, what)
    else:
        dO = synth.round_to_io(np.random.default_rng(seed + 3).standard_normal((B, H, N, d), dtype=np.float32),
                               "bf16")
        O = lib.forward(Q, K, V)
        grads = lib.backward(Q, K, V, O, to_dev(dO, "bf16"))
        torch.cuda.synchronize()
        for nm, gt, rf, sc in zip(("dQ", "dK", "dV"), grads, bwd.grad_causal(q, k, v, dO), grad_scales(q, k, v, dO)):
            check_grad(to_host(gt), rf, sc, f"{what} {nm}")


def _decode_case(lib, rng, pick):
    """One decode step (plain, FAVOR+, decay, gated, per-channel gated) from
    a random state: o, S', z' against the oracle's step."""
    import torch
    sub = pick(["plain", "plain", "favor", "decay", "gated", "gla"])
    B, H = int(rng.integers(1, 65)), int(rng.integers(1, 9))
    d = pick([64, 128])
    io = pick(["bf16", "f32"]) if sub == "plain" else "bf16"
    seed = int(rng.integers(0, 2**31))
    what = f"decode {sub} B{B} H{H} d{d} {io} seed {seed}"
    phi, om = ("favor", synth.draw_omega(256, d)) if sub == "favor" else ("elu1", None)
    r = 256 if sub == "favor" else d
    g = np.random.default_rng(seed)
    S = g.standard_normal((B, H, r, d)).astype(np.float32)
    z = g.uniform(1.0, 100.0, (B, H, r)).astype(np.float32)
    q, k, v = (np.ascontiguousarray(x[:, :, 0]) for x in synth.draw_qkv(B, H, 1, d, d, seed=seed + 1, io=io))
    kw = {}
    if sub == "decay":
        gam = (np.float32(1.0) - np.float32(2.0) ** (-g.uniform(3, 10, size=H)).astype(np.float32)).astype(np.float32)
        kw["gamma"] = f32_dev(gam)
        ref = dec.decode_step_decay(S, z, q, k, v, gam.astype(np.float64))
    elif sub == "gated":
        log_a = synth.draw_log_gates(B, H, 1, seed=seed + 2)[:, :, 0]
        kw["log_gate"] = f32_dev(np.ascontiguousarray(log_a))
        ref = gat.decode_step_gated(S, z, q, k, v, np.exp(log_a.astype(np.float64)))
    elif sub == "gla":
        log_a = synth.draw_log_gates_ch(B, H, 1, d, seed=seed + 3)[:, :, 0]
        kw["log_gate_ch"] = f32_dev(np.ascontiguousarray(log_a))
        ref = glo.decode_step_gla(S, z, q, k, v, np.maximum(np.exp(log_a.astype(np.float64)), FLOOR))
    else:
        ref = ora.decode_step(S, z, q, k, v, phi=phi, omega=om)
    o, S1, z1 = lib.decode_step(f32_dev(S), f32_dev(z), to_dev(q, io), to_dev(k, io), to_dev(v, io), phi=phi,
                                omega=f32_dev(om) if om is not None else None, inplace=False, **kw)
    torch.cuda.synchronize()
    check_close(to_host(o), ref[0], io, what + " o")
    _check_state(to_host(S1), ref[1], "f32", what + " S'")
    _check_state(to_host(z1), ref[2], "f32", what + " z'")


@pytest.mark.parametrize("seed", [101, 202, 303])
def test_random_sweep(lib, span, seed):
    rng = np.random.default_rng(seed)
    om = synth.draw_omega(256, 64)
    for _ in range(60):
        _case(lib, rng, om, span)
