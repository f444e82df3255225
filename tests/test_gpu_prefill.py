"""GPU parity of la_forward against the fp64 oracle.

Every case feeds the same seeded inputs (already rounded to the I/O type) to
the HIP library and to the oracle and compares element by element (full
outputs where the oracle finishes in seconds, sampled rows computed one by
one from the definition at the full workload sizes).
"""

import os

import numpy as np
import pytest

from oracle import linear_attention as ora
from kernelized_linear_attention_elu_amd import synth
from tests.golden import load
from tests.gpu_util import check_close, f32_dev, rel_rms_error, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=["single_pass", "three_kernel"])
def path(request, monkeypatch):
    """Every test runs on both prefill paths: the single-pass kernel (causal
    bf16 d = 64, chunk 64) and the three-kernel path (everything else, and
    everything when LA_FUSED=0)."""
    monkeypatch.setenv("LA_FUSED", "1" if request.param == "single_pass" else "0")
    return request.param


@pytest.fixture
def span(monkeypatch):
    """Set the LA_SPAN override (tokens per workgroup) for one test."""
    def _set(tokens):
        if tokens is None:
            monkeypatch.delenv("LA_SPAN", raising=False)
        else:
            monkeypatch.setenv("LA_SPAN", str(tokens))
    _set(None)
    return _set


def _run(lib, q, k, v, io, **kw):
    Q, K, V = (to_dev(x, io) for x in (q, k, v))
    out = lib.forward(Q, K, V, **kw)
    import torch
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------- hand examples

@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_worked_example_padded(lib, io):
    """The pages' 3-token example through the identity map, zero-padded to
    d = d_v = 64 (zero features add nothing to any dot product)."""
    g = load("worked_example.txt")
    q = np.zeros((1, 1, 3, 64), np.float32)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    q[0, 0, :, :2] = g["phi_q3"]
    k[0, 0, :, :2] = g["phi_k"]
    v[0, 0, :, :2] = g["v"]
    O, S, z = _run(lib, q, k, v, io, phi="identity", return_state=True)
    o = to_host(O)[0, 0]
    tol = 1e-6 if io == "f32" else 1e-2
    np.testing.assert_allclose(o[2, :2], g["o3"], atol=tol)
    np.testing.assert_allclose(o[0, :2], v[0, 0, 0, :2], atol=tol)     # o_1 = v_1
    np.testing.assert_array_equal(o[:, 2:], 0.0)
    Sh, zh = to_host(S)[0, 0], to_host(z)[0, 0]
    np.testing.assert_allclose(Sh[:2, :2], g["S3"], atol=1e-6)
    np.testing.assert_allclose(zh[:2], g["z3"], atol=1e-6)
    assert np.all(Sh[2:] == 0) and np.all(Sh[:, 2:] == 0) and np.all(zh[2:] == 0)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_same_key_twice_padded(lib, io):
    g = load("same_key_twice.txt")
    q = np.zeros((1, 1, 2, 64), np.float32)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    q[0, 0, :, 0] = g["phi_q"]
    k[0, 0, :, 0] = g["phi_k"].ravel()
    v[0, 0, :, 0] = g["v"].ravel()
    O = to_host(_run(lib, q, k, v, io, phi="identity"))
    assert abs(O[0, 0, 1, 0] - g["normalised_readout"]) < 1e-6
    assert abs(O[0, 0, 0, 0] - 2.0) < 1e-6


# ---------------------------------------------------------------- tiny workload (fp32)

@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("span_tokens", [None, 64])
def test_tiny_fp32(lib, span, chunk, span_tokens):
    span(span_tokens if span_tokens is None or span_tokens % chunk == 0 else None)
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, std=w.std, io=w.io)
    ref, S_ref, z_ref = ora.recurrent_attention(q, k, v)
    dense = ora.explicit_attention(q, k, v)
    assert np.max(np.abs(ref - dense)) < 1e-10
    O, S, z = _run(lib, q, k, v, "f32", chunk=chunk, return_state=True)
    check_close(to_host(O), ref, "f32", "O")
    np.testing.assert_allclose(to_host(S), S_ref, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(to_host(z), z_ref, rtol=1e-5, atol=1e-4)


def test_tiny_fp32_noncausal(lib, span):
    span(64)
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, std=w.std, io=w.io)
    ref, S_ref, z_ref = ora.noncausal_attention(q, k, v)
    O, S, z = _run(lib, q, k, v, "f32", causal=False, return_state=True)
    check_close(to_host(O), ref, "f32", "O")
    np.testing.assert_allclose(to_host(z), z_ref, rtol=1e-5)


# ---------------------------------------------------------------- prefill workload (full)

@pytest.fixture(scope="module")
def prefill_data():
    w = synth.WORKLOADS["prefill"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    ref, S_ref, z_ref = ora.recurrent_attention(q, k, v)
    return q, k, v, ref, S_ref, z_ref


@pytest.mark.parametrize("chunk", [64, 16, 32, 128])
def test_prefill_bf16_full(lib, span, prefill_data, chunk):
    q, k, v, ref, S_ref, z_ref = prefill_data
    O, S, z = _run(lib, q, k, v, "bf16", chunk=chunk, return_state=True)
    got = to_host(O)
    check_close(got, ref, "bf16", f"O chunk={chunk}")
    assert rel_rms_error(got, ref) < 5e-3
    check_close(to_host(S), S_ref, "bf16", "S_N")
    check_close(to_host(z), z_ref, "bf16", "z_N")


def test_prefill_bf16_split_spans(lib, span, prefill_data):
    """The span length changes only the summation order."""
    q, k, v, ref, _, _ = prefill_data
    for tokens in (64, 512, 4096):
        span(tokens)
        check_close(to_host(_run(lib, q, k, v, "bf16")), ref, "bf16", f"span={tokens}")


# ---------------------------------------------------------------- long workload (sampled)

def _sample_rows(N, chunk, rng, extra=6):
    rows = {0, 1, chunk - 1, chunk, N - 1, N // 2, 1023, 1024}
    rows.update(rng.integers(0, N, size=extra).tolist())
    return sorted(r for r in rows if 0 <= r < N)


@pytest.fixture(scope="module")
def long_data():
    w = synth.WORKLOADS["long"]
    return synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)


@pytest.mark.parametrize("causal", [True, False])
def test_long_bf16_sampled(lib, span, long_data, causal):
    q, k, v = long_data
    w = synth.WORKLOADS["long"]
    O, S, z = _run(lib, q, k, v, "bf16", causal=causal, return_state=True)
    O = to_host(O)
    rng = np.random.default_rng(7)
    for h in range(w.H):
        rows = _sample_rows(w.N, w.chunk, rng)
        fn = ora.causal_rows if causal else ora.noncausal_rows
        ref = fn(q[0, h], k[0, h], v[0, h], rows)
        check_close(O[0, h, rows], ref, "bf16", f"head {h}")
    # final state = full sums, for every head
    fk = ora.phi_elu1(k[0])
    S_ref = np.swapaxes(fk, -1, -2) @ v[0].astype(np.float64)
    z_ref = fk.sum(axis=-2)
    check_close(to_host(S)[0], S_ref, "bf16", "S_N")
    check_close(to_host(z)[0], z_ref, "bf16", "z_N")
    if not causal:
        # every row uses the same sums: the last causal row equals the last row
        last = ora.causal_rows(q[0, 0], k[0, 0], v[0, 0], [w.N - 1])
        check_close(O[0, 0, -1:], last, "bf16", "last row")


# ---------------------------------------------------------------- wide heads (sampled)

def test_wide_bf16_sampled(lib, span):
    w = synth.WORKLOADS["wide"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    O = to_host(_run(lib, q, k, v, "bf16"))
    rng = np.random.default_rng(11)
    for b in range(w.B):
        for h in range(w.H):
            rows = sorted({0, 63, 64, 2047, 2048, w.N - 1, int(rng.integers(0, w.N))})
            ref = ora.causal_rows(q[b, h], k[b, h], v[b, h], rows)
            check_close(O[b, h, rows], ref, "bf16", f"b{b} h{h}")


# ---------------------------------------------------------------- invariants and edges

def test_no_future_leakage_bitwise(lib, span):
    span(256)
    q, k, v = synth.draw_qkv(1, 4, 1000, 64, 64, io="bf16")
    base = to_host(_run(lib, q, k, v, "bf16"))
    for t0 in (512, 300, 77):      # span-aligned, mid-span, mid-chunk
        k2, v2 = k.copy(), v.copy()
        k2[..., t0:, :] = synth.round_to_io(k2[..., t0:, :] + 3.0, "bf16")
        v2[..., t0:, :] = synth.round_to_io(v2[..., t0:, :] - 5.0, "bf16")
        out = to_host(_run(lib, q, k2, v2, "bf16"))
        np.testing.assert_array_equal(out[..., :t0, :], base[..., :t0, :])
        assert np.max(np.abs(out[..., t0:, :] - base[..., t0:, :])) > 1e-3


def test_nonfinite_future_key_is_masked(lib, span):
    """A NaN key at token j reaches no row before j: the causal mask selects
    instead of multiplying."""
    span(256)
    q, k, v = synth.draw_qkv(1, 2, 600, 64, 64, io="bf16")
    base = to_host(_run(lib, q, k, v, "bf16"))
    for j in (300, 77, 64):
        k2 = k.copy()
        k2[0, 1, j, 3] = np.nan
        out = to_host(_run(lib, q, k2, v, "bf16"))
        np.testing.assert_array_equal(out[0, 1, :j], base[0, 1, :j])
        np.testing.assert_array_equal(out[0, 0], base[0, 0])           # other head untouched
        assert np.all(np.isnan(out[0, 1, j:]))


def test_deterministic(lib, span):
    q, k, v = synth.draw_qkv(2, 3, 3000, 64, 64, io="bf16")
    a = to_host(_run(lib, q, k, v, "bf16"))
    b = to_host(_run(lib, q, k, v, "bf16"))
    np.testing.assert_array_equal(a, b)


def test_constant_values_give_constant_output(lib, span):
    span(128)
    q, k, _ = synth.draw_qkv(1, 2, 700, 64, 64, io="bf16")
    v = np.broadcast_to(synth.round_to_io(np.linspace(-2, 2, 64, dtype=np.float32), "bf16"),
                        (1, 2, 700, 64)).copy()
    check_close(to_host(_run(lib, q, k, v, "bf16")), v, "bf16", "constant V")


@pytest.mark.parametrize("N", [1, 17, 100, 4097])
@pytest.mark.parametrize("chunk", [16, 64])
def test_tail_lengths(lib, span, N, chunk):
    span(128)
    q, k, v = synth.draw_qkv(1, 3, N, 64, 64, io="bf16")
    ref, S_ref, z_ref = ora.recurrent_attention(q, k, v)
    O, S, z = _run(lib, q, k, v, "bf16", chunk=chunk, return_state=True)
    check_close(to_host(O), ref, "bf16", f"N={N}")
    check_close(to_host(S), S_ref, "bf16", "S")
    check_close(to_host(z), z_ref, "bf16", "z")


def test_empty_sequence_returns_initial_state(lib):
    import torch
    S0 = np.random.default_rng(1).random((1, 2, 64, 64)).astype(np.float32)
    z0 = np.random.default_rng(2).random((1, 2, 64)).astype(np.float32) + 1
    e = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    O, S, z = lib.forward(e, e, e, S0=f32_dev(S0), z0=f32_dev(z0), return_state=True)
    torch.cuda.synchronize()
    assert O.shape == (1, 2, 0, 64)
    np.testing.assert_array_equal(to_host(S), S0)
    np.testing.assert_array_equal(to_host(z), z0)


@pytest.mark.parametrize("causal", [True, False])
def test_split_prefill_equals_one_shot(lib, span, causal):
    span(256)
    q, k, v = synth.draw_qkv(2, 2, 1500, 64, 64, io="bf16")
    n1 = 700
    full = to_host(_run(lib, q, k, v, "bf16", causal=causal)) if causal else None
    a, S1, z1 = _run(lib, q[..., :n1, :], k[..., :n1, :], v[..., :n1, :], "bf16", return_state=True)
    Q2, K2, V2 = (to_dev(x[..., n1:, :], "bf16") for x in (q, k, v))
    b = lib.forward(Q2, K2, V2, causal=causal, S0=S1, z0=z1)
    if causal:
        ref, _, _ = ora.recurrent_attention(q, k, v)
        check_close(np.concatenate([to_host(a), to_host(b)], axis=-2), ref, "bf16", "split")
        check_close(full, ref, "bf16", "one shot")
    else:
        # queries after the split see every key: earlier ones through the state
        ref, _, _ = ora.noncausal_attention(q[..., n1:, :], k, v)
        check_close(to_host(b), ref, "bf16", "non-causal with state")


def test_single_pass_is_used_and_never_times_out(lib, path):
    """With the single pass selected, the long causal shape runs on it, and
    none of its bounded waits for earlier spans expires (the kernel counts
    expiries in word 1 of its workspace)."""
    import torch
    w = synth.WORKLOADS["long"]
    n_span, single = lib.forward_config(w.B, w.H, w.N, w.d, w.dv)
    assert single == (path == "single_pass")
    if not single:
        return
    q, k, v = synth.draw_qkv(w.B, 4, 8192, w.d, w.dv, io=w.io)
    ws = torch.empty(lib.workspace_bytes(w.B, 4, 8192, w.d, w.dv), dtype=torch.uint8, device="cuda")
    Q, K, V = (to_dev(x, "bf16") for x in (q, k, v))
    O = lib.forward(Q, K, V, workspace=ws)
    torch.cuda.synchronize()
    hdr = ws[:8].cpu().numpy().view(np.uint32)
    assert hdr[0] == 4 * 8192 // 256          # every workgroup took one ticket
    assert hdr[1] == 0                        # no expired wait
    rows = [0, 255, 256, 4095, 8191]
    for h in range(4):
        check_close(to_host(O)[0, h, rows], ora.causal_rows(q[0, h], k[0, h], v[0, h], rows), "bf16", f"h{h}")
