"""GPU parity of la_forward against the fp64 oracle.

Every case feeds the same seeded inputs (already rounded to the I/O type) to
the HIP library and to the oracle and compares every element, under both
parity gates of tests/gates.py (the elementwise tolerance and the per-row
relative gate).  At the full workload sizes the oracle's token recurrence
runs on every (batch, head) in a process pool (oracle/heads.py).
"""

import numpy as np
import pytest

from oracle import heads
from oracle import linear_attention as ora
from kernelized_linear_attention_elu_amd import synth
from tests.golden import load
from tests.gpu_util import check_close, f32_dev, rel_rms_error, to_dev, to_host

pytestmark = pytest.mark.gpu


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


# ---------------------------------------------------------------- d = 128 at every chunk

@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("tokens", [None, "2c"])
def test_d128_every_chunk(lib, span, chunk, causal, tokens):
    """d = 128 (eight waves per workgroup: two waves per row block at chunk
    64, four at 32, eight at 16) at every chunk it supports, with one span or
    several per head and a ragged last chunk: every element, S_N and z_N."""
    if tokens == "2c":
        span(2 * chunk)
    q, k, v = synth.draw_qkv(2, 3, 333, 128, 128, seed=1280 + chunk)
    ref, S_ref, z_ref = ora.recurrent_attention(q, k, v) if causal else ora.noncausal_attention(q, k, v)
    O, S, z = _run(lib, q, k, v, "bf16", chunk=chunk, causal=causal, return_state=True)
    check_close(to_host(O), ref, "bf16", f"O d128 chunk={chunk} causal={causal}")
    check_close(to_host(S), S_ref, "bf16", "S_N")
    check_close(to_host(z), z_ref, "bf16", "z_N")


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("N", [1, 17])
def test_d128_short(lib, span, chunk, N):
    """d = 128 with fewer tokens than one chunk (the staging masks and the
    loads past the end), causal."""
    q, k, v = synth.draw_qkv(1, 2, N, 128, 128, seed=1290 + N + chunk)
    ref, S_ref, z_ref = ora.recurrent_attention(q, k, v)
    O, S, z = _run(lib, q, k, v, "bf16", chunk=chunk, return_state=True)
    check_close(to_host(O), ref, "bf16", f"O d128 N={N} chunk={chunk}")
    check_close(to_host(S), S_ref, "bf16", "S_N")
    check_close(to_host(z), z_ref, "bf16", "z_N")


# ---------------------------------------------------------------- long and wide workloads (full)

def _recurrent_head(q, k, v, phi="elu1", omega=None):
    return ora.recurrent_attention(q, k, v, phi=phi, omega=omega)


@pytest.fixture(scope="module")
def long_case():
    """The long workload (B1 H32 N32768 d64 bf16) and its fp64 references:
    the causal recurrence of every head, and the non-causal sums."""
    w = synth.WORKLOADS["long"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    causal = heads.map_heads(_recurrent_head, q, k, v)
    noncausal = ora.noncausal_attention(q, k, v)
    return q, k, v, {True: causal, False: noncausal}


@pytest.mark.parametrize("causal", [True, False])
def test_long_bf16_full(lib, span, long_case, causal):
    """Every output of every head, and the final state, in the bench's launch
    configuration.  Late causal rows (and every non-causal row) are far
    below the elementwise floor; the per-row gate is what holds them."""
    q, k, v, refs = long_case
    ref, S_ref, z_ref = refs[causal]
    O, S, z = _run(lib, q, k, v, "bf16", causal=causal, return_state=True)
    _, _, worst = check_close(to_host(O), ref, "bf16", "O")
    print(f"long causal={causal}: worst row relative error {worst:.3e}", flush=True)
    check_close(to_host(S), S_ref, "bf16", "S_N")
    check_close(to_host(z), z_ref, "bf16", "z_N")
    if not causal:
        # every row uses the same sums: the last causal row equals the last row
        check_close(to_host(O)[:, :, -1:], refs[True][0][:, :, -1:], "bf16", "last row")


@pytest.mark.parametrize("causal", [True, False])
def test_wide_bf16_full(lib, span, causal):
    """The wide workload (B2 H16 N65536 d128 bf16): every output of every
    (batch, head) and the final state (non-causal: the full sums)."""
    w = synth.WORKLOADS["wide"]
    q, k, v = synth.draw_qkv(w.B, w.H, w.N, w.d, w.dv, io=w.io)
    O, S, z = _run(lib, q, k, v, "bf16", causal=causal, return_state=True)
    O, S, z = to_host(O), to_host(S), to_host(z)
    if causal:
        ref, S_ref, z_ref = heads.map_heads(_recurrent_head, q, k, v)
    else:
        ref, S_ref, z_ref = ora.noncausal_attention(q, k, v)
    del q, k, v
    _, _, worst = check_close(O, ref, "bf16", "O")
    print(f"wide causal={causal}: worst row relative error {worst:.3e}", flush=True)
    check_close(S, S_ref, "bf16", "S_N")
    check_close(z, z_ref, "bf16", "z_N")


# ---------------------------------------------------------------- the longest sequence of one head

@pytest.mark.parametrize("d", [64, 128])
def test_longest_head(lib, d):
    """The longest sequence one head takes in bf16: a head's Q/K/V/O are
    addressed through 32-bit buffer offsets, so N * 2d bytes must stay below
    2^31 (N <= 2^24 - 1 at d = 64, 2^23 - 1 at d = 128); here
    N = 2^31 / (2d) - 37, with a ragged last chunk.  The inputs are drawn on the device (a host draw of 3 x 2^30 values takes
    minutes) and read back for the oracle.  Compared: sampled rows (both
    ends, chunk and span edges, the rows whose byte offsets pass 2^30 and
    come within a chunk of 2^31) and the final state.  The oracle's state
    before a sampled row is the sum of its full-sequence sums over the
    whole 2^20-token pieces before the row's piece; from there causal_rows
    takes the row's piece with that state as S0, z0 (the split-prefill
    handoff, pinned on the CPU)."""
    import torch
    from kernelized_linear_attention_elu_amd import hostio
    N = (1 << 31) // (2 * d) - 37
    Q, K, V = synth.draw_qkv_device(1, 1, N, d, d)
    O, S, z = lib.forward(Q, K, V, return_state=True)
    torch.cuda.synchronize()
    n_span = lib.forward_config(1, 1, N, d, d)[0]
    n_ch = (N + 63) // 64
    edges = [s * n_ch // n_span * 64 for s in (1, n_span // 2, n_span - 1)]
    half = (1 << 30) // (2 * d)  # the first row at byte offset 2^30
    rows = sorted({0, 1, 63, 64, half - 1, half, N - 65, ((N - 1) // 64) * 64, N - 2, N - 1}
                  | {e - 1 for e in edges} | set(edges))
    idx = torch.tensor(rows, device=Q.device)
    got = to_host(O[0, 0].index_select(0, idx))
    qrows = to_host(Q[0, 0].index_select(0, idx))
    S, z = to_host(S)[0, 0], to_host(z)[0, 0]
    del O
    kb, vb = (hostio.download_bytes(t).view(np.uint16) for t in (K, V))
    del Q, K, V
    torch.cuda.empty_cache()

    def vals(bits, a, b):
        return (bits[a * d:b * d].astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(b - a, d)

    P = 1 << 20
    pre_S, pre_z = [np.zeros((d, d))], [np.zeros(d)]
    for a in range(0, N, P):
        b = min(a + P, N)
        kk = vals(kb, a, b)
        _, Sp, zp = ora.noncausal_attention(kk[:1], kk, vals(vb, a, b))
        pre_S.append(pre_S[-1] + Sp)
        pre_z.append(pre_z[-1] + zp)
    ref = np.empty((len(rows), d))
    for i, t in enumerate(rows):
        a = t // P * P
        kk, vv = vals(kb, a, t + 1), vals(vb, a, t + 1)
        qq = np.zeros_like(kk)
        qq[-1] = qrows[i]
        ref[i] = ora.causal_rows(qq, kk, vv, [t - a], S0=pre_S[a // P], z0=pre_z[a // P])[0]
    _, _, worst = check_close(got, ref, "bf16", f"O rows {rows}")
    print(f"longest head d={d} N={N}: {len(rows)} rows, worst row relative error {worst:.3e}", flush=True)
    check_close(S, pre_S[-1], "bf16", "S_N")
    check_close(z, pre_z[-1], "bf16", "z_N")


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
