"""The timed entry points (la_forward_timed, la_backward_timed) record HIP
events around the library's kernels and change nothing else: their outputs
equal the untimed calls' bit for bit, with every event slot filled or only
some, and the recorded intervals are valid (non-negative, and together no
longer than the host's wall time around the call)."""

import time

import numpy as np
import pytest

from kernelized_linear_attention_elu_amd import synth
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


def _events(lib, n):
    return [lib.event_create() for _ in range(n)]


def _destroy(lib, evs):
    for e in evs:
        if e is not None:
            lib.event_destroy(e)


@pytest.mark.parametrize("kw", [{}, {"causal": False}, {"gamma": True}, {"log_gate": True}, {"log_gate_ch": True}])
def test_forward_timed_equals_untimed(lib, kw):
    import torch
    B, H, N, d = 1, 3, 777, 64
    q, k, v = synth.draw_qkv(B, H, N, d, d, seed=31)
    Q, K, V = (to_dev(x, "bf16") for x in (q, k, v))
    args = dict(kw)
    if args.pop("gamma", False):
        args["gamma"] = torch.tensor([0.99, 0.9, 0.5], dtype=torch.float32, device="cuda")
    if args.pop("log_gate", False):
        args["log_gate"] = to_dev(synth.draw_log_gates(B, H, N, seed=32), "f32")
    if args.pop("log_gate_ch", False):
        args["log_gate_ch"] = to_dev(synth.draw_log_gates_ch(B, H, N, d, seed=33), "f32")
    ref = to_host(lib.forward(Q, K, V, **args))
    nk = lib.LA_FORWARD_KERNELS
    evs = _events(lib, 2 * nk)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    got = lib.forward(Q, K, V, events=evs, **args)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    np.testing.assert_array_equal(to_host(got), ref)
    ms = [lib.event_elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(nk)]
    assert all(m >= 0.0 for m in ms), ms
    assert 0.0 < sum(ms) <= wall_ms, (ms, wall_ms)
    # only the last kernel's pair, as the bench records it inside its timed steps
    part = [None] * (2 * nk - 2) + evs[2 * nk - 2:]
    got2 = lib.forward(Q, K, V, events=part, **args)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(got2), ref)
    assert lib.event_elapsed_ms(evs[2 * nk - 2], evs[2 * nk - 1]) > 0.0
    _destroy(lib, evs)


def test_backward_timed_equals_untimed(lib):
    import torch
    q, k, v = synth.draw_qkv(1, 2, 300, 64, 64, seed=34)
    dO = synth.round_to_io(np.random.default_rng(35).standard_normal((1, 2, 300, 64), dtype=np.float32), "bf16")
    Q, K, V, G = (to_dev(x, "bf16") for x in (q, k, v, dO))
    O = lib.forward(Q, K, V)
    ref = [to_host(t) for t in lib.backward(Q, K, V, O, G)]
    nk = lib.LA_BACKWARD_KERNELS
    evs = _events(lib, 2 * nk)
    got = lib.backward(Q, K, V, O, G, events=evs)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(to_host(a), b)
    ms = [lib.event_elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(nk)]
    assert all(m >= 0.0 for m in ms) and sum(ms) > 0.0, ms
    _destroy(lib, evs)
