"""GPU test of la_forward_noalloc (the entry point that allocates nothing):
through the C ABI it gives the same outputs and final state as la_forward
with a workspace, bit for bit, on two calls in a row (the second with a
smaller input, so that it runs over what the first left in the shared
scratch), and both agree with the fp64 oracle under the parity gates."""

import numpy as np
import pytest

from oracle import linear_attention as ora
from kernelized_linear_attention_elu_amd import synth
from tests.gpu_util import check_close, f32_dev, to_dev, to_host

pytestmark = pytest.mark.gpu


def _pair(lib, q, k, v, **kw):
    import torch
    Q, K, V = (to_dev(x, "bf16") for x in (q, k, v))
    print(f"la_forward_noalloc shape {q.shape} {kw}", flush=True)
    a = lib.forward(Q, K, V, return_state=True, **kw)
    b = lib.forward_noalloc(Q, K, V, return_state=True, **kw)
    torch.cuda.synchronize()
    return [to_host(t) for t in a], [to_host(t) for t in b]


@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_equals_forward_twice(lib, causal):
    big = synth.draw_qkv(1, 8, 8192, 64, 64, seed=61)
    small = synth.draw_qkv(2, 3, 700, 64, 64, seed=62)
    for q, k, v in (big, small):
        a, b = _pair(lib, q, k, v, causal=causal)
        for x, y, name in zip(a, b, ("O", "S_N", "z_N")):
            np.testing.assert_array_equal(y, x, err_msg=name)
        fn = ora.recurrent_attention if causal else ora.noncausal_attention
        if q.shape[-2] <= 1000:
            ref, S_ref, z_ref = fn(q, k, v)
            check_close(b[0], ref, "bf16", "O")
            check_close(b[1], S_ref, "bf16", "S_N")
            check_close(b[2], z_ref, "bf16", "z_N")


def test_noalloc_with_initial_state(lib):
    import torch
    q, k, v = synth.draw_qkv(1, 2, 900, 64, 64, seed=63)
    n1 = 333
    Q, K, V = (to_dev(x, "bf16") for x in (q, k, v))
    _, S1, z1 = lib.forward_noalloc(Q[:, :, :n1].contiguous(), K[:, :, :n1].contiguous(),
                                    V[:, :, :n1].contiguous(), return_state=True)
    O2 = lib.forward_noalloc(Q[:, :, n1:].contiguous(), K[:, :, n1:].contiguous(), V[:, :, n1:].contiguous(),
                             S0=S1, z0=z1)
    torch.cuda.synchronize()
    ref, _, _ = ora.recurrent_attention(q, k, v)
    check_close(to_host(O2), ref[:, :, n1:], "bf16", "second part")
