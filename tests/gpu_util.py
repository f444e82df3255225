"""Helpers shared by the GPU parity tests: host<->device transfer of the
seeded inputs and the tolerance rule.

Tolerances: fp32 I/O, max |gpu - oracle| <= 1e-4; bf16 I/O with fp32 state,
|gpu - oracle| <= 2e-2 + 2e-2 |oracle| elementwise.  The oracle runs in fp64
on exactly the values the GPU sees (inputs already rounded to the I/O type).
"""

from __future__ import annotations

import numpy as np

from kernelized_linear_attention_elu_amd import hostio, synth

TOL_F32_ABS = 1e-4
TOL_BF16_ABS = 2e-2
TOL_BF16_REL = 2e-2


def to_dev(x, io, device="cuda"):
    """float32 numpy array (already representable in ``io``) -> device tensor
    (copied through pinned staging memory)."""
    if io == "bf16":
        return hostio.upload_bf16_bits(synth.bf16_bits(x), device)
    return hostio.upload_f32(x, device)


def f32_dev(x, device="cuda"):
    return hostio.upload_f32(x, device)


def to_host(t):
    """Device tensor -> float64 numpy array (exact for bf16 and fp32)."""
    return hostio.download_f64(t.detach())


def check_close(got, ref, io, what=""):
    """Assert the tolerance rule; returns (max_abs, max_excess) for reporting."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    if io == "f32":
        bound = np.full_like(ref, TOL_F32_ABS)
    else:
        bound = TOL_BF16_ABS + TOL_BF16_REL * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (
        f"{what}: max |err| {err.max():.3e}, worst at {worst}: got {got[worst]!r} ref {ref[worst]!r} "
        f"bound {bound[worst]:.3e}")
    return float(err.max()), float((err - bound).max())


def rel_rms_error(got, ref):
    """Diagnostic: RMS error over RMS of the reference (per whole array)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.mean((got - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-300))
