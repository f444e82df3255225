"""Helpers shared by the GPU parity tests: host<->device transfer of the
seeded inputs, and the parity gates of tests/gates.py (the elementwise
tolerance and the per-row relative gate).  The oracle runs in fp64 on
exactly the values the GPU sees (inputs already rounded to the I/O type).
"""

from __future__ import annotations

import numpy as np

from kernelized_linear_attention_elu_amd import hostio, synth

from tests.gates import (TOL_BF16_ABS, TOL_BF16_REL, TOL_F32_ABS, check_close, check_rows,  # noqa: F401
                         rel_rms_error, row_errors)


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
