"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and rounds them to the I/O format; it
holds none of the linear-attention arithmetic, so that the HIP path and the
CPU oracle can consume identical inputs while sharing no computation.

Recipe:

* ``numpy.random.default_rng(seed)``; float32 standard normals drawn in the
  order Q, K, V, each over its full [B, H, N, d] (or [B, H, N, d_v]) shape;
* scaled by ``std`` (default d ** -0.25, i.e. variance 1/sqrt(d));
* rounded to bfloat16 with round-to-nearest-even when the I/O type is bf16.
  The returned float32 arrays hold exactly the values the GPU sees;
* FAVOR+ projections: r // d independent blocks, each an orthogonal matrix
  from the QR factorisation of a d x d standard-normal draw (signs fixed by
  the diagonal of R) whose rows are rescaled by the norms of independent
  d-dimensional standard-normal draws, so that every row is marginally
  N(0, I_d) while rows inside a block are orthogonal.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DATA_SEED = 0
OMEGA_SEED = 1
DECODE_STATE_SEED = 2


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.
    Inputs are finite Gaussians, so NaN handling is not needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_values(bits):
    """bfloat16 bit patterns -> the float32 values they encode (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_to_io(x, io):
    """Round float32 values to what the I/O dtype can hold ('bf16' or 'f32')."""
    if io == "bf16":
        return bf16_values(bf16_bits(x))
    if io == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown io dtype {io!r}")


def default_std(d):
    """Per-element standard deviation d**-0.25 (variance 1/sqrt(d))."""
    return float(d) ** -0.25


def draw_qkv(B, H, N, d, dv, seed=DATA_SEED, std=None, io="bf16"):
    """Q, K [B,H,N,d] and V [B,H,N,dv] as float32 arrays already rounded to
    the I/O dtype.  ``std=None`` means d**-0.25; pass 1.0 for N(0, 1)."""
    rng = np.random.default_rng(seed)
    s = default_std(d) if std is None else float(std)
    out = []
    for shape in ((B, H, N, d), (B, H, N, d), (B, H, N, dv)):
        x = rng.standard_normal(shape, dtype=np.float32)
        if s != 1.0:
            x *= np.float32(s)
        out.append(round_to_io(x, io))
    return tuple(out)


def draw_qkv_device(B, H, N, d, dv, seed=DATA_SEED, std=None, device="cuda"):
    """Q, K [B,H,N,d] and V [B,H,N,dv] as bf16 device tensors, drawn from
    torch's seeded generator on the device: N(0, std^2) in float32
    (std=None means d**-0.25), then rounded to bf16 (nearest even).  For
    sizes whose host draw would take minutes; a comparison reads the values
    back from the device."""
    import torch
    g = torch.Generator(device=device).manual_seed(int(seed))
    s = default_std(d) if std is None else float(std)
    out = []
    for shape in ((B, H, N, d), (B, H, N, d), (B, H, N, dv)):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        x.mul_(s)
        out.append(x.to(torch.bfloat16))
        del x
    return tuple(out)


def draw_omega(r, d, seed=OMEGA_SEED):
    """FAVOR+ projection rows, float32 [r, d]: block-orthogonal Gaussian rows."""
    rng = np.random.default_rng(seed)
    blocks = []
    remaining = r
    while remaining > 0:
        g = rng.standard_normal((d, d))
        qm, rm = np.linalg.qr(g)
        qm = qm * np.sign(np.diag(rm))[None, :]          # Haar-distributed
        norms = np.linalg.norm(rng.standard_normal((d, d)), axis=1)
        block = qm.T * norms[:, None]                   # orthogonal rows
        take = min(d, remaining)
        blocks.append(block[:take])
        remaining -= take
    return np.ascontiguousarray(np.concatenate(blocks, axis=0), dtype=np.float32)


def draw_decode_history(n_seq, H, T, d, dv, seed=DECODE_STATE_SEED, io="bf16"):
    """History tokens (K [n_seq,H,T,d], V [n_seq,H,T,dv]) from which a decode
    state is built by whichever side consumes them."""
    rng = np.random.default_rng(seed)
    s = default_std(d)
    k = rng.standard_normal((n_seq, H, T, d), dtype=np.float32) * np.float32(s)
    v = rng.standard_normal((n_seq, H, T, dv), dtype=np.float32) * np.float32(s)
    return round_to_io(k, io), round_to_io(v, io)


def draw_decode_token(n_seq, H, d, dv, seed=DATA_SEED, io="bf16"):
    """One new token per (sequence, head): q, k [n_seq,H,d], v [n_seq,H,dv]."""
    rng = np.random.default_rng(seed)
    s = default_std(d)
    q = rng.standard_normal((n_seq, H, d), dtype=np.float32) * np.float32(s)
    k = rng.standard_normal((n_seq, H, d), dtype=np.float32) * np.float32(s)
    v = rng.standard_normal((n_seq, H, dv), dtype=np.float32) * np.float32(s)
    return round_to_io(q, io), round_to_io(k, io), round_to_io(v, io)


def decay_gammas(H):
    """Per-head decays for the decayed (RetNet-form) workloads, float32 [H]:
    gamma_h = 1 - 2^-(5 + 7 h / (H - 1)), one time scale per head from
    1 - 1/32 to 1 - 1/4096 (the pages give no values beyond gamma = 0.99; a
    spread of fixed per-head rates is what they describe).  Deterministic."""
    h = np.arange(H, dtype=np.float64)
    e = 5.0 + 7.0 * h / max(H - 1, 1)
    return (1.0 - 2.0 ** (-e)).astype(np.float32)


GATE_SEED = 20251203


def draw_log_gates(B, H, N, seed=GATE_SEED, resets=0):
    """Per-token natural-log gates for the gated (SSD-form) workloads, float32
    [B, H, N]: log a_t = -dt_t * A_h with dt_t log-uniform in [1e-3, 1e-1]
    and A_h = 1 + 15 h / (H - 1), the step and rate ranges Mamba-2 initialises
    its selective step and scalar decay with (the pages give no values; they
    describe a large step forgetting the history and a small one keeping it).
    ``resets`` tokens per head, at seeded positions, get log a = -inf (a zero
    gate).  Deterministic."""
    rng = np.random.default_rng(seed)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(B, H, N)))
    A = 1.0 + 15.0 * np.arange(H, dtype=np.float64) / max(H - 1, 1)
    out = (-dt * A[None, :, None]).astype(np.float32)
    for b in range(B):
        for h in range(H):
            if resets and N:
                out[b, h, rng.choice(N, size=min(resets, N), replace=False)] = -np.inf
    return out


def draw_log_gates_ch(B, H, N, r, seed=GATE_SEED + 1, resets=0):
    """Per-token, per-key-channel natural-log gates for the GLA-form
    workloads, float32 [B, H, N, r]: log a = log(sigmoid(x)) / 16 with
    x ~ N(0, 2^2), GLA's sigmoid(x)^(1/16) gate form (the pages give no
    values).  ``resets`` (token, channel) entries per head, at seeded
    positions, get log a = -inf (a zero gate).  Deterministic."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, N, r), dtype=np.float32) * np.float32(2.0)
    out = (-np.logaddexp(np.float32(0.0), -x) / np.float32(16.0)).astype(np.float32)
    for b in range(B):
        for h in range(H):
            if resets and N:
                t = rng.integers(0, N, size=resets)
                f = rng.integers(0, r, size=resets)
                out[b, h, t, f] = -np.inf
    return out


@dataclass(frozen=True)
class Workload:
    """Shapes of one named workload (no arithmetic)."""
    name: str
    B: int
    H: int
    N: int
    d: int
    dv: int
    io: str
    phi: str
    r: int
    chunk: int
    std: float | None  # None: d**-0.25
    causal: tuple


WORKLOADS = {
    # tiny CPU-checkable case, N(0,1) inputs, fp32 I/O
    "tiny": Workload("tiny", 1, 1, 256, 64, 64, "f32", "elu1", 64, 64, 1.0, (True,)),
    # prefill B4 H16 N4096 d64 bf16
    "prefill": Workload("prefill", 4, 16, 4096, 64, 64, "bf16", "elu1", 64, 64, None, (True,)),
    # long prefill B1 H32 N32768 d64 bf16, causal and non-causal
    "long": Workload("long", 1, 32, 32768, 64, 64, "bf16", "elu1", 64, 64, None, (True, False)),
    # wide heads B2 H16 N65536 d128 bf16
    "wide": Workload("wide", 2, 16, 65536, 128, 128, "bf16", "elu1", 128, 64, None, (True,)),
    # Performer FAVOR+ r=256, B2 H16 N16384 d64 bf16
    "favor": Workload("favor", 2, 16, 16384, 64, 64, "bf16", "favor", 256, 64, None, (True,)),
}

# decode step after the wide prefill: 256 sequences x 32 heads, d = dv = 128,
# fp32 state built from a 256-token history
DECODE_WORKLOAD = dict(n_seq=256, H=32, d=128, dv=128, history=256, io="bf16")
