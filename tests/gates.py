"""Parity gates shared by the GPU tests and their CPU self-checks (NumPy only).

Two rules apply to every compared array; both must hold.

1. Elementwise (the stated tolerance): fp32 I/O, |gpu - oracle| <= 1e-4;
   bf16 I/O with fp32 state, |gpu - oracle| <= 2e-2 + 2e-2 |oracle|.

2. Per row: for every row (the last axis: one token's output vector, one
   feature row of a state), ||gpu_row - oracle_row||_2 / ||oracle_row||_2
   must stay below ROW_BF16 (bf16 I/O) or ROW_F32 (fp32 I/O).

   Why a second rule: late outputs of a long causal sequence are weighted
   means over many values and shrink like sigma / sqrt(t) (|o| about 0.005
   at t = 32768 for the long workload), below the 2e-2 absolute floor of
   rule 1, so rule 1 alone would accept an all-zero row there.  Rule 2 is
   scale-free.

   Where ROW_BF16 comes from: a bf16 output row passes through five
   roundings to bf16 on the way (phi(q), phi(k), the carried state read
   out on the matrix cores, the masked weights, the output itself).  Each
   is a relative error of at most 2^-9 per value, with an RMS of at most
   2^-9 / sqrt(3) = 1.13e-3 (uniform rounding error at the bottom of a
   binade).  In quadrature that is sqrt(5) x 1.13e-3 = 2.5e-3 relative per
   row; the gate is four times that, 1e-2.  (An fp64 emulation of exactly
   these roundings on the prefill shapes gives a per-row mean of 1.7e-3
   and a maximum of 3.7e-3.)  It rejects an all-zero or half-size output
   (relative error 1 and 0.5) and a dropped or doubled piece of the
   history, which moves a row by a sizeable fraction of itself.
   fp32 I/O keeps its operands in fp32: ROW_F32 = 1e-4, the elementwise
   figure, relative.

   Rows whose oracle norm is exactly zero must come back as exact zeros.
"""

from __future__ import annotations

import numpy as np

TOL_F32_ABS = 1e-4
TOL_BF16_ABS = 2e-2
TOL_BF16_REL = 2e-2
ROW_BF16 = 1e-2
ROW_F32 = 1e-4


def row_bound(io):
    return ROW_F32 if io == "f32" else ROW_BF16


def row_errors(got, ref):
    """||got_row - ref_row|| / ||ref_row|| over the last axis (0 where both
    rows are zero, inf where only the reference row is)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    en = np.linalg.norm(got - ref, axis=-1)
    rn = np.linalg.norm(ref, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(rn > 0, en / np.where(rn > 0, rn, 1.0), np.where(en > 0, np.inf, 0.0))
    return rel


def check_rows(got, ref, io, what="", bound=None):
    """Assert rule 2; returns the largest per-row relative error."""
    bound = row_bound(io) if bound is None else bound
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rel = row_errors(got, ref)
    worst = np.unravel_index(np.argmax(rel), rel.shape) if rel.size else ()
    assert rel.size == 0 or rel.max() <= bound, (
        f"{what}: row {worst} relative error {rel[worst]:.3e} > {bound:.1e} "
        f"(mean {rel.mean():.3e}, rows over: {int(np.sum(rel > bound))} of {rel.size})")
    return float(rel.max()) if rel.size else 0.0


def check_close(got, ref, io, what="", rows=True, row_bound_=None):
    """Assert rule 1 and (unless rows=False) rule 2.  Returns (max_abs,
    max_excess over the elementwise bound, max per-row relative error)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    if io == "f32":
        bound = np.full_like(ref, TOL_F32_ABS)
    else:
        bound = TOL_BF16_ABS + TOL_BF16_REL * np.abs(ref)
    if err.size:
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), (
            f"{what}: max |err| {err.max():.3e}, worst at {worst}: got {got[worst]!r} ref {ref[worst]!r} "
            f"bound {bound[worst]:.3e}")
    rmax = check_rows(got, ref, io, what, row_bound_) if rows else 0.0
    return (float(err.max()) if err.size else 0.0,
            float((err - bound).max()) if err.size else 0.0, rmax)


def rel_rms_error(got, ref):
    """RMS error over RMS of the reference (whole array)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.mean((got - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-300))


# ---------------------------------------------------------------- gradients
#
# Gradients cancel more than outputs do.  dphi(q_i) = sum_{j<=i} (dO_i.(v_j -
# o_i) / D_i) phi(k_j), and the kernels form it as S_i g_i + h_i z_i (plus the
# in-chunk terms): two sums that cancel the common part of the features
# (mean of ELU+1 about 1.06 against a spread of about 0.35 at sigma =
# d^-1/4), so each term's rounding comes out about three times larger
# relative to the result.  About six bf16-rounded operands enter (phi(q),
# phi(k), g = dO / D, the masked W, the bf16 state or reverse-sum tile, the
# forward output O): 3 x sqrt(6) x 1.13e-3 = 8.3e-3 relative RMS on average.
# An fp64 emulation of exactly these roundings for dQ (prefill shapes) gives
# a per-row mean of 1.1e-2.  Three gates:
#
#   * per head, the relative RMS error of the whole gradient array <= 3e-2
#     (rejects a gradient scaled by 0.9);
#   * per block of 64 rows (a chunk), the relative RMS error <= 5e-2
#     (rejects a wrong chunk, span or boundary: a dropped history or suffix
#     term moves a block by a sizeable fraction of itself).  A ragged tail of
#     fewer than 16 rows joins the block before it: a block of one or two
#     rows averages nothing, and a last row whose dot product dO.(v - o)
#     cancels (dK of a head's last token is phi(q) dO.(v - o) / D) would
#     then be held to 5e-2 of a near-zero norm, tighter than its row gate;
#   * per row, the error <= 1e-1 of the row's norm or <= 2^-4 of the
#     magnitude m of the two sums the kernels form for it
#     (tests/grad_scales.py), whichever is larger.  The second term is for
#     rows whose terms cancel almost entirely: dQ of a head's first token is
#     exactly zero (o_0 = v_0) and the next few rows keep a small fraction
#     of their terms; the kernels reach them as a difference of rounded
#     sums, and the dot products inside those sums can cancel as well (the
#     worst measured row, the second token of a long head, came within
#     0.046 m).  Where those dot products cancel almost entirely, m takes
#     1/16 of their terms' magnitude instead (tests/grad_scales.py).  For
#     typical rows m is three to five times the row's norm.
#
# A head or block whose reference is zero up to 1e-9 of m (a single token)
# is judged by its rows alone.  A head of fewer than 16 rows (one block) is
# held to the larger of its relative gate and 2^-6 of its magnitude m: all
# of its rows are early rows, which cancel (an fp64 model of the dQ pass's
# bf16 roundings over 240 random heads of 2 to 200 tokens: relative head
# error up to 0.14 at 2 tokens and 0.057 at 4, under 0.03 from 5 tokens;
# head error against m at most 2^-7.6).

GRAD_HEAD = 3e-2
GRAD_BLOCK = 5e-2
GRAD_ROW = 1e-1
GRAD_FLOOR = 2.0 ** -4
GRAD_SHORT_FLOOR = 2.0 ** -6
GRAD_BLOCK_ROWS = 64
GRAD_TAIL_ROWS = 16


def _rel_rms(err2, ref2, m2):
    """Relative RMS error from summed squares; 0 where the reference is zero
    up to 1e-9 of m (judged by the row gate instead)."""
    en, rn, mn = np.sqrt(err2), np.sqrt(ref2), np.sqrt(m2)
    judged = rn > 1e-9 * mn
    return np.where(judged, en / np.where(judged, rn, 1.0), 0.0)


def _over(err2, ref2, m2, rel, short):
    """Which heads or blocks exceed their gate: rel of the reference's norm,
    or (short heads) 2^-6 of m where that is larger; zero references are
    left to the row gate."""
    en, rn, mn = np.sqrt(err2), np.sqrt(ref2), np.sqrt(m2)
    bound = np.maximum(rel * rn, GRAD_SHORT_FLOOR * mn) if short else rel * rn
    return (rn > 1e-9 * mn) & (en > bound)


def check_grad(got, ref, scale, what=""):
    """The gradient gates above.  ``got``, ``ref``, ``scale``: [..., N, d]
    (``scale``: the magnitudes m of tests/grad_scales.py); a head is
    everything but the last two axes.  Returns (largest head RMS error,
    largest block RMS error, largest row error as a fraction of its
    bound)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    assert got.shape == ref.shape == scale.shape, (got.shape, ref.shape, scale.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if ref.size == 0:
        return 0.0, 0.0, 0.0
    e2 = np.sum((got - ref) ** 2, axis=-1)
    r2 = np.sum(ref ** 2, axis=-1)
    m2 = np.sum(scale ** 2, axis=-1)
    n = e2.shape[-1]
    short = n < GRAD_TAIL_ROWS
    head = _rel_rms(e2.sum(-1), r2.sum(-1), m2.sum(-1))
    assert not _over(e2.sum(-1), r2.sum(-1), m2.sum(-1), GRAD_HEAD, short).any(), (
        f"{what}: head relative RMS error {head.max():.3e} > {GRAD_HEAD:.0e} (per head: {np.round(head.ravel(), 4)})")
    nb = (n + GRAD_BLOCK_ROWS - 1) // GRAD_BLOCK_ROWS
    # a ragged tail of fewer than GRAD_TAIL_ROWS rows joins the block before it
    if nb > 1 and n - (nb - 1) * GRAD_BLOCK_ROWS < GRAD_TAIL_ROWS:
        nb -= 1
    bid = np.minimum(np.arange(n) // GRAD_BLOCK_ROWS, nb - 1)
    blk = lambda x: np.stack([x[..., bid == b].sum(-1) for b in range(nb)], axis=-1)
    block = _rel_rms(blk(e2), blk(r2), blk(m2))
    wb = np.unravel_index(np.argmax(block), block.shape)
    assert not _over(blk(e2), blk(r2), blk(m2), GRAD_BLOCK, short).any(), (
        f"{what}: block {wb} (rows {GRAD_BLOCK_ROWS * wb[-1]}..) relative RMS error {block[wb]:.3e} > "
        f"{GRAD_BLOCK:.0e} (blocks over: {int(np.sum(block > GRAD_BLOCK))} of {block.size})")
    er, rr, sr = np.sqrt(e2), np.sqrt(r2), np.sqrt(m2)
    bound = np.maximum(GRAD_ROW * rr, GRAD_FLOOR * sr)
    with np.errstate(divide="ignore", invalid="ignore"):
        frac = np.where(bound > 0, er / np.where(bound > 0, bound, 1.0), np.where(er > 0, np.inf, 0.0))
    worst = np.unravel_index(np.argmax(frac), frac.shape)
    assert frac.max() <= 1.0, (
        f"{what}: row {worst} error {er[worst]:.3e} over its bound {bound[worst]:.3e} "
        f"(|ref row| {rr[worst]:.3e}, m {sr[worst]:.3e}; rows over: {int(np.sum(frac > 1))} of {frac.size})")
    return float(head.max()), float(block.max()), float(frac.max())
