"""fp64 CPU oracle for causal linear attention with a data-dependent scalar
gate per token (the scalar-decay form of Mamba-2's SSD).

TEST INFRASTRUCTURE ONLY, like ``oracle.linear_attention``: nothing in the
product path may import, call or link this module (only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``).
It shares no code with the HIP library.

Source: "Linear attention and SSM" (t6page.pages.dev), section "How does
Mamba-2's SSD unify SSM and attention": with the state transition
restricted to a scalar times the identity, A_t = a_t I, the whole output is
Y = M X with M = (C B^T) o L and L_ij = a_{i:j}^x, the product of the gates
between j and i (i >= j), i.e. structured masked attention
Y = ((Q K^T) o L) V with Q <-> C, K <-> B; causal linear attention is the
special case where L is the plain causal mask (every a = 1).  L is
1-semiseparable: its lower-triangular submatrices have rank at most 1.

Readings taken:

* the product a_{i:j}^x runs over the gates after j up to and including i,
  a_{j+1} ... a_i (so L_ii = 1): this is the recurrence
  S_t = a_t S_{t-1} + phi(k_t) v_t^T, o_t = phi(q_t)^T S_t written out;
* phi of the hot path is applied to q and k (the identity gives the page's
  Q K^T form);
* optional normalisation as for the fixed decay (oracle.decay):
  z_t = a_t z_{t-1} + phi(k_t), o_t = phi(q_t)^T S_t / phi(q_t)^T z_t;
* one gate per (batch, head, token), a in (0, 1];
* an initial state S0, z0 enters o_t (0-based t) with a_0 a_1 ... a_t.

Every function upcasts to float64.  Pins: tests/test_oracle_gated_pins.py.
"""

from __future__ import annotations

import numpy as np

from oracle.linear_attention import feature_map

__all__ = ["gate_mask", "explicit_gated", "recurrent_gated", "decode_step_gated", "causal_rows_gated"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def gate_mask(a):
    """L[..., i, j] = a_{j+1} a_{j+2} ... a_i for j <= i (1 on the diagonal),
    0 above it, formed by products (no logarithms).  a: [..., N]."""
    a = _f64(a)
    n = a.shape[-1]
    L = np.zeros(a.shape[:-1] + (n, n))
    for i in range(n):
        run = np.ones(a.shape[:-1])
        L[..., i, i] = 1.0
        for j in range(i - 1, -1, -1):
            run = run * a[..., j + 1]
            L[..., i, j] = run
    return L


def explicit_gated(q, k, v, a, phi="elu1", omega=None, normalize=True, S0=None, z0=None):
    """Structured masked attention: A = (phi(Q) phi(K)^T) o L, O = A V
    (divided by rowsum(A) when normalising), plus the gated initial state
    (a_0 ... a_i) phi(q_i)^T S0.  Small N only (O(N^2) memory, O(N^2) loops)."""
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    a = _f64(a)
    L = gate_mask(a)
    A = (fq @ np.swapaxes(fk, -1, -2)) * L
    num = A @ v
    den = np.sum(A, axis=-1)
    if S0 is not None:
        lead = np.cumprod(a, axis=-1)                    # a_0 ... a_i
        num = num + lead[..., None] * (fq @ _f64(S0))
        den = den + lead * np.einsum("...nr,...r->...n", fq, _f64(z0))
    if not normalize:
        return num
    return num / den[..., None]


def recurrent_gated(q, k, v, a, phi="elu1", omega=None, normalize=True, S0=None, z0=None):
    """Token recurrence: S = a_t S + phi(k_t) v_t^T, z = a_t z + phi(k_t),
    o_t = phi(q_t)^T S (/ phi(q_t)^T z).  Returns (O, S_N, z_N)."""
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    a = _f64(a)
    lead = fq.shape[:-2]
    n, r = fq.shape[-2], fq.shape[-1]
    dv = v.shape[-1]
    S = np.zeros(lead + (r, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(lead + (r,)) if z0 is None else _f64(z0).copy()
    out = np.empty(lead + (n, dv))
    for t in range(n):
        at = a[..., t]
        kt = fk[..., t, :]
        S = at[..., None, None] * S + kt[..., :, None] * v[..., t, None, :]
        z = at[..., None] * z + kt
        qt = fq[..., t, :]
        num = np.einsum("...r,...rc->...c", qt, S)
        if normalize:
            num = num / np.einsum("...r,...r->...", qt, z)[..., None]
        out[..., t, :] = num
    return out, S, z


def decode_step_gated(S, z, q, k, v, a, phi="elu1", omega=None, normalize=True):
    """One gated step: S' = a S + phi(k) v^T, z' = a z + phi(k), o as above.
    a: one gate per (batch, head) for this token."""
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    a = _f64(a)
    S_new = a[..., None, None] * _f64(S) + fk[..., :, None] * v[..., None, :]
    z_new = a[..., None] * _f64(z) + fk
    o = np.einsum("...r,...rc->...c", fq, S_new)
    if normalize:
        o = o / np.einsum("...r,...r->...", fq, z_new)[..., None]
    return o, S_new, z_new


def causal_rows_gated(q, k, v, a, rows, phi="elu1", omega=None, normalize=True):
    """Rows of one head's output from the definition: o_t = sum_{j<=t}
    (a_{j+1} ... a_t) w_j v_j (/ the same sum of weights) with
    w_j = phi(q_t) . phi(k_j).  q, k: [N, d]; v: [N, dv]; a: [N]."""
    v = _f64(v)
    a = _f64(a)
    out = np.empty((len(rows), v.shape[-1]))
    for idx, t in enumerate(rows):
        fq = feature_map(phi, q[t], omega)
        fk = feature_map(phi, k[: t + 1], omega)
        # lag products a_{j+1} ... a_t for j = 0..t (reverse cumulative product)
        tail = np.ones(t + 1)
        if t > 0:
            tail[:-1] = np.cumprod(a[1: t + 1][::-1])[::-1]
        w = (fk @ fq) * tail
        num = w @ v[: t + 1]
        out[idx] = num / np.sum(w) if normalize else num
    return out
