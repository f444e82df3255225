"""fp64 CPU oracle for causal linear attention with a fixed per-head decay.

TEST INFRASTRUCTURE ONLY, like ``oracle.linear_attention``: nothing in the
product path may import, call or link this module (only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``).
It shares no code with the HIP library.

Source: "Efficient attention variants: from sparse and low-rank to linear
attention" (bailixisu.com), sec. 7.1 (RetNet): the state is multiplied by a
fixed per-head gamma before each write, S_t = gamma S_{t-1} + k_t v_t^T,
o_t = q_t^T S_t, so that record j enters o_t with gamma^(t-j); with
gamma = 0.99 a record 100 steps old weighs about 0.366.  The section states
that such recurrences leave out output normalisation and need not use the
z denominator of the non-negative kernels (sec. 5).

Readings taken (the page gives only the recurrence above):

* the feature map phi of the hot path is applied to q and k as before
  (phi = identity gives the page's formula exactly);
* with ``normalize=True`` the normaliser decays with the state,
  z_t = gamma z_{t-1} + phi(k_t), and o_t = phi(q_t)^T S_t / phi(q_t)^T z_t,
  a weighted mean of v_j with weights gamma^(t-j) phi(q_t).phi(k_j); with
  gamma = 1 this is the plain causal linear attention of sec. 5;
* with ``normalize=False`` o_t = phi(q_t)^T S_t, the page's form;
* gamma is one value per (batch, head) pair (broadcast from an array
  whose shape is a suffix of the leading dimensions, e.g. [H]);
* an initial state S0, z0 is decayed like any earlier record: it enters
  o_t (0-based t) with gamma^(t+1).

Every function upcasts to float64.  Pins: tests/test_oracle_decay_pins.py.
"""

from __future__ import annotations

import numpy as np

from oracle.linear_attention import feature_map

__all__ = ["explicit_decay", "recurrent_decay", "decode_step_decay", "causal_rows_decay"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _gamma(gamma, lead):
    return np.broadcast_to(_f64(gamma), lead)


def explicit_decay(q, k, v, gamma, phi="elu1", omega=None, normalize=True, S0=None, z0=None):
    """Explicit weight form: A[i, j] = gamma^(i - j) phi(q_i) . phi(k_j) for
    j <= i (zero above the diagonal), O = A V (divided by rowsum(A) when
    normalising), plus the decayed initial state gamma^(i+1) phi(q_i)^T S0
    (and z0).  O(N^2) memory: small N only."""
    fq = feature_map(phi, q, omega)                     # [..., N, r]
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    lead = fq.shape[:-2]
    n = fq.shape[-2]
    g = _gamma(gamma, lead)[..., None, None]            # [..., 1, 1]
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    expo = np.where(j <= i, i - j, 0).astype(np.float64)
    decay = np.where(j <= i, g ** expo, 0.0)            # [..., N, N]
    a = (fq @ np.swapaxes(fk, -1, -2)) * decay
    num = a @ v
    den = np.sum(a, axis=-1)
    if S0 is not None:
        lag = g[..., 0] ** (np.arange(n) + 1.0)          # [..., N]
        num = num + lag[..., None] * (fq @ _f64(S0))
        den = den + lag * np.einsum("...nr,...r->...n", fq, _f64(z0))
    if not normalize:
        return num
    return num / den[..., None]


def recurrent_decay(q, k, v, gamma, phi="elu1", omega=None, normalize=True, S0=None, z0=None):
    """Token recurrence of sec. 7.1: for t = 0..N-1, S = gamma S + phi(k_t)
    v_t^T and z = gamma z + phi(k_t) (write), then o_t = phi(q_t)^T S
    (divided by phi(q_t)^T z when normalising).  Returns (O, S_N, z_N)."""
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    lead = fq.shape[:-2]
    n, r = fq.shape[-2], fq.shape[-1]
    dv = v.shape[-1]
    g = _gamma(gamma, lead)
    S = np.zeros(lead + (r, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(lead + (r,)) if z0 is None else _f64(z0).copy()
    out = np.empty(lead + (n, dv))
    for t in range(n):
        kt = fk[..., t, :]
        S = g[..., None, None] * S + kt[..., :, None] * v[..., t, None, :]
        z = g[..., None] * z + kt
        qt = fq[..., t, :]
        num = np.einsum("...r,...rc->...c", qt, S)
        if normalize:
            num = num / np.einsum("...r,...r->...", qt, z)[..., None]
        out[..., t, :] = num
    return out, S, z


def decode_step_decay(S, z, q, k, v, gamma, phi="elu1", omega=None, normalize=True):
    """One step of the decayed recurrence: S' = gamma S + phi(k) v^T,
    z' = gamma z + phi(k), o = phi(q)^T S' (/ phi(q)^T z').  Returns
    (o, S', z')."""
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    g = _gamma(gamma, fq.shape[:-1])
    S_new = g[..., None, None] * _f64(S) + fk[..., :, None] * v[..., None, :]
    z_new = g[..., None] * _f64(z) + fk
    o = np.einsum("...r,...rc->...c", fq, S_new)
    if normalize:
        o = o / np.einsum("...r,...r->...", fq, z_new)[..., None]
    return o, S_new, z_new


def causal_rows_decay(q, k, v, rows, gamma, phi="elu1", omega=None, normalize=True):
    """Rows of one head's output straight from the definition:
    o_t = sum_{j<=t} gamma^(t-j) w_j v_j (/ sum_{j<=t} gamma^(t-j) w_j) with
    w_j = phi(q_t) . phi(k_j).  q, k: [N, d]; v: [N, dv]; gamma: scalar."""
    v = _f64(v)
    g = float(gamma)
    out = np.empty((len(rows), v.shape[-1]))
    for idx, t in enumerate(rows):
        fq = feature_map(phi, q[t], omega)
        fk = feature_map(phi, k[: t + 1], omega)
        w = (fk @ fq) * g ** (t - np.arange(t + 1, dtype=np.float64))
        num = w @ v[: t + 1]
        out[idx] = num / np.sum(w) if normalize else num
    return out
