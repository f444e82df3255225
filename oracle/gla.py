"""fp64 CPU oracle for causal linear attention with a data-dependent gate per
key channel (the GLA form; RWKV-5/6's state update has the same shape).

TEST INFRASTRUCTURE ONLY, like ``oracle.linear_attention``: nothing in the
product path may import, call or link this module (only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``).
It shares no code with the HIP library.

Source: "Efficient attention variants: from sparse and low-rank to linear
attention" (bailixisu.com), sec. 7.2 (GLA): S_t = diag(alpha_t) S_{t-1} +
k_t v_t^T with alpha_t in (0, 1)^d; entry f of alpha_t sets how much of row
f of the state (key channel f) is kept, the same for every value column, and
it depends on the input, so each position and channel forgets at its own
rate.  "Linear attention and SSM" (t6page.pages.dev), section "Why is
linear attention equivalent to an RNN", gives RWKV-5/6's M_s = diag(w)
M_{s-1} + k_s^T v_s as an instance of the same decayed-state update.

Readings taken (as for the fixed decay, oracle.decay):

* the feature map phi of the hot path is applied to q and k; the gates act
  on the feature rows of S (r = d for the pointwise maps);
* the normaliser is gated like the state, z_t = diag(alpha_t) z_{t-1} +
  phi(k_t); the read-out is o_t = phi(q_t)^T S_t / phi(q_t)^T z_t, or
  phi(q_t)^T S_t with ``normalize=False`` (the page's form);
* record j enters o_t through channel f with the product alpha_{j+1,f} ...
  alpha_{t,f} (so a record is not gated at its own step);
* an initial state S0, z0 enters o_t (0-based t) through channel f with
  alpha_{0,f} ... alpha_{t,f}.

Every function upcasts to float64.  Pins: tests/test_oracle_gla_pins.py.
"""

from __future__ import annotations

import numpy as np

from oracle.linear_attention import feature_map

__all__ = ["explicit_gla", "recurrent_gla", "decode_step_gla", "causal_rows_gla"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _lag_products(alpha, i, j):
    """alpha_{j+1} ... alpha_i per channel (ones when j == i): [..., r]."""
    out = np.ones(alpha.shape[:-2] + alpha.shape[-1:])
    for l in range(j + 1, i + 1):
        out = out * alpha[..., l, :]
    return out


def explicit_gla(q, k, v, alpha, phi="elu1", omega=None, normalize=True, S0=None, z0=None):
    """Weight form: A[i, j] = sum_f phi(q_i)_f phi(k_j)_f prod_{l=j+1..i}
    alpha_{l,f} for j <= i, O = A V (divided by rowsum(A) when normalising),
    plus the gated initial state.  alpha: [..., N, r].  O(N^2 r) loops: small
    N only."""
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    alpha = _f64(alpha)
    n = fq.shape[-2]
    lead = fq.shape[:-2]
    A = np.zeros(lead + (n, n))
    for i in range(n):
        for j in range(i + 1):
            A[..., i, j] = np.sum(fq[..., i, :] * fk[..., j, :] * _lag_products(alpha, i, j), axis=-1)
    num = A @ v
    den = np.sum(A, axis=-1)
    if S0 is not None:
        S0 = _f64(S0)
        z0 = _f64(z0)
        run = np.ones(lead + fq.shape[-1:])
        for i in range(n):
            run = run * alpha[..., i, :]                   # alpha_0 ... alpha_i
            g = fq[..., i, :] * run
            num[..., i, :] += np.einsum("...r,...rc->...c", g, S0)
            den[..., i] += np.einsum("...r,...r->...", g, z0)
    if not normalize:
        return num
    return num / den[..., None]


def recurrent_gla(q, k, v, alpha, phi="elu1", omega=None, normalize=True, S0=None, z0=None):
    """Token recurrence: S = diag(alpha_t) S + phi(k_t) v_t^T, z = alpha_t z +
    phi(k_t), o_t = phi(q_t)^T S (/ phi(q_t)^T z).  Returns (O, S_N, z_N)."""
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    alpha = _f64(alpha)
    lead = fq.shape[:-2]
    n, r = fq.shape[-2], fq.shape[-1]
    dv = v.shape[-1]
    S = np.zeros(lead + (r, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(lead + (r,)) if z0 is None else _f64(z0).copy()
    out = np.empty(lead + (n, dv))
    for t in range(n):
        at = alpha[..., t, :]
        kt = fk[..., t, :]
        S = at[..., :, None] * S + kt[..., :, None] * v[..., t, None, :]
        z = at * z + kt
        qt = fq[..., t, :]
        num = np.einsum("...r,...rc->...c", qt, S)
        if normalize:
            num = num / np.einsum("...r,...r->...", qt, z)[..., None]
        out[..., t, :] = num
    return out, S, z


def decode_step_gla(S, z, q, k, v, alpha, phi="elu1", omega=None, normalize=True):
    """One step: S' = diag(alpha) S + phi(k) v^T, z' = alpha z + phi(k).
    alpha: [..., r], this token's gates."""
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    alpha = _f64(alpha)
    S_new = alpha[..., :, None] * _f64(S) + fk[..., :, None] * v[..., None, :]
    z_new = alpha * _f64(z) + fk
    o = np.einsum("...r,...rc->...c", fq, S_new)
    if normalize:
        o = o / np.einsum("...r,...r->...", fq, z_new)[..., None]
    return o, S_new, z_new


def causal_rows_gla(q, k, v, alpha, rows, phi="elu1", omega=None, normalize=True):
    """Rows of one head's output from the definition: o_t = sum_{j<=t} w_j v_j
    (/ sum_j w_j) with w_j = sum_f phi(q_t)_f phi(k_j)_f (alpha_{j+1,f} ...
    alpha_{t,f}).  q, k: [N, d]; v: [N, dv]; alpha: [N, r]."""
    v = _f64(v)
    alpha = _f64(alpha)
    out = np.empty((len(rows), v.shape[-1]))
    for idx, t in enumerate(rows):
        fq = feature_map(phi, q[t], omega)
        fk = feature_map(phi, k[: t + 1], omega)
        # per-channel lag products alpha_{j+1} ... alpha_t, j = 0..t
        tail = np.ones((t + 1, alpha.shape[-1]))
        if t > 0:
            tail[:-1] = np.cumprod(alpha[1: t + 1][::-1], axis=0)[::-1]
        w = np.sum(fk * tail * fq[None, :], axis=-1)
        num = w @ v[: t + 1]
        out[idx] = num / np.sum(w) if normalize else num
    return out
