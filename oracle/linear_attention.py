"""fp64 CPU oracle for causal kernelized linear attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; the only thing both sides share is the seeded input generator, which
holds none of the method's arithmetic.

Sources (web pages, cited by title and section):

* [LAK] "Linear attention kernel" (operatorworld.com, ai-linear-attention-kernel),
  sections "Rewrite: associativity is the whole story", "Choice of phi",
  "Recurrent form".
* [EAV] "Efficient attention variants: from sparse and low-rank to linear
  attention" (bailixisu.com), sections 4 (linear attention), 5 (causal linear
  attention), 5.1 (hand-worked example), 6 (Performer), 10 (hands-on check).
* [LASSM] "Linear attention and SSM" (t6page.pages.dev), sections "How does
  linear attention remove softmax" (eq. attn-linssm-kernel) and "Why is linear
  attention an RNN" (eq. attn-linssm-recurrence).

What is computed (plain definitions, written out; no blocking, no fusion):

* feature maps phi: ELU(x)+1 with alpha=1, Performer positive random features
  (FAVOR+), and the identity (used to feed the pages' hand examples, which give
  features directly);
* the explicit form: weights A = phi(Q) phi(K)^T, lower-triangular with the
  diagonal kept when causal, O = (A V) / rowsum(A);
* the recurrent form: S_t = S_{t-1} + phi(k_t) v_t^T, z_t = z_{t-1} + phi(k_t),
  o_t = phi(q_t)^T S_t / phi(q_t)^T z_t, with S_0 = 0, z_0 = 0 (or a given state);
* the non-causal reassociated form: S = phi(K)^T V, z = sum_j phi(k_j),
  O = phi(Q) S / phi(Q) z;
* one decode step of the recurrence;
* single output rows of the causal / non-causal definition (for sampled parity
  checks at sizes where the full forms are too slow).

Readings taken where the pages are silent:
normalised read-out; the causal mask keeps j == t; no scaling of q, k before
ELU+1; alpha = 1; no epsilon in the denominator; S_0 = 0, z_0 = 0 unless a
state is given; FAVOR+ keeps the 1/sqrt(r) factor and uses x = u / d**(1/4);
every (batch, head) has its own state.

Arrays use the layout [..., N, d] for Q, K, [..., N, d_v] for V and O,
[..., r, d_v] for S and [..., r] for z, where "..." are independent batch/head
dimensions.  Every function upcasts its inputs to float64.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(worked examples printed on the pages, closed forms, invariants, agreement of
the independent explicit and recurrent algorithms, and a Monte Carlo check of
the FAVOR+ expectation identity).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "phi_elu1",
    "phi_favor",
    "phi_identity",
    "feature_map",
    "explicit_attention",
    "recurrent_attention",
    "noncausal_attention",
    "decode_step",
    "causal_rows",
    "noncausal_rows",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Feature maps
# --------------------------------------------------------------------------

def phi_elu1(x):
    """ELU(x) + 1 with alpha = 1, elementwise ([LAK] "Choice of phi";
    [EAV] sec. 4 and sec. 10; [LASSM] "Why is linear attention an RNN").

    ELU(x) is x for x > 0 and alpha * (e^x - 1) otherwise; adding 1 gives
    x + 1 for x > 0 and e^x for x <= 0.  The second branch is evaluated as
    e^x itself (forming e^x - 1 and adding 1 back cancels to 0 for x below
    about -37 and would lose positivity).  The exponential is only evaluated
    on non-positive arguments.
    """
    x = _f64(x)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_favor(u, omega):
    """Performer positive random features (FAVOR+), [EAV] sec. 6.

    With x = u / d**(1/4) (so that x.y = q.k / sqrt(d)), and for each random
    row w of ``omega`` ([r, d]), the feature is exp(w.x - |x|^2 / 2) / sqrt(r).
    The expectation over w ~ N(0, I) of phi(x).phi(y) * r / r equals exp(x.y).
    ``u``: [..., d]; returns [..., r].
    """
    u = _f64(u)
    omega = _f64(omega)
    d = u.shape[-1]
    r = omega.shape[0]
    x = u / d ** 0.25
    proj = x @ omega.T                                  # [..., r]
    half_sq_norm = 0.5 * np.sum(x * x, axis=-1, keepdims=True)
    return np.exp(proj - half_sq_norm) / np.sqrt(r)


def phi_identity(u):
    """Identity map: the features are the inputs themselves.  Used to feed
    the hand-worked examples of [EAV] sec. 5.1 and sec. 7.3, which state the
    features phi(k) directly."""
    return _f64(u)


def feature_map(kind, x, omega=None):
    """Dispatch on the feature-map name: "elu1", "favor" or "identity"."""
    if kind == "elu1":
        return phi_elu1(x)
    if kind == "favor":
        if omega is None:
            raise ValueError("favor feature map needs omega [r, d]")
        return phi_favor(x, omega)
    if kind == "identity":
        return phi_identity(x)
    raise ValueError(f"unknown feature map {kind!r}")


# --------------------------------------------------------------------------
# Full-sequence forms
# --------------------------------------------------------------------------

def explicit_attention(q, k, v, phi="elu1", causal=True, omega=None):
    """Explicit N x N weight form ([EAV] sec. 4 figure 2, sec. 10 dense
    function; [LASSM] table "left product").

    A[i, j] = phi(q_i) . phi(k_j); when causal every j > i is set to zero
    and the diagonal is kept; O = (A V) / rowsum(A).  O(N^2) memory: only for
    small N.
    """
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    a = fq @ np.swapaxes(fk, -1, -2)                    # [..., N, N]
    if causal:
        n = a.shape[-1]
        keep = np.tril(np.ones((n, n), dtype=bool))     # j <= i
        a = np.where(keep, a, 0.0)
    num = a @ v
    den = np.sum(a, axis=-1, keepdims=True)
    return num / den


def recurrent_attention(q, k, v, phi="elu1", omega=None, S0=None, z0=None):
    """Token-by-token recurrence ([LAK] "Recurrent form"; [EAV] sec. 5;
    [LASSM] eq. attn-linssm-recurrence, with the denominator of
    eq. attn-linssm-kernel).

    For t = 1..N: first write S_t = S_{t-1} + phi(k_t) v_t^T and
    z_t = z_{t-1} + phi(k_t), then read o_t = phi(q_t)^T S_t / phi(q_t)^T z_t
    (so token t attends to itself).  S_0, z_0 default to zero.

    The loop runs over tokens; batch/head dimensions are vectorised.
    Returns (O, S_N, z_N).
    """
    fq = feature_map(phi, q, omega)                     # [..., N, r]
    fk = feature_map(phi, k, omega)
    v = _f64(v)                                         # [..., N, dv]
    lead = fq.shape[:-2]
    n, r = fq.shape[-2], fq.shape[-1]
    dv = v.shape[-1]
    S = np.zeros(lead + (r, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(lead + (r,)) if z0 is None else _f64(z0).copy()
    out = np.empty(lead + (n, dv))
    for t in range(n):
        kt = fk[..., t, :]                              # [..., r]
        S += kt[..., :, None] * v[..., t, None, :]      # outer product
        z += kt
        qt = fq[..., t, :]
        num = np.einsum("...r,...rc->...c", qt, S)
        den = np.einsum("...r,...r->...", qt, z)
        out[..., t, :] = num / den[..., None]
    return out, S, z


def noncausal_attention(q, k, v, phi="elu1", omega=None, S0=None, z0=None):
    """Non-causal reassociated form, right product first ([LAK] "Rewrite:
    associativity"; [EAV] sec. 4; [LASSM] table "right product first").

    S = S0 + phi(K)^T V, z = z0 + sum_j phi(k_j), O = phi(Q) S / phi(Q) z.
    Returns (O, S, z).
    """
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    S = np.swapaxes(fk, -1, -2) @ v                     # [..., r, dv]
    z = np.sum(fk, axis=-2)                             # [..., r]
    if S0 is not None:
        S = S + _f64(S0)
    if z0 is not None:
        z = z + _f64(z0)
    num = fq @ S
    den = np.einsum("...nr,...r->...n", fq, z)
    return num / den[..., None], S, z


def decode_step(S, z, q, k, v, phi="elu1", omega=None):
    """One autoregressive step of the recurrence ([EAV] sec. 5; [LAK]
    "Recurrent form"; [LASSM] "Why is linear attention an RNN").

    S: [..., r, dv], z: [..., r], q, k: [..., d], v: [..., dv].
    S' = S + phi(k) v^T, z' = z + phi(k), o = phi(q)^T S' / phi(q)^T z'.
    Returns (o, S', z').
    """
    fq = feature_map(phi, q, omega)
    fk = feature_map(phi, k, omega)
    v = _f64(v)
    S_new = _f64(S) + fk[..., :, None] * v[..., None, :]
    z_new = _f64(z) + fk
    num = np.einsum("...r,...rc->...c", fq, S_new)
    den = np.einsum("...r,...r->...", fq, z_new)
    return num / den[..., None], S_new, z_new


# --------------------------------------------------------------------------
# Single rows of the definition (sampled parity at full size)
# --------------------------------------------------------------------------

def causal_rows(q, k, v, rows, phi="elu1", omega=None, S0=None, z0=None):
    """Rows ``rows`` of the causal output of one head, straight from the
    definition: o_t = (phi(q_t)^T S0 + sum_{j<=t} w_j v_j) /
    (phi(q_t)^T z0 + sum_{j<=t} w_j) with w_j = phi(q_t) . phi(k_j)
    ([EAV] sec. 4 and sec. 5).

    q, k: [N, d]; v: [N, dv]; rows: iterable of token indices.
    Returns [len(rows), dv].
    """
    v = _f64(v)
    out = np.empty((len(rows), v.shape[-1]))
    for idx, t in enumerate(rows):
        fq = feature_map(phi, q[t], omega)              # [r]
        fk = feature_map(phi, k[: t + 1], omega)        # [t+1, r]
        w = fk @ fq                                     # [t+1]
        num = w @ v[: t + 1]
        den = np.sum(w)
        if S0 is not None:
            num = num + fq @ _f64(S0)
            den = den + fq @ _f64(z0)
        out[idx] = num / den
    return out


def noncausal_rows(q, k, v, rows, phi="elu1", omega=None):
    """Rows of the non-causal output of one head: every key contributes,
    o_i = sum_j w_j v_j / sum_j w_j with w_j = phi(q_i) . phi(k_j)
    ([EAV] sec. 4)."""
    v = _f64(v)
    fk = feature_map(phi, k, omega)                     # [N, r]
    out = np.empty((len(rows), v.shape[-1]))
    for idx, t in enumerate(rows):
        fq = feature_map(phi, q[t], omega)
        w = fk @ fq
        out[idx] = (w @ v) / np.sum(w)
    return out
