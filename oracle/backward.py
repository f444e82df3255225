"""fp64 CPU oracle for the gradients of causal kernelized linear attention.

TEST INFRASTRUCTURE ONLY, like ``oracle.linear_attention``: nothing in the
product path may import, call or link this module (only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``).
It shares no code with the HIP library.

The pages do not derive a backward pass: "Efficient attention variants"
(bailixisu.com) names backpropagation among the costs that decide whether a
linear layer is fast in practice (sec. 8) and leaves it out of its hands-on
check (sec. 10).  What is differentiated here is the forward the pages do
define (sec. 5, causal, normalised): with A = tril(phi(Q) phi(K)^T) (the
diagonal kept), D = rowsum(A) and O = diag(D)^-1 A V, and a given upstream
gradient dO of the same shape as O, the reverse-mode chain rule on that
explicit quadratic form gives

    dA     = (dO V^T - rowsum(dO * O) 1^T) / D      (row-wise; kept only on and
                                                     below the diagonal)
    dphi(Q) = dA phi(K),   dphi(K) = dA^T phi(Q),   dV = (diag(D)^-1 A)^T dO,
    dQ = dphi(Q) * phi'(Q),  dK = dphi(K) * phi'(K)  (elementwise)

with phi' of ELU+1 (alpha = 1) equal to 1 for x > 0 and e^x otherwise, and
1 for the identity.  Readings: no initial state (S_0 = 0, z_0 = 0); the
feature map's own parameters (FAVOR+'s omega) are not differentiated.

Everything is fp64 and O(N^2): small N only.  Pins (finite differences of the
forward oracle, closed forms): tests/test_oracle_backward_pins.py.
"""

from __future__ import annotations

import numpy as np

from oracle.linear_attention import feature_map

__all__ = ["phi_prime", "grad_causal", "grad_rows"]


def phi_prime(phi, x):
    """Derivative of the pointwise feature map, elementwise."""
    x = np.asarray(x, dtype=np.float64)
    if phi == "elu1":
        return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    if phi == "identity":
        return np.ones_like(x)
    raise ValueError(f"no derivative for feature map {phi!r}")


def grad_causal(q, k, v, dO, phi="elu1"):
    """(dQ, dK, dV) of sum(dO * O) for the causal normalised output O of
    q, k [..., N, d], v [..., N, dv] (the chain rule written out on the
    explicit form above)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    fq = feature_map(phi, q)
    fk = feature_map(phi, k)
    n = fq.shape[-2]
    mask = np.tril(np.ones((n, n)))
    A = (fq @ np.swapaxes(fk, -1, -2)) * mask
    D = A.sum(axis=-1)
    O = (A @ v) / D[..., None]
    rho = np.sum(dO * O, axis=-1)                                  # [..., N]
    dA = ((dO @ np.swapaxes(v, -1, -2)) - rho[..., None]) / D[..., None] * mask
    dfq = dA @ fk
    dfk = np.swapaxes(dA, -1, -2) @ fq
    dv = np.swapaxes(A / D[..., None], -1, -2) @ dO
    return dfq * phi_prime(phi, q), dfk * phi_prime(phi, k), dv


def grad_rows(q, k, v, dO, rows, phi="elu1"):
    """The same gradients at selected token rows, for long sequences: one
    forward token loop (prefix sums S_t, z_t of the recurrence, then D_t,
    O_t, g_t = dO_t / D_t, h_t = -(dO_t . O_t) / D_t) and one reverse loop
    (suffix sums R_t = sum_{i>=t} phi(q_i) g_i^T, u_t = sum_{i>=t} phi(q_i)
    h_i), from which
        dphi(q_t) = S_t g_t + h_t z_t,  dphi(k_t) = R_t v_t + u_t,
        dv_t = R_t^T phi(k_t),
    i.e. the sums of grad_causal regrouped by the associativity the
    recurrent form rests on.  Vectorised over the leading dimensions; returns
    (dQ, dK, dV) at ``rows`` ([..., len(rows), d] etc.).  Pinned against
    grad_causal in tests/test_oracle_backward_pins.py."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    fq = feature_map(phi, q)
    fk = feature_map(phi, k)
    lead = fq.shape[:-2]
    n, r = fq.shape[-2], fq.shape[-1]
    dv_ = v.shape[-1]
    want = {t: i for i, t in enumerate(rows)}
    gq = np.empty(lead + (len(rows), r))
    gk = np.empty(lead + (len(rows), r))
    gv = np.empty(lead + (len(rows), dv_))
    g = np.empty(lead + (n, dv_))
    h = np.empty(lead + (n,))
    S = np.zeros(lead + (r, dv_))
    z = np.zeros(lead + (r,))
    for t in range(n):
        S = S + fk[..., t, :, None] * v[..., t, None, :]
        z = z + fk[..., t, :]
        D = np.einsum("...r,...r->...", fq[..., t, :], z)
        O = np.einsum("...r,...rc->...c", fq[..., t, :], S) / D[..., None]
        g[..., t, :] = dO[..., t, :] / D[..., None]
        h[..., t] = -np.einsum("...c,...c->...", dO[..., t, :], O) / D
        if t in want:
            gq[..., want[t], :] = np.einsum("...rc,...c->...r", S, g[..., t, :]) + h[..., t, None] * z
    R = np.zeros(lead + (r, dv_))
    u = np.zeros(lead + (r,))
    for t in range(n - 1, -1, -1):
        R = R + fq[..., t, :, None] * g[..., t, None, :]
        u = u + fq[..., t, :] * h[..., t, None]
        if t in want:
            gk[..., want[t], :] = np.einsum("...rc,...c->...r", R, v[..., t, :]) + u
            gv[..., want[t], :] = np.einsum("...rc,...r->...c", R, fk[..., t, :])
    sel = list(rows)
    return gq * phi_prime(phi, q[..., sel, :]), gk * phi_prime(phi, k[..., sel, :]), gv
