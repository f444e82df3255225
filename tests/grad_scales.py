"""Magnitudes of the intermediate sums the backward kernels form, for the
cancellation floor of the gradient gate (tests/gates.py, check_grad).

Each gradient row is a difference of two large sums that cancel most of
each other:
    dphi(q_i) = S_i g_i + h_i z_i,                  (forward prefix sums)
    dphi(k_j) = R_j v_j + u_j,                      (reverse suffix sums)
with S_i = sum_{j<=i} phi(k_j) v_j^T, z_i = sum_{j<=i} phi(k_j),
g_i = dO_i / D_i, h_i = -(dO_i . O_i) / D_i, R_j = sum_{i>=j} phi(q_i) g_i^T,
u_j = sum_{i>=j} phi(q_i) h_i (the chain rule of oracle/backward.py,
regrouped by the associativity of the recurrent form).  bf16 rounding
inside the kernels is relative to these sums, not to their difference, so
the floor of a row is taken relative to
    m(dQ_i) = |phi'(q_i)| (|S_i g_i| + |h_i| z_i),
    m(dK_j) = |phi'(k_j)| (|R_j v_j| + |u_j|),
    m(dV_j) = Ra_j^T phi(k_j),  Ra_j = sum_{i>=j} phi(q_i) |dO_i|^T / D_i
(dV is a single sum of mixed-sign terms; its magnitude sum).
The dot products over the value channels inside those sums (S_i g_i,
dO_i . O_i in h_i, R_j v_j) take operands that the kernels hold in bf16 (g,
the published S, O), whose rounding is relative to the products' terms, not
to the dot product.  Where a dot product cancels almost entirely the sums are
small against that: for a head's first token o_0 = v_0, so S_0 g_0 and h_0 z_0
are equal and opposite and dQ_0 = 0, and when v_0 . dO_0 is itself a small
fraction of |v_0| . |dO_0| the rounding of g_0 and O_0 outweighs both sums.
So each magnitude is at least 1/16 of the same sums taken with the channel
products in absolute value,
    m'(dQ_i) = |phi'(q_i)| (|S_i| |g_i| + (|dO_i| . |O_i|) / D_i z_i),
    m'(dK_j) = |phi'(k_j)| (|R_j| |v_j| + sum_{i>=j} |phi(q_i)| (|dO_i| . |O_i|) / D_i),
which puts the floor of such rows (2^-4 m, tests/gates.py) at 2^-8 of m',
about 2^-9 bf16 rounding of two or three operands.  For typical rows m'/16
is below m (the dot products cancel like sqrt(d_v)) and m is unchanged.
One forward and one reverse fp64 token loop, vectorised over the leading
axes.  Test infrastructure: NumPy, built on the oracle's feature maps.
"""

from __future__ import annotations

import numpy as np

from oracle import backward as bwd
from oracle import linear_attention as ora


def grad_scales(q, k, v, dO, phi="elu1"):
    fq = ora.feature_map(phi, q)
    fk = ora.feature_map(phi, k)
    v = np.asarray(v, np.float64)
    dO = np.asarray(dO, np.float64)
    lead = fq.shape[:-2]
    n, r = fq.shape[-2], fq.shape[-1]
    dv = v.shape[-1]
    S = np.zeros(lead + (r, dv))
    z = np.zeros(lead + (r,))
    D = np.empty(lead + (n,))
    g = np.empty(lead + (n, dv))
    h = np.empty(lead + (n,))
    sq = np.empty(fq.shape)
    sq_in = np.empty(fq.shape)
    h_in = np.empty(lead + (n,))  # (|dO_i| . |O_i|) / D_i
    for t in range(n):
        S += fk[..., t, :, None] * v[..., t, None, :]
        z += fk[..., t, :]
        Dt = np.einsum("...r,...r->...", fq[..., t, :], z)
        Ot = np.einsum("...r,...rc->...c", fq[..., t, :], S) / Dt[..., None]
        D[..., t] = Dt
        g[..., t, :] = dO[..., t, :] / Dt[..., None]
        h[..., t] = -np.einsum("...c,...c->...", dO[..., t, :], Ot) / Dt
        h_in[..., t] = np.einsum("...c,...c->...", np.abs(dO[..., t, :]), np.abs(Ot)) / np.abs(Dt)
        sq[..., t, :] = np.abs(np.einsum("...rc,...c->...r", S, g[..., t, :])) + np.abs(h[..., t, None]) * z
        sq_in[..., t, :] = (np.einsum("...rc,...c->...r", np.abs(S), np.abs(g[..., t, :]))
                            + h_in[..., t, None] * np.abs(z))
    sq = np.maximum(sq, sq_in / 16.0) * np.abs(bwd.phi_prime(phi, q))
    R = np.zeros(lead + (r, dv))
    Ra = np.zeros(lead + (r, dv))
    u = np.zeros(lead + (r,))
    sk = np.empty(fk.shape)
    sk_in = np.empty(fk.shape)
    sv = np.empty(v.shape)
    adO = np.abs(dO)
    u_in = np.zeros(lead + (r,))
    for t in range(n - 1, -1, -1):
        R += fq[..., t, :, None] * g[..., t, None, :]
        Ra += fq[..., t, :, None] * (adO[..., t, None, :] / D[..., t, None, None])
        u += fq[..., t, :] * h[..., t, None]
        u_in += np.abs(fq[..., t, :]) * h_in[..., t, None]
        sk[..., t, :] = np.abs(np.einsum("...rc,...c->...r", R, v[..., t, :])) + np.abs(u)
        sk_in[..., t, :] = np.einsum("...rc,...c->...r", np.abs(R), np.abs(v[..., t, :])) + u_in
        sv[..., t, :] = np.einsum("...rc,...r->...c", Ra, fk[..., t, :])
    sk = np.maximum(sk, sk_in / 16.0) * np.abs(bwd.phi_prime(phi, k))
    return sq, sk, sv
