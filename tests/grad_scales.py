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
    for t in range(n):
        S += fk[..., t, :, None] * v[..., t, None, :]
        z += fk[..., t, :]
        Dt = np.einsum("...r,...r->...", fq[..., t, :], z)
        Ot = np.einsum("...r,...rc->...c", fq[..., t, :], S) / Dt[..., None]
        D[..., t] = Dt
        g[..., t, :] = dO[..., t, :] / Dt[..., None]
        h[..., t] = -np.einsum("...c,...c->...", dO[..., t, :], Ot) / Dt
        sq[..., t, :] = np.abs(np.einsum("...rc,...c->...r", S, g[..., t, :])) + np.abs(h[..., t, None]) * z
    sq *= np.abs(bwd.phi_prime(phi, q))
    R = np.zeros(lead + (r, dv))
    Ra = np.zeros(lead + (r, dv))
    u = np.zeros(lead + (r,))
    sk = np.empty(fk.shape)
    sv = np.empty(v.shape)
    adO = np.abs(dO)
    for t in range(n - 1, -1, -1):
        R += fq[..., t, :, None] * g[..., t, None, :]
        Ra += fq[..., t, :, None] * (adO[..., t, None, :] / D[..., t, None, None])
        u += fq[..., t, :] * h[..., t, None]
        sk[..., t, :] = np.abs(np.einsum("...rc,...c->...r", R, v[..., t, :])) + np.abs(u)
        sv[..., t, :] = np.einsum("...rc,...r->...c", Ra, fk[..., t, :])
    sk *= np.abs(bwd.phi_prime(phi, k))
    return sq, sk, sv
