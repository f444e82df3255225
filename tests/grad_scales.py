"""Magnitude sums of the gradient terms, for the cancellation floor of the
gradient gate (tests/gates.py, check_grad).

Each gradient entry is a sum of terms of mixed sign:
    dQ_i = phi'(q_i) sum_{j<=i} (dO_i.v_j + rho_i) / D_i phi(k_j),
    dK_j = phi'(k_j) sum_{i>=j} (dO_i.v_j + rho_i) / D_i phi(q_i),
    dV_j = sum_{i>=j} A_ij / D_i dO_i,
with A_ij = phi(q_i).phi(k_j), D_i = sum_{j<=i} A_ij and rho_i = -dO_i.O_i.
The scale of an entry is the same sum with every factor replaced by its
magnitude.  With phi >= 0 these are prefix and suffix sums again:
    scale(dQ_i) = |phi'(q_i)| (Sa_i |dO_i| + |rho_i| z_i) / D_i,
        Sa_i = sum_{j<=i} phi(k_j) |v_j|^T,  z_i = sum_{j<=i} phi(k_j);
    scale(dK_j) = |phi'(k_j)| (Ra_j |v_j| + ua_j),
        Ra_j = sum_{i>=j} phi(q_i) |dO_i|^T / D_i,  ua_j = sum_{i>=j} phi(q_i) |rho_i| / D_i;
    scale(dV_j) = Ra_j^T phi(k_j).
One forward and one reverse token loop, vectorised over the leading axes.
Test infrastructure: NumPy, built on the oracle's feature maps.
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
    av, adO = np.abs(v), np.abs(dO)
    Sa = np.zeros(lead + (r, dv))
    S = np.zeros(lead + (r, dv))
    z = np.zeros(lead + (r,))
    D = np.empty(lead + (n,))
    rho = np.empty(lead + (n,))
    sq = np.empty(fq.shape)
    for t in range(n):
        S += fk[..., t, :, None] * v[..., t, None, :]
        Sa += fk[..., t, :, None] * av[..., t, None, :]
        z += fk[..., t, :]
        Dt = np.einsum("...r,...r->...", fq[..., t, :], z)
        Ot = np.einsum("...r,...rc->...c", fq[..., t, :], S) / Dt[..., None]
        D[..., t] = Dt
        rho[..., t] = np.abs(np.einsum("...c,...c->...", dO[..., t, :], Ot))
        sq[..., t, :] = (np.einsum("...rc,...c->...r", Sa, adO[..., t, :]) + rho[..., t, None] * z) / Dt[..., None]
    sq *= np.abs(bwd.phi_prime(phi, q))
    Ra = np.zeros(lead + (r, dv))
    ua = np.zeros(lead + (r,))
    sk = np.empty(fk.shape)
    sv = np.empty(v.shape)
    for t in range(n - 1, -1, -1):
        Ra += fq[..., t, :, None] * (adO[..., t, None, :] / D[..., t, None, None])
        ua += fq[..., t, :] * (rho[..., t, None] / D[..., t, None])
        sk[..., t, :] = np.einsum("...rc,...c->...r", Ra, av[..., t, :]) + ua
        sv[..., t, :] = np.einsum("...rc,...r->...c", Ra, fk[..., t, :])
    sk *= np.abs(bwd.phi_prime(phi, k))
    return sq, sk, sv
