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

__all__ = ["phi_prime", "grad_causal"]


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
