"""Dense dual (quadratic) form of the SSD map, fp64, for tiny inputs only.

TEST INFRASTRUCTURE ONLY: used by the oracle's self-checks; the HIP path never
imports it.

The duality the Mamba-2 reading report states (sections 2.2 and 2.3): a
scalar-identity SSM and 1-semiseparable masked attention are the same linear
map. Written as masked attention with C as the query, B as the key and the
input as the value ("Transformers are SSMs" reading report, abstract: the dual
quadratic form (L o Q K^T) V), per (batch, head):

    Y = (L o (C B^T) o 1 dt^T) X + D X,
    L[i, j] = exp(A * sum_{t=j+1..i} dt_t)   for i >= j (so L[i, i] = 1),
    L[i, j] = 0                               for i <  j.

The mask is the data-dependent decay mask L_ij = prod_{t=j+1..i} a_t of the
reading report's section 2.2 with a_t = exp(dt_t A). The dt_j factor on
column j is the zero-order-hold input scaling (Bbar = Delta B, "Mamba
principles in depth", section 2.2). The exponent is summed directly over
t = j+1..i (not taken as a difference of prefix sums), so no cancellation
enters the check.

The final state follows from the same map read at the last row:
    S_T = sum_j exp(A * sum_{t=j+1..T-1} dt_t) * dt_j * x_j (outer) B_j.
"""
from __future__ import annotations

import numpy as np


def decay_mask(dt_col: np.ndarray, a: float) -> np.ndarray:
    """L for one (batch, head): dt_col has shape (T,), fp64."""
    T = dt_col.shape[0]
    L = np.zeros((T, T), dtype=np.float64)
    for i in range(T):
        # seg[j] = sum_{t=j+1..i} dt_t for j = 0..i, summed from t = i downwards
        seg = np.zeros(i + 1, dtype=np.float64)
        if i > 0:
            seg[:i] = np.cumsum(dt_col[i:0:-1])[::-1]
        L[i, : i + 1] = np.exp(a * seg)
    return L


def dual_form(X, dt, A, B, C, D, ngroups: int):
    """X (Bz,T,H,P), dt (Bz,T,H), A (H,), B/C (Bz,T,G,N), D (H,); all fp64.

    Returns (Y (Bz,T,H,P), final_state (Bz,H,P,N)).
    """
    X = np.asarray(X, np.float64)
    dt = np.asarray(dt, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    Bz, T, H, P = X.shape
    N = B.shape[-1]
    Y = np.zeros_like(X)
    final = np.zeros((Bz, H, P, N), dtype=np.float64)
    for b in range(Bz):
        for h in range(H):
            g = (h * ngroups) // H
            Cg, Bg = C[b, :, g, :], B[b, :, g, :]
            d = dt[b, :, h]
            L = decay_mask(d, float(A[h]))
            M = L * (Cg @ Bg.T) * d[None, :]
            x = X[b, :, h, :]
            Y[b, :, h, :] = M @ x + float(D[h]) * x
            # decay from each token j to the end of the sequence: the last row of L
            w = L[T - 1, :] * d if T > 0 else np.zeros(0)
            final[b, h] = (x * w[:, None]).T @ Bg
    return Y, final
