"""float64 oracle for the query and key projections of the affinities.

TEST INFRASTRUCTURE: only tests, the build entry module's smoke check and the
benchmark's CPU-baseline leg may use this module.  It imports nothing from the
product package and shares no code with the HIP library.

SequenceO1 reading notes, section 3.1, Eq. (6), writes the affinities with
projections W_Q, W_K in R^{d x d}:
    Z = (P W_Q)(X W_K)^T / sqrt(d).
Since (P W_Q)(X W_K)^T = (P W_Q W_K^T) X^T, the folded table
    P_eff = P W_Q W_K^T                  (k x d)
turns the projected affinities into the kernel's Z = P_eff X^T / sqrt(d); the
aggregation of Eq. (9) still sums the unprojected X.

Backward of the fold, with M = W_Q W_K^T and G = dL/dP_eff:
    dP = G M^T,   dM = P^T G,   dW_Q = dM W_K,   dW_K = dM^T W_Q.

Pins (tests/test_oracle_projections.py): identity weights give P_eff = P; the
folded forward equals a scalar-loop evaluation of Eq. (6) in its unfolded form
with non-symmetric weights; central finite differences for the fold's
backward, alone and chained through the sketch's backward.
"""

from __future__ import annotations

import math

import numpy as np


def fold_prototypes_ref(P, Wq, Wk):
    """P_eff = P W_Q W_K^T (Eq. (6) regrouped), float64."""
    P = np.asarray(P, dtype=np.float64)
    Wq = np.asarray(Wq, dtype=np.float64)
    Wk = np.asarray(Wk, dtype=np.float64)
    return (P @ Wq) @ Wk.T


def fold_prototypes_backward_ref(P, Wq, Wk, dPeff):
    """Gradients (dP, dW_Q, dW_K) of a loss L given G = dL/dP_eff, where
    P_eff = P W_Q W_K^T."""
    P = np.asarray(P, dtype=np.float64)
    Wq = np.asarray(Wq, dtype=np.float64)
    Wk = np.asarray(Wk, dtype=np.float64)
    G = np.asarray(dPeff, dtype=np.float64)
    M = Wq @ Wk.T
    dM = P.T @ G
    return G @ M.T, dM @ Wk, dM.T @ Wq


def projected_forward_brute(offsets, X, P, Wq, Wk):
    """Eq. (6)-(9) with the projections applied as printed, by scalar loops:
    q_j = p_j W_Q, k_i = x_i W_K, z_ji = q_j . k_i / sqrt(d), softmax over j,
    S_j = sum_i A_ji x_i.  For tiny inputs only."""
    X = np.asarray(X, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    Wq = np.asarray(Wq, dtype=np.float64)
    Wk = np.asarray(Wk, dtype=np.float64)
    k, d = P.shape
    B = len(offsets) - 1
    c = 1.0 / math.sqrt(d)
    q = [[math.fsum(P[j, a] * Wq[a, b] for a in range(d)) for b in range(d)] for j in range(k)]
    S = np.zeros((B, k, d))
    for u in range(B):
        rows = range(int(offsets[u]), int(offsets[u + 1]))
        for i in rows:
            kv = [math.fsum(X[i, a] * Wk[a, b] for a in range(d)) for b in range(d)]
            z = [c * math.fsum(q[j][b] * kv[b] for b in range(d)) for j in range(k)]
            m = max(z)
            e = [math.exp(v - m) for v in z]
            tot = math.fsum(e)
            for j in range(k):
                for b in range(d):
                    S[u, j, b] += e[j] / tot * X[i, b]
    return S
