"""float64 oracle for the token-wise normalised sketch (the vanilla-attention
baseline of Table 1).

TEST INFRASTRUCTURE: only tests, the build entry module's smoke check and the
benchmark's CPU-baseline leg may use this module.  It imports nothing from the
product package and shares no code with the HIP library.

SequenceO1 reading notes, section 3.5 (why prototype-wise normalisation,
appendix C) and section 7.1 (SA vs vanilla attention, Table 1): the baseline
normalises the same affinities Z = P X^T / sqrt(d) (Eq. 6) over the tokens
instead of over the prototypes, so that each prototype's weights form a
distribution p(i | j) over the user's history:
    A[j, i] = exp Z[j, i] / sum_i' exp Z[j, i']      (softmax over tokens)
    S[j]    = sum_i A[j, i] x_i                        (a weighted mean)
per user, with the per-prototype statistic lse[j] = log sum_i exp Z[j, i].
Readings: an empty history gives S = 0 and lse = -inf (the empty sum), and
mass normalisation does not apply (each row of A already sums to 1).

Backward (chain rule; G = dS):
    dA[j, i]  = G[j] . x_i
    D[j]      = sum_i A[j, i] dA[j, i] = G[j] . S[j]
    dZ[j, i]  = A[j, i] (dA[j, i] - D[j])
    dX_i      = sum_j A[j, i] G[j] + (1/sqrt d) sum_j dZ[j, i] p_j
    dP_j      = (1/sqrt d) sum_u sum_i dZ[j, i] x_i  (summed over users for a
                                                      shared table)

Pins: tests/test_oracle_tokenwise.py (scalar loops, closed forms for n = 1
and k = 1, token-permutation invariance, finite differences, torch float64
autograd).
"""

from __future__ import annotations

import math

import numpy as np

_CHUNK = 1 << 14


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def tokenwise_forward_ref(offsets, X, P):
    """Returns (S [B, k, d], lse [B, k]) in float64 for a shared table P
    [k, d]."""
    X = _as64(X)
    P = _as64(P)
    k, d = P.shape
    B = len(offsets) - 1
    c = 1.0 / math.sqrt(d)
    S = np.zeros((B, k, d))
    lse = np.full((B, k), -np.inf)
    for u in range(B):
        lo, hi = int(offsets[u]), int(offsets[u + 1])
        if hi == lo:
            continue
        Z = (P @ X[lo:hi].T) * c                    # k x n
        m = Z.max(axis=1, keepdims=True)
        E = np.exp(Z - m)
        s = E.sum(axis=1, keepdims=True)
        S[u] = (E / s) @ X[lo:hi]
        lse[u] = (m + np.log(s))[:, 0]
    return S, lse


def tokenwise_backward_ref(offsets, X, P, dS):
    """Gradients (dX [T, d], dP [k, d]) of L = sum(dS * S), float64."""
    X = _as64(X)
    P = _as64(P)
    dS = _as64(dS)
    k, d = P.shape
    B = len(offsets) - 1
    c = 1.0 / math.sqrt(d)
    dX = np.zeros_like(X)
    dP = np.zeros_like(P)
    for u in range(B):
        lo, hi = int(offsets[u]), int(offsets[u + 1])
        if hi == lo:
            continue
        Xu = X[lo:hi]
        Z = (P @ Xu.T) * c
        A = np.exp(Z - Z.max(axis=1, keepdims=True))
        A /= A.sum(axis=1, keepdims=True)
        G = dS[u]
        dA = G @ Xu.T                               # k x n
        D = np.einsum("jd,jd->j", G, A @ Xu)        # G_j . S_j
        dZ = A * (dA - D[:, None])
        dX[lo:hi] = A.T @ G + c * (dZ.T @ P)
        dP += c * (dZ @ Xu)
    return dX, dP


def tokenwise_forward_brute(offsets, X, P):
    """Scalar loops with math.fsum, for tiny inputs."""
    X = [[float(v) for v in row] for row in X]
    P = [[float(v) for v in row] for row in P]
    k, d = len(P), len(P[0])
    B = len(offsets) - 1
    S = [[[0.0] * d for _ in range(k)] for _ in range(B)]
    lse = [[-math.inf] * k for _ in range(B)]
    for u in range(B):
        toks = list(range(offsets[u], offsets[u + 1]))
        if not toks:
            continue
        for j in range(k):
            z = [math.fsum(P[j][e] * X[i][e] for e in range(d)) / math.sqrt(d) for i in toks]
            m = max(z)
            ex = [math.exp(v - m) for v in z]
            den = math.fsum(ex)
            lse[u][j] = m + math.log(den)
            for e in range(d):
                S[u][j][e] = math.fsum(ex[t] / den * X[i][e] for t, i in enumerate(toks))
    return np.array(S), np.array(lse)
