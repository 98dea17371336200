"""Pure-Python scalar Sketch Attention for tiny inputs — TEST INFRASTRUCTURE.

Every sum is an exactly-rounded math.fsum and every value is a Python float, so
this shares no arithmetic with numpy's BLAS path in sa_ref.  Use it for n <= 16,
k <= 8, d <= 4; it is O(B n k d) Python operations.

Follows the SequenceO1 reading notes, section 3.1: Eq. (6) affinities with the
1/sqrt(d) scale, Eq. (8) softmax over the prototype index j for each token i,
Eq. (9) aggregation over tokens; plus the per-prototype mass and the
mass-normalised (weighted-mean) sketch.
"""

from __future__ import annotations

import math


def _tables(P, B):
    """One table per user: P is k rows (shared by all users) or B tables of k
    rows (user u uses P[u])."""
    if isinstance(P[0][0], (list, tuple)):
        if len(P) != B:
            raise ValueError("need one table per user")
        return [[[float(v) for v in row] for row in tab] for tab in P]
    shared = [[float(v) for v in row] for row in P]
    return [shared] * B


def brute_forward(offsets, X, P, mass_norm=False):
    """offsets: list of ints (B+1); X: list of T rows (lists of d floats);
    P: list of k rows, or a list of B such tables (one per user).
    Returns (S [B][k][d], lse [T], mass [B][k])."""
    X = [[float(v) for v in row] for row in X]
    B = len(offsets) - 1
    tables = _tables(P, B)
    k = len(tables[0])
    d = len(tables[0][0])
    c = 1.0 / math.sqrt(d)
    S = [[[0.0] * d for _ in range(k)] for _ in range(B)]
    mass = [[0.0] * k for _ in range(B)]
    lse = [0.0] * len(X)
    for u in range(B):
        P = tables[u]
        toks = list(range(offsets[u], offsets[u + 1]))
        # A[j][t] for the tokens of this user
        A = {}
        for i in toks:
            z = [c * math.fsum(P[j][e] * X[i][e] for e in range(d)) for j in range(k)]
            m = max(z)
            ex = [math.exp(zj - m) for zj in z]
            den = math.fsum(ex)
            lse[i] = m + math.log(den)
            for j in range(k):
                A[(j, i)] = ex[j] / den
        for j in range(k):
            mu = math.fsum(A[(j, i)] for i in toks)
            mass[u][j] = mu
            for e in range(d):
                v = math.fsum(A[(j, i)] * X[i][e] for i in toks)
                if mass_norm:
                    v = v / mu if mu > 0 else 0.0
                S[u][j][e] = v
    return S, lse, mass


def brute_loss(offsets, X, P, dS, mass_norm=False):
    """L = sum_{u,j,e} dS[u][j][e] * S[u][j][e], the scalar whose gradient the
    backward computes; used with finite differences."""
    S, _, _ = brute_forward(offsets, X, P, mass_norm)
    terms = []
    for u in range(len(S)):
        for j in range(len(S[u])):
            for e in range(len(S[u][j])):
                terms.append(dS[u][j][e] * S[u][j][e])
    return math.fsum(terms)


def hard_assignment_sketch(offsets, X, P):
    """The hard limit of the prototype-wise softmax (the EM analogy of the
    reading notes, section 3.3 / appendix E: soft assignment as a
    responsibility): every token goes to its arg-max prototype, and S[j] is the
    plain sum of the tokens assigned to j.  Ties are not resolved: callers use
    well-separated logits."""
    X = [[float(v) for v in row] for row in X]
    P = [[float(v) for v in row] for row in P]
    k = len(P)
    d = len(P[0])
    B = len(offsets) - 1
    S = [[[0.0] * d for _ in range(k)] for _ in range(B)]
    for u in range(B):
        members = [[] for _ in range(k)]
        for i in range(offsets[u], offsets[u + 1]):
            z = [math.fsum(P[j][e] * X[i][e] for e in range(d)) for j in range(k)]
            members[max(range(k), key=lambda j: z[j])].append(i)
        for j in range(k):
            for e in range(d):
                S[u][j][e] = math.fsum(X[i][e] for i in members[j])
    return S
