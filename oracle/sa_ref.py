"""float64 numpy oracle for Sketch Attention forward and backward.

TEST INFRASTRUCTURE: only tests, the build entry module's smoke check and the
benchmark's CPU-baseline leg may use this module.  It imports nothing from the
product package and shares no code with the HIP library.

Notation (SequenceO1 reading notes, section 3.1): X is one user's history,
n x d, rows x_i; P is the prototype table, k x d, rows p_j (Eq. 5), shared by
all users; or, in the refinement layers of section 3.3, Eq. (12)-(14), one
table per user (the user's own sketch, projected, serves as the queries).  The
pages
call the affinity matrix S and the sketch X~; here the affinities are Z and the
sketch is S, matching the C interface.

Forward, one user (reading notes section 3.1):
  Z = P X^T / sqrt(d)                      Eq. (6), with W_Q, W_K folded into P
  A[j, i] = exp Z[j, i] / sum_j' exp Z[j', i]   Eq. (7)-(8): softmax over the k
                                                prototypes, per token
  U = A X                                  Eq. (9): the sketch, k x d
  mu[j] = sum_i A[j, i]                    per-prototype mass
  S = U  (plain sum)  or  S[j] = U[j] / mu[j]  (mass normalisation; mu = 0
                                             gives a zero row)
and the per-token statistic lse[i] = log sum_j exp Z[j, i] that the FlashSA
paragraph of the paper's HTML page names (max and log-sum-exp).

The mass normalisation is not printed on the pages; it is read as the weighted
mean of the tokens each prototype receives.  The backward is not printed
either: it is the chain rule through the four lines above, written out in
sa_backward_ref.

Pins (tests/test_oracle_*.py): brute-force scalar loops on tiny inputs, the
column-sum invariant of Eq. (7), closed forms for k = 1, P = 0, n = 1 (scipy
softmax) and d = 1 (logistic), the hard-assignment limit, token / prototype
permutation symmetries, scipy logsumexp for lse, central finite differences
and torch float64 autograd for the backward, and uniform-dS / linearity
identities.
"""

from __future__ import annotations

import numpy as np

# Token chunk for the per-user loops: keeps the k x chunk float64 intermediates
# at or below 128 MiB for k = 1024.
_CHUNK = 16384


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def _check_offsets(offsets, total):
    off = np.asarray(offsets, dtype=np.int64)
    if off.ndim != 1 or off.size < 1 or off[0] != 0 or off[-1] != total:
        raise ValueError("offsets must start at 0 and end at the token count")
    if np.any(np.diff(off) < 0):
        raise ValueError("offsets must be non-decreasing")
    return off


def prototype_softmax(Z):
    """Eq. (7)-(8) of the reading notes: softmax of a k x m affinity block over
    axis 0 (the prototypes), separately for every token column.

    Returns (A, lse) with A of shape k x m and lse[i] = log sum_j exp Z[j, i].
    Shifts each column by its maximum before exponentiating (the numerically
    robust form the FlashSA paragraph asks for).
    """
    Z = _as64(Z)
    m = Z.max(axis=0)
    E = np.exp(Z - m[None, :])
    ell = E.sum(axis=0)
    A = E / ell[None, :]
    lse = m + np.log(ell)
    return A, lse


def affinities(P, Xu):
    """Eq. (6): Z = P Xu^T / sqrt(d) for one block of tokens (k x m)."""
    P = _as64(P)
    Xu = _as64(Xu)
    d = P.shape[1]
    return (P @ Xu.T) / np.sqrt(d)


def _user_tables(P, B):
    """P as one table per user: a shared [k, d] table (reading notes Eq. (5):
    the prototypes are global) is used by every user; a [B, k, d] stack gives
    user u its own table P[u] (the refinement layers of section 3.3,
    Eq. (12)-(14), whose queries are the user's own sketch).  Returns (tables, per_user)."""
    P = _as64(P)
    if P.ndim == 2:
        return [P] * B, False
    if P.ndim == 3 and P.shape[0] == B:
        return [P[u] for u in range(B)], True
    raise ValueError("P must be [k, d] or [B, k, d]")


def sa_forward_ref(offsets, X, P, mass_norm=False):
    """Sketch Attention forward over a CSR-ragged batch.

    offsets : int64 [B+1], offsets[0] = 0, non-decreasing, offsets[B] = T.
    X       : [T, d] histories of all users, concatenated (any float dtype;
              upcast exactly to float64).
    P       : [k, d] prototypes shared by every user, or [B, k, d] with one
              table per user.
    Returns (S [B, k, d], lse [T], mass [B, k]), all float64.
    """
    X = _as64(X)
    T, d = X.shape
    off = _check_offsets(offsets, T)
    B = off.size - 1
    tables, _ = _user_tables(P, B)
    k = tables[0].shape[0]
    S = np.zeros((B, k, d))
    mass = np.zeros((B, k))
    lse = np.zeros(T)
    for u in range(B):
        lo, hi = int(off[u]), int(off[u + 1])
        Pu = tables[u]
        U = np.zeros((k, d))
        mu = np.zeros(k)
        for c0 in range(lo, hi, _CHUNK):
            c1 = min(hi, c0 + _CHUNK)
            Xc = X[c0:c1]
            A, l = prototype_softmax(affinities(Pu, Xc))
            lse[c0:c1] = l
            U += A @ Xc              # Eq. (9)
            mu += A.sum(axis=1)
        mass[u] = mu
        if mass_norm:
            nz = mu > 0
            S[u][nz] = U[nz] / mu[nz, None]
        else:
            S[u] = U
    return S, lse, mass


def sa_backward_ref(offsets, X, P, dS, mass_norm=False):
    """Gradients of L = sum(dS * S) with respect to X and P.

    The chain rule through the forward above, one user at a time:
      plain sum:   G = dS,  c = 0
      mass norm:   G[j] = dS[j] / mu[j],  c[j] = G[j] . S[j]   (mu[j] = 0: the
                   row is a constant zero, so G[j] = 0 and c[j] = 0)
      dA[j, i]   = G[j] . x_i - c[j]           (U and mu both depend on A)
      g_i        = sum_j A[j, i] G[j]          (the direct path of Eq. 9)
      delta_i    = sum_j A[j, i] dA[j, i]      (softmax over prototypes)
      dZ[j, i]   = A[j, i] (dA[j, i] - delta_i)
      dX_i       = g_i + (1/sqrt d) sum_j dZ[j, i] p_j      (Eq. 6)
      dP_u       = (1/sqrt d) sum_i dZ[j, i] x_i over the user's tokens
    A shared table's gradient is the sum of the users' dP_u; a per-user stack
    [B, k, d] gets dP[u] = dP_u.
    Returns (dX [T, d], dP [k, d] or [B, k, d]) in float64.
    """
    X = _as64(X)
    dS = _as64(dS)
    T, d = X.shape
    off = _check_offsets(offsets, T)
    B = off.size - 1
    tables, per_user = _user_tables(P, B)
    k = tables[0].shape[0]
    if dS.shape != (B, k, d):
        raise ValueError("dS must be [B, k, d]")
    S, _, mass = sa_forward_ref(off, X, P, mass_norm)
    scale = 1.0 / np.sqrt(d)
    dX = np.zeros((T, d))
    dP = np.zeros((B, k, d)) if per_user else np.zeros((k, d))
    for u in range(B):
        lo, hi = int(off[u]), int(off[u + 1])
        Pu = tables[u]
        dPu = dP[u] if per_user else dP
        if mass_norm:
            mu = mass[u]
            G = np.zeros((k, d))
            nz = mu > 0
            G[nz] = dS[u][nz] / mu[nz, None]
            cvec = np.einsum("jd,jd->j", G, S[u])
        else:
            G = dS[u]
            cvec = np.zeros(k)
        for c0 in range(lo, hi, _CHUNK):
            c1 = min(hi, c0 + _CHUNK)
            Xc = X[c0:c1]
            A, _ = prototype_softmax(affinities(Pu, Xc))
            dA = G @ Xc.T - cvec[:, None]
            g = A.T @ G
            delta = np.einsum("ji,ji->i", A, dA)
            dZ = A * (dA - delta[None, :])
            dX[c0:c1] = g + scale * (dZ.T @ Pu)
            dPu += scale * (dZ @ Xc)
    return dX, dP


def sa_lse_ref(X, P):
    """Per-token log-sum-exp over the prototypes for a flat token array."""
    X = _as64(X)
    out = np.empty(X.shape[0])
    for c0 in range(0, X.shape[0], _CHUNK):
        c1 = min(X.shape[0], c0 + _CHUNK)
        out[c0:c1] = prototype_softmax(affinities(P, X[c0:c1]))[1]
    return out
