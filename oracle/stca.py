"""float64 oracle for the reordered single-query STCA attention.

TEST INFRASTRUCTURE: only tests, the build entry module's smoke check and the
benchmark's CPU-baseline leg may use this module.  It imports nothing from the
product package and shares no code with the HIP library.

SequenceO1 reading notes, section 5.1 (single-query reordering of STCA),
Eq. (24)-(25): STCA has one query per layer (the target), so per head
    u     = (q W_Q) W_K^T              in R^{1 x D}
    alpha = softmax(u X^T / sqrt(d_h)) in R^{1 x L}
    o     = (alpha X) W_V
which never forms X W_K or X W_V over the L history rows: the length-
dependent work is the two reductions u X^T and alpha X, 4 L D per head.

Readings: h heads of width d_h = D / h; head j uses columns
j d_h .. (j+1) d_h - 1 of W_Q, W_K, W_V (D x D), so u_j = (q W_Q[:, j]) W_K[:, j]^T
and o_j = (alpha_j X) W_V[:, j]; the heads' outputs are concatenated (the
output projection W_O and the FFN that follow are outside the attention).
Each target attends over its own user's rows (a ragged batch: targets are
grouped by user); a user without rows gives o = 0.

The whole layer of Eq. (26) adds the output projection W_O (2 D^2 per
target) and the query-side SwiGLU FFN (12 D^2 per target: Eq. (23) with
hidden width w_f = 2 D).  The page counts their flops only; it prints no
residual connections or normalisation.  Reading taken (stca_layer_ref): the
two sublayers are residual, as in a standard transformer layer, with no
normalisation (the page lists none; its FLOP convention leaves out layer
norms anyway):
    a = q + o W_O,        y = a + (silu(a W1) * (a W3)) W2,
W_O: D x D, W1, W3: D x 2D, W2: 2D x D, no biases.

Pins: tests/test_oracle_stca.py (the unreordered form with X W_K and X W_V
materialised, closed forms, finite properties; for the layer, torch's
scaled_dot_product_attention and silu on the unreordered form, W2 = 0 and
W_O = 0 special cases).
"""

from __future__ import annotations

import math

import numpy as np


def stca_attention_ref(x_off, X, t_off, Q, Wq, Wk, Wv, h):
    """x_off [B+1] rows of X per user; t_off [B+1] targets (rows of Q) per
    user.  X [L_total, D], Q [R, D], Wq, Wk, Wv [D, D].  Returns (o [R, D],
    lse [R, h]) with lse the log-sum-exp of the scaled scores (natural log;
    -inf for a user without rows)."""
    X = np.asarray(X, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    Wq, Wk, Wv = (np.asarray(w, dtype=np.float64) for w in (Wq, Wk, Wv))
    R, D = Q.shape
    dh = D // h
    o = np.zeros((R, D))
    lse = np.full((R, h), -np.inf)
    B = len(x_off) - 1
    for u in range(B):
        Xu = X[int(x_off[u]):int(x_off[u + 1])]
        for r in range(int(t_off[u]), int(t_off[u + 1])):
            if Xu.shape[0] == 0:
                continue
            for j in range(h):
                cols = slice(j * dh, (j + 1) * dh)
                uj = (Q[r] @ Wq[:, cols]) @ Wk[:, cols].T          # Eq. (24), reordered
                s = (Xu @ uj) / math.sqrt(dh)
                m = s.max()
                a = np.exp(s - m)
                lse[r, j] = m + math.log(a.sum())
                a /= a.sum()
                o[r, cols] = (a @ Xu) @ Wv[:, cols]
    return o, lse


def stca_attention_unreordered(x_off, X, t_off, Q, Wq, Wk, Wv, h):
    """The standard form: K = X W_K and V = X W_V materialised per head."""
    X = np.asarray(X, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    R, D = Q.shape
    dh = D // h
    o = np.zeros((R, D))
    for u in range(len(x_off) - 1):
        Xu = X[int(x_off[u]):int(x_off[u + 1])]
        if Xu.shape[0] == 0:
            continue
        for r in range(int(t_off[u]), int(t_off[u + 1])):
            for j in range(h):
                cols = slice(j * dh, (j + 1) * dh)
                K = Xu @ Wk[:, cols]
                V = Xu @ Wv[:, cols]
                s = K @ (Q[r] @ Wq[:, cols]) / math.sqrt(dh)
                a = np.exp(s - s.max())
                o[r, cols] = (a / a.sum()) @ V
    return o


def _silu(x):
    return x / (1.0 + np.exp(-x))


def stca_layer_ref(x_off, X, t_off, Q, Wq, Wk, Wv, Wo, W1, W3, W2, h):
    """One STCA layer for every target (reading notes section 5.1, Eq. (26)):
    the reordered attention of stca_attention_ref, then the output projection
    and the query-side SwiGLU FFN, each as a residual sublayer.  Returns
    (y [R, D], o [R, D], lse [R, h])."""
    o, lse = stca_attention_ref(x_off, X, t_off, Q, Wq, Wk, Wv, h)
    Q = np.asarray(Q, dtype=np.float64)
    Wo, W1, W3, W2 = (np.asarray(w, dtype=np.float64) for w in (Wo, W1, W3, W2))
    a = Q + o @ Wo
    y = a + (_silu(a @ W1) * (a @ W3)) @ W2
    return y, o, lse
