"""float64 oracle for the stacked Sketch Attention block (refinement layers).

TEST INFRASTRUCTURE: only tests, the build entry module's smoke check and the
benchmark's CPU-baseline leg may use this module.  It imports nothing from the
product package and shares no code with the HIP library.

SequenceO1 reading notes, section 3.3 (stacked refinement), Eq. (12)-(16).
Starting from the shared prototype table, X~(0) = P(0), each layer l computes
    Z(l)    = (X~(l) W_Q(l)) (X W_K(l))^T / sqrt(d)              Eq. (12)
    A(l)    = softmax over the prototypes of Z(l)                  Eq. (13)
    X^(l+1) = A(l) X                                               Eq. (14)
    X-(l+1) = LN(X~(l) + X^(l+1))                                  Eq. (15)
    X~(l+1) = LN(X-(l+1) + FFN(X-(l+1)))                           Eq. (16)
per user, and the block's output is X~(N) (N = N_sa layers; the pages use 2).

Readings where the pages are silent:
  - FFN is the SwiGLU FFN of hidden width 2d: FFN(x) = (silu(x W1) * (x W3)) W2
    with W1, W3 in R^{d x 2d}, W2 in R^{2d x d}, no biases.  It is the FFN
    the pages use elsewhere (Eq. 20, 27), and its count under the paper's
    convention (Eq. 23: 6 T w w_f with w_f = 2w) is the 12 L_s d^2 "sketch
    FFN" term of Eq. (29).
  - LN is layer normalisation over the d features of a row with a learned
    scale and shift, eps = 1e-5: LN(v) = (v - mean v) / sqrt(var v + eps) * g + b
    (biased variance).
  - The aggregation is the plain sum of Eq. (14); Eq. (12)'s projections are
    applied as the folded table X~ W_Q W_K^T (oracle/projections.py).
Layer 0's queries are the shared table, so its residual X~(0) = P(0) is the
same for every user; later layers' queries are each user's own X~(l).

The backward is the chain rule through these lines, written out in
block_backward_ref; pins in tests/test_oracle_block.py (scalar-loop forward,
layer-norm and SwiGLU identities, finite differences of the whole block, and
torch float64 autograd of an independent torch forward).
"""

from __future__ import annotations

import math

import numpy as np

from oracle.projections import fold_prototypes_backward_ref, fold_prototypes_ref
from oracle.sa_ref import sa_backward_ref, sa_forward_ref

LN_EPS = 1e-5


def _as64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Layer normalisation over the last axis.

def layer_norm_ref(v, g, b, eps=LN_EPS):
    """Returns (y, xhat, rstd): y = xhat * g + b with xhat = (v - mean) rstd,
    rstd = 1 / sqrt(var + eps), biased variance over the last axis."""
    v = _as64(v)
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (v - mu) * rstd
    return xhat * _as64(g) + _as64(b), xhat, rstd


def layer_norm_backward_ref(dy, xhat, rstd, g):
    """Gradients (dv, dg, db) of y = LN(v) given dy, from the saved xhat and
    rstd.  With h = dy * g:  dv = rstd (h - mean(h) - xhat mean(h xhat)),
    dg = sum over rows of dy xhat, db = sum over rows of dy."""
    dy = _as64(dy)
    h = dy * _as64(g)
    dv = rstd * (h - h.mean(axis=-1, keepdims=True)
                 - xhat * (h * xhat).mean(axis=-1, keepdims=True))
    rows = dy.reshape(-1, dy.shape[-1])
    return dv, (rows * xhat.reshape(rows.shape)).sum(axis=0), rows.sum(axis=0)


# ---------------------------------------------------------------------------
# SwiGLU FFN, hidden width 2d.

def silu(u):
    return u / (1.0 + np.exp(-u))


def swiglu_ffn_ref(x, W1, W3, W2):
    """Returns (F, U1, U3): U1 = x W1, U3 = x W3, F = (silu(U1) * U3) W2."""
    x = _as64(x)
    U1 = x @ _as64(W1)
    U3 = x @ _as64(W3)
    return (silu(U1) * U3) @ _as64(W2), U1, U3


def swiglu_ffn_backward_ref(dF, x, U1, U3, W1, W3, W2):
    """Gradients (dx, dW1, dW3, dW2) of F = swiglu_ffn(x) given dF.
    silu'(u) = s (1 + u (1 - s)) with s the logistic function."""
    dF = _as64(dF)
    x = _as64(x)
    s = 1.0 / (1.0 + np.exp(-U1))
    Gm = U1 * s * U3                      # silu(U1) * U3
    dG = dF @ _as64(W2).T
    dW2 = Gm.T @ dF
    dU3 = dG * U1 * s
    dU1 = dG * U3 * s * (1.0 + U1 * (1.0 - s))
    dx = dU1 @ _as64(W1).T + dU3 @ _as64(W3).T
    return dx, x.T @ dU1, x.T @ dU3, dW2


# ---------------------------------------------------------------------------
# The block.

LAYER_KEYS = ("Wq", "Wk", "g1", "b1", "W1", "W3", "W2", "g2", "b2")


def block_forward_ref(offsets, X, P0, layers):
    """offsets [B+1], X [T, d], P0 [k, d] (shared table), layers: list of
    dicts with the LAYER_KEYS arrays (Wq, Wk, W1, W3, W2 and the two layer
    norms' g, b).  Returns (out [B, k, d], saved) where saved holds each
    layer's intermediates for block_backward_ref."""
    X = _as64(X)
    P0 = _as64(P0)
    B = len(offsets) - 1
    k, d = P0.shape
    q = P0                                   # X~(0): [k, d], shared
    saved = []
    for L in layers:
        Peff = fold_prototypes_ref(q.reshape(-1, d), L["Wq"], L["Wk"]).reshape(q.shape)
        Xh, _, _ = sa_forward_ref(offsets, X, Peff)                    # [B, k, d]
        r1 = (q if q.ndim == 3 else q[None, :, :]) + Xh                # Eq. (15)
        xbar, xh1, rs1 = layer_norm_ref(r1, L["g1"], L["b1"])
        F, U1, U3 = swiglu_ffn_ref(xbar.reshape(-1, d), L["W1"], L["W3"], L["W2"])
        r2 = xbar + F.reshape(B, k, d)                                  # Eq. (16)
        out, xh2, rs2 = layer_norm_ref(r2, L["g2"], L["b2"])
        saved.append(dict(q=q, Peff=Peff, xbar=xbar, xh1=xh1, rs1=rs1, U1=U1, U3=U3,
                          xh2=xh2, rs2=rs2))
        q = out
    return q, saved


def block_backward_ref(offsets, X, P0, layers, dout):
    """Gradients of L = sum(dout * out) with respect to X, P0 and every
    layer's parameters: returns (dX [T, d], dP0 [k, d], grads) with grads a
    list of dicts keyed like the layers."""
    X = _as64(X)
    P0 = _as64(P0)
    _, saved = block_forward_ref(offsets, X, P0, layers)
    B = len(offsets) - 1
    k, d = P0.shape
    dX = np.zeros_like(X)
    grads = [None] * len(layers)
    dq = _as64(dout)                                   # dL/dX~(l+1)
    for li in range(len(layers) - 1, -1, -1):
        L, s = layers[li], saved[li]
        # X~(l+1) = LN2(r2), r2 = xbar + F(xbar)
        dr2, dg2, db2 = layer_norm_backward_ref(dq, s["xh2"], s["rs2"], L["g2"])
        dxF, dW1, dW3, dW2 = swiglu_ffn_backward_ref(dr2.reshape(-1, d), s["xbar"].reshape(-1, d),
                                                     s["U1"], s["U3"], L["W1"], L["W3"], L["W2"])
        dxbar = dr2 + dxF.reshape(B, k, d)
        # xbar = LN1(r1), r1 = q + Xh
        dr1, dg1, db1 = layer_norm_backward_ref(dxbar, s["xh1"], s["rs1"], L["g1"])
        # Xh = SA(X, Peff): dS = dr1
        dXl, dPeff = sa_backward_ref(offsets, X, s["Peff"], dr1)
        dX += dXl
        q = s["q"]
        dqf, dWq, dWk = fold_prototypes_backward_ref(q.reshape(-1, d), L["Wq"], L["Wk"],
                                                     dPeff.reshape(-1, d))
        dqf = dqf.reshape(q.shape)
        # the residual: q enters r1 directly (broadcast over users in layer 0)
        dq = dqf + (dr1 if q.ndim == 3 else dr1.sum(axis=0))
        grads[li] = dict(Wq=dWq, Wk=dWk, g1=dg1, b1=db1, W1=dW1, W3=dW3, W2=dW2, g2=dg2, b2=db2)
    return dX, dq, grads


# ---------------------------------------------------------------------------
# Scalar loops for tiny inputs (pins).

def block_forward_brute(offsets, X, P0, layers):
    """The block by pure-Python scalar loops with math.fsum: Eq. (12) with
    the projections applied as printed (q = x~ W_Q, key = x W_K), the softmax
    over prototypes, Eq. (14)-(16) with the readings above.  For d <= 4,
    k <= 4, a handful of tokens."""
    X = [[float(v) for v in row] for row in X]
    P0 = [[float(v) for v in row] for row in P0]
    B = len(offsets) - 1
    k, d = len(P0), len(P0[0])

    def mat(a):
        return [[float(v) for v in row] for row in np.asarray(a, dtype=np.float64)]

    def vec(a):
        return [float(v) for v in np.asarray(a, dtype=np.float64)]

    def ln(v, g, b):
        mu = math.fsum(v) / d
        var = math.fsum((x - mu) ** 2 for x in v) / d
        r = 1.0 / math.sqrt(var + LN_EPS)
        return [(v[e] - mu) * r * g[e] + b[e] for e in range(d)]

    def mv(v, W):   # row vector times matrix
        return [math.fsum(v[a] * W[a][c] for a in range(len(v))) for c in range(len(W[0]))]

    q = [[row[:] for row in P0] for _ in range(B)]
    for L in layers:
        Wq, Wk, W1, W3, W2 = (mat(L[n]) for n in ("Wq", "Wk", "W1", "W3", "W2"))
        g1, b1, g2, b2 = (vec(L[n]) for n in ("g1", "b1", "g2", "b2"))
        new = []
        for u in range(B):
            toks = range(offsets[u], offsets[u + 1])
            qq = [mv(q[u][j], Wq) for j in range(k)]
            Xh = [[0.0] * d for _ in range(k)]
            terms = [[[] for _ in range(d)] for _ in range(k)]
            for i in toks:
                kv = mv(X[i], Wk)
                z = [math.fsum(qq[j][e] * kv[e] for e in range(d)) / math.sqrt(d) for j in range(k)]
                m = max(z)
                ex = [math.exp(v - m) for v in z]
                den = math.fsum(ex)
                for j in range(k):
                    for e in range(d):
                        terms[j][e].append(ex[j] / den * X[i][e])
            for j in range(k):
                Xh[j] = [math.fsum(terms[j][e]) for e in range(d)]
            rows = []
            for j in range(k):
                xbar = ln([q[u][j][e] + Xh[j][e] for e in range(d)], g1, b1)
                u1, u3 = mv(xbar, W1), mv(xbar, W3)
                gm = [u1[c] / (1.0 + math.exp(-u1[c])) * u3[c] for c in range(len(u1))]
                f = mv(gm, W2)
                rows.append(ln([xbar[e] + f[e] for e in range(d)], g2, b2))
            new.append(rows)
        q = new
    return np.array(q)
