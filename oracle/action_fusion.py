"""float64 oracle for the action-side SwiGLU fusion that builds the history
rows.

TEST INFRASTRUCTURE: only tests, the build entry module's smoke check and the
benchmark's CPU-baseline leg may use this module.  It imports nothing from the
product package and shares no code with the HIP library.

SequenceO1 reading notes, section 3.6 (appendix D), Eq. (20): each history
event has an item embedding e_i and an action-type embedding a_i, and the row
the sketch consumes is
    x_i = e_i + FFN_SwiGLU([e_i; a_i])
where the FFN maps the concatenation back to e_i's width.  Readings where the
page is silent: e_i, a_i in R^d (a_i is row t_i of an action table A with
one row per action type); FFN_SwiGLU(v) = (silu(v W1) * (v W3)) W2 with
W1, W3 in R^{2d x 2d} and W2 in R^{2d x d}; no biases.  The hidden width
is a choice, not something the page fixes: Eq. 23's rule (hidden width twice
the FFN's input width) would give 4d for the 2d-wide [e_i; a_i]; 2d, twice the
row width d of e_i, is used instead and is fixed in the library.

Backward (L = sum(dx * x)):  with v = [e; a], U1 = v W1, U3 = v W3,
G = silu(U1) U3, s = logistic(U1):
    dG = dx W2^T,  dW2 = G^T dx
    dU1 = dG U3 s (1 + U1 (1 - s)),  dU3 = dG silu(U1)
    dv = dU1 W1^T + dU3 W3^T,  dW1 = v^T dU1,  dW3 = v^T dU3
    de = dx + dv[:, :d],  dA[t] = sum of dv[i, d:] over the events of type t.

Pins: tests/test_oracle_action_fusion.py.
"""

from __future__ import annotations

import numpy as np


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def _silu(u):
    return u / (1.0 + np.exp(-u))


def action_fusion_ref(e, types, A, W1, W3, W2):
    """Returns x [T, d] (float64)."""
    e = _as64(e)
    v = np.concatenate([e, _as64(A)[np.asarray(types, dtype=np.int64)]], axis=1)
    return e + (_silu(v @ _as64(W1)) * (v @ _as64(W3))) @ _as64(W2)


def action_fusion_backward_ref(e, types, A, W1, W3, W2, dx):
    """Gradients (de, dA, dW1, dW3, dW2) of L = sum(dx * x)."""
    e = _as64(e)
    A = _as64(A)
    W1, W3, W2 = _as64(W1), _as64(W3), _as64(W2)
    dx = _as64(dx)
    t = np.asarray(types, dtype=np.int64)
    d = e.shape[1]
    v = np.concatenate([e, A[t]], axis=1)
    U1, U3 = v @ W1, v @ W3
    s = 1.0 / (1.0 + np.exp(-U1))
    G = U1 * s * U3
    dG = dx @ W2.T
    dW2 = G.T @ dx
    dU1 = dG * U3 * s * (1.0 + U1 * (1.0 - s))
    dU3 = dG * U1 * s
    dv = dU1 @ W1.T + dU3 @ W3.T
    dA = np.zeros_like(A)
    np.add.at(dA, t, dv[:, d:])
    return dx + dv[:, :d], dA, v.T @ dU1, v.T @ dU3, dW2
