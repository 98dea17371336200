"""Pins for the float64 oracle of the reordered single-query STCA attention
(SequenceO1 reading notes, section 5.1, Eq. (24)-(25)).  No GPU."""

import math

import numpy as np

from oracle.stca import stca_attention_ref, stca_attention_unreordered


def _case(seed, x_lens, t_lens, D=8, h=2):
    rng = np.random.default_rng(seed)
    x_off = np.concatenate([[0], np.cumsum(x_lens)]).astype(np.int64)
    t_off = np.concatenate([[0], np.cumsum(t_lens)]).astype(np.int64)
    X = rng.standard_normal((int(x_off[-1]), D))
    Q = rng.standard_normal((int(t_off[-1]), D))
    W = [rng.standard_normal((D, D)) * 0.5 for _ in range(3)]
    return x_off, X, t_off, Q, W


def test_reordering_equals_the_standard_form():
    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(0, [5, 0, 7], [2, 1, 3])
    o, _ = stca_attention_ref(x_off, X, t_off, Q, Wq, Wk, Wv, 2)
    assert np.max(np.abs(o - stca_attention_unreordered(x_off, X, t_off, Q, Wq, Wk, Wv, 2))) < 1e-12


def test_closed_forms():
    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(1, [1, 4], [2, 1], D=4, h=2)
    o, lse = stca_attention_ref(x_off, X, t_off, Q, Wq, Wk, Wv, 2)
    # one history row: every head attends to it with weight 1
    for r in range(2):
        for j in range(2):
            cols = slice(2 * j, 2 * j + 2)
            assert np.allclose(o[r, cols], X[0] @ Wv[:, cols], atol=1e-13)
    # W_Q = 0: uniform weights, o = mean row times W_V; lse = log n
    o0, lse0 = stca_attention_ref(x_off, X, t_off, Q, np.zeros((4, 4)), Wk, Wv, 2)
    assert np.allclose(o0[2], X[1:5].mean(axis=0) @ Wv, atol=1e-13)
    assert np.allclose(lse0[2], math.log(4), atol=1e-14)
    # a user without rows
    x_off2 = np.array([0, 0, 5])
    o2, lse2 = stca_attention_ref(x_off2, X, t_off, Q, Wq, Wk, Wv, 2)
    assert np.array_equal(o2[:2], np.zeros((2, 4))) and np.all(np.isneginf(lse2[:2]))


def test_history_row_order_does_not_matter():
    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(2, [6], [3])
    perm = np.random.default_rng(3).permutation(6)
    a, la = stca_attention_ref(x_off, X, t_off, Q, Wq, Wk, Wv, 2)
    b, lb = stca_attention_ref(x_off, X[perm], t_off, Q, Wq, Wk, Wv, 2)
    assert np.allclose(a, b, atol=1e-13) and np.allclose(la, lb, atol=1e-13)
