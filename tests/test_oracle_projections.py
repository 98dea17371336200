"""Pins for the float64 oracle of the folded query/key projections (no GPU).

SequenceO1 reading notes, section 3.1, Eq. (6): Z = (P W_Q)(X W_K)^T / sqrt(d).
The oracle folds the projections into the prototype table; these tests pin
the fold against the unfolded form evaluated by scalar loops, against identity
weights, and its backward against central finite differences.
"""

import numpy as np
import pytest

from oracle.brute import brute_loss
from oracle.projections import (fold_prototypes_backward_ref, fold_prototypes_ref,
                                projected_forward_brute)
from oracle.sa_ref import sa_backward_ref, sa_forward_ref


def _weights(rng, d):
    # non-symmetric, so a transposed weight anywhere changes the result
    return rng.standard_normal((d, d)) * 0.7, rng.standard_normal((d, d)) * 0.7


def test_identity_weights_leave_prototypes():
    rng = np.random.default_rng(0)
    P = rng.standard_normal((5, 4))
    I = np.eye(4)
    assert np.array_equal(fold_prototypes_ref(P, I, I), P)


def test_fold_is_not_symmetric_in_the_weights():
    # the two weights enter on different sides: swapping them changes P_eff
    rng = np.random.default_rng(1)
    P = rng.standard_normal((3, 4))
    Wq, Wk = _weights(rng, 4)
    assert not np.allclose(fold_prototypes_ref(P, Wq, Wk), fold_prototypes_ref(P, Wk, Wq))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_folded_forward_matches_unfolded_eq6(seed):
    rng = np.random.default_rng(seed)
    k, d = 3, 4
    lengths = [3, 0, 5]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    X = rng.standard_normal((int(off[-1]), d))
    P = rng.standard_normal((k, d))
    Wq, Wk = _weights(rng, d)
    S_fold, _, _ = sa_forward_ref(off, X, fold_prototypes_ref(P, Wq, Wk))
    S_loop = projected_forward_brute(off.tolist(), X, P, Wq, Wk)
    assert np.max(np.abs(S_fold - S_loop)) < 1e-12


@pytest.mark.parametrize("seed", [0, 1])
def test_fold_backward_finite_differences(seed):
    rng = np.random.default_rng(seed)
    k, d = 3, 4
    P = rng.standard_normal((k, d))
    Wq, Wk = _weights(rng, d)
    G = rng.standard_normal((k, d))
    dP, dWq, dWk = fold_prototypes_backward_ref(P, Wq, Wk, G)

    def loss(P_, Wq_, Wk_):
        return float(np.sum(G * fold_prototypes_ref(P_, Wq_, Wk_)))

    h = 1e-6
    for arr, grad, which in ((P, dP, 0), (Wq, dWq, 1), (Wk, dWk, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args_p = [P.copy(), Wq.copy(), Wk.copy()]
            args_m = [P.copy(), Wq.copy(), Wk.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.max(np.abs(num - grad)) < 1e-7


@pytest.mark.parametrize("mass_norm", [False, True])
def test_chained_backward_finite_differences(mass_norm):
    # dL/dW through the sketch: sa_backward_ref gives dL/dP_eff, the fold's
    # backward carries it to (P, W_Q, W_K).  Checked against central
    # differences of the brute-force loss of the folded forward.
    rng = np.random.default_rng(3)
    k, d = 3, 2
    lengths = [2, 3]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    X = rng.standard_normal((int(off[-1]), d))
    P = rng.standard_normal((k, d))
    Wq, Wk = _weights(rng, d)
    dS = rng.standard_normal((len(lengths), k, d))
    _, dPeff = sa_backward_ref(off, X, fold_prototypes_ref(P, Wq, Wk), dS, mass_norm)
    dP, dWq, dWk = fold_prototypes_backward_ref(P, Wq, Wk, dPeff)

    def loss(P_, Wq_, Wk_):
        return brute_loss(off.tolist(), X.tolist(), fold_prototypes_ref(P_, Wq_, Wk_).tolist(),
                          dS.tolist(), mass_norm)

    h = 1e-6
    for arr, grad, which in ((P, dP, 0), (Wq, dWq, 1), (Wk, dWk, 2)):
        for idx in np.ndindex(arr.shape):
            args_p = [P.copy(), Wq.copy(), Wk.copy()]
            args_m = [P.copy(), Wq.copy(), Wk.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(num - grad[idx]) < 1e-6 * max(1.0, abs(num))
