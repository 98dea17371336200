"""Pins for the float64 forward oracle (no GPU).

Each test checks the oracle against something other than itself: pure-Python
brute force, closed forms, scipy routines, or invariants that the SequenceO1
reading notes (section 3.1, Eq. (6)-(9)) fix.
"""

import math

import numpy as np
import pytest
from scipy.special import expit, logsumexp, softmax

from oracle.brute import brute_forward, hard_assignment_sketch
from oracle.sa_ref import prototype_softmax, sa_forward_ref, sa_lse_ref, affinities


def _rand_problem(rng, lengths, k, d, p_std=None):
    T = int(sum(lengths))
    X = rng.standard_normal((T, d))
    P = rng.standard_normal((k, d)) * (p_std if p_std is not None else 1.0)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return off, X, P


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("mass_norm", [False, True])
def test_matches_brute_force(seed, mass_norm):
    rng = np.random.default_rng(seed)
    B = 1 + seed % 3
    lengths = rng.integers(0, 9, size=B)
    lengths[0] = max(lengths[0], 1)
    k = int(rng.integers(1, 8))
    d = int(rng.integers(1, 5))
    off, X, P = _rand_problem(rng, lengths, k, d, p_std=1.5)
    S, lse, mass = sa_forward_ref(off, X, P, mass_norm)
    Sb, lseb, massb = brute_forward(off.tolist(), X.tolist(), P.tolist(), mass_norm)
    np.testing.assert_allclose(S, np.array(Sb).reshape(S.shape), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mass, np.array(massb).reshape(mass.shape), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lseb), rtol=1e-12, atol=1e-12)


def test_empty_user_in_middle_is_zero():
    rng = np.random.default_rng(1)
    off, X, P = _rand_problem(rng, [5, 0, 3], 4, 3)
    for mn in (False, True):
        S, _, mass = sa_forward_ref(off, X, P, mn)
        assert np.all(S[1] == 0) and np.all(mass[1] == 0)
        S0, _, _ = sa_forward_ref(np.array([0, 5]), X[:5], P, mn)
        np.testing.assert_array_equal(S[0], S0[0])


def test_column_sums_are_one():
    # Eq. (7): sum_j A[j, i] = 1 for every token, also for sharp logits.
    rng = np.random.default_rng(2)
    X = rng.standard_normal((300, 16))
    for scale in (0.1, 1.0, 30.0):
        P = rng.standard_normal((37, 16)) * scale
        A, _ = prototype_softmax(affinities(P, X))
        assert A.shape == (37, 300)
        np.testing.assert_allclose(A.sum(axis=0), 1.0, rtol=0, atol=1e-14)
        assert np.all(A >= 0)


def test_softmax_axis_is_prototypes_not_tokens():
    # A token-wise softmax (over axis 1) would make rows sum to one instead.
    rng = np.random.default_rng(3)
    X = rng.standard_normal((7, 4))
    P = rng.standard_normal((5, 4))
    A, _ = prototype_softmax(affinities(P, X))
    ref = softmax(P @ X.T / 2.0, axis=0)
    np.testing.assert_allclose(A, ref, rtol=1e-13, atol=1e-15)
    assert not np.allclose(A.sum(axis=1), 1.0)


def test_lse_matches_scipy_logsumexp():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((50, 8))
    P = rng.standard_normal((9, 8)) * 20.0
    ref = logsumexp(P @ X.T / math.sqrt(8), axis=0)
    np.testing.assert_allclose(sa_lse_ref(X, P), ref, rtol=1e-13, atol=1e-12)
    _, lse, _ = sa_forward_ref(np.array([0, 20, 50]), X, P)
    np.testing.assert_allclose(lse, ref, rtol=1e-13, atol=1e-12)


def test_sum_over_prototypes_equals_sum_of_tokens():
    # Plain sum: sum_j S_j = sum_j sum_i A_ji x_i = sum_i x_i (Eq. 7 + Eq. 9);
    # and the masses add up to the token count.
    rng = np.random.default_rng(5)
    off, X, P = _rand_problem(rng, [400, 1, 77], 33, 12, p_std=0.7)
    S, _, mass = sa_forward_ref(off, X, P)
    for u in range(3):
        xs = X[off[u]:off[u + 1]]
        np.testing.assert_allclose(S[u].sum(axis=0), xs.sum(axis=0), rtol=1e-12, atol=1e-11)
        np.testing.assert_allclose(mass[u].sum(), xs.shape[0], rtol=1e-13)


def test_k1_is_plain_sum_or_mean():
    rng = np.random.default_rng(6)
    off, X, P = _rand_problem(rng, [10, 25], 1, 6)
    S, _, mass = sa_forward_ref(off, X, P, False)
    Sm, _, _ = sa_forward_ref(off, X, P, True)
    for u in range(2):
        xs = X[off[u]:off[u + 1]]
        np.testing.assert_allclose(S[u, 0], xs.sum(axis=0), rtol=1e-13, atol=1e-12)
        np.testing.assert_allclose(Sm[u, 0], xs.mean(axis=0), rtol=1e-13, atol=1e-13)
        assert mass[u, 0] == pytest.approx(xs.shape[0], rel=1e-15)


def test_zero_prototypes_split_evenly():
    rng = np.random.default_rng(7)
    off, X, _ = _rand_problem(rng, [13], 5, 3)
    P = np.zeros((5, 3))
    S, lse, mass = sa_forward_ref(off, X, P)
    np.testing.assert_allclose(S[0], np.tile(X.sum(axis=0) / 5, (5, 1)), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(mass[0], 13 / 5, rtol=1e-14)
    np.testing.assert_allclose(lse, math.log(5), rtol=1e-15)
    Sm, _, _ = sa_forward_ref(off, X, P, True)
    np.testing.assert_allclose(Sm[0], np.tile(X.mean(axis=0), (5, 1)), rtol=1e-13, atol=1e-13)


def test_single_token_is_scipy_softmax_times_x():
    rng = np.random.default_rng(8)
    d = 7
    x = rng.standard_normal(d)
    P = rng.standard_normal((11, d)) * 3
    S, _, mass = sa_forward_ref(np.array([0, 1]), x[None, :], P)
    w = softmax(P @ x / math.sqrt(d))
    np.testing.assert_allclose(S[0], np.outer(w, x), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(mass[0], w, rtol=1e-13)


def test_two_prototypes_width_one_closed_form():
    # d = 1, k = 2: A[0, i] = sigmoid((p0 - p1) x_i), so
    # S_0 = sum_i sigmoid((p0 - p1) x_i) x_i and S_1 = sum_i x_i - S_0.
    x = np.array([[0.5], [-1.25], [2.0], [0.0]])
    P = np.array([[1.5], [-0.5]])
    S, _, mass = sa_forward_ref(np.array([0, 4]), x, P)
    a0 = expit(2.0 * x[:, 0])
    np.testing.assert_allclose(S[0, 0, 0], np.sum(a0 * x[:, 0]), rtol=1e-14)
    np.testing.assert_allclose(S[0, 1, 0], np.sum((1 - a0) * x[:, 0]), rtol=1e-14)
    np.testing.assert_allclose(mass[0], [a0.sum(), 4 - a0.sum()], rtol=1e-14)


def test_hard_assignment_limit():
    # Very sharp prototypes: the soft sketch becomes the hard clustering sum.
    rng = np.random.default_rng(9)
    k, d = 4, 3
    P = rng.standard_normal((k, d))
    X = rng.standard_normal((40, d))
    Z = P @ X.T
    top2 = np.sort(Z, axis=0)[-2:]
    keep = (top2[1] - top2[0]) > 0.05        # drop near-ties
    X = X[keep]
    off = np.array([0, X.shape[0]])
    S, _, _ = sa_forward_ref(off, X, P * 2e4)
    Sh = np.array(hard_assignment_sketch(off.tolist(), X.tolist(), P.tolist()))
    np.testing.assert_allclose(S, Sh, rtol=0, atol=1e-9)


def test_token_permutation_invariance():
    rng = np.random.default_rng(10)
    off, X, P = _rand_problem(rng, [64], 6, 5)
    perm = rng.permutation(64)
    for mn in (False, True):
        S, lse, _ = sa_forward_ref(off, X, P, mn)
        S2, lse2, _ = sa_forward_ref(off, X[perm], P, mn)
        np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse2, lse[perm], rtol=1e-14)


def test_prototype_permutation_and_duplicates():
    rng = np.random.default_rng(11)
    off, X, P = _rand_problem(rng, [30], 5, 4)
    perm = rng.permutation(5)
    S, _, _ = sa_forward_ref(off, X, P)
    S2, _, _ = sa_forward_ref(off, X, P[perm])
    np.testing.assert_allclose(S2[0], S[0][perm], rtol=1e-12, atol=1e-13)
    Pd = np.vstack([P, P[2:3]])
    Sd, _, _ = sa_forward_ref(off, X, Pd)
    np.testing.assert_allclose(Sd[0, 2], Sd[0, 5], rtol=1e-14, atol=1e-15)


def test_mass_norm_rows_are_weighted_means():
    rng = np.random.default_rng(12)
    off, X, P = _rand_problem(rng, [50], 8, 6, p_std=2.0)
    S, _, mass = sa_forward_ref(off, X, P, True)
    lo, hi = X.min(axis=0), X.max(axis=0)
    assert np.all(S[0] >= lo - 1e-12) and np.all(S[0] <= hi + 1e-12)
    Sp, _, _ = sa_forward_ref(off, X, P, False)
    np.testing.assert_allclose(S[0] * mass[0][:, None], Sp[0], rtol=1e-12, atol=1e-12)


def test_chunking_does_not_change_result():
    # More tokens than one internal chunk.
    rng = np.random.default_rng(13)
    n = 16384 + 37
    X = rng.standard_normal((n, 4))
    P = rng.standard_normal((3, 4))
    S, lse, mass = sa_forward_ref(np.array([0, n]), X, P)
    Z = P @ X.T / 2.0
    A = softmax(Z, axis=0)
    np.testing.assert_allclose(S[0], A @ X, rtol=1e-11, atol=1e-9)
    np.testing.assert_allclose(lse, logsumexp(Z, axis=0), rtol=1e-13)
    np.testing.assert_allclose(mass[0], A.sum(axis=1), rtol=1e-12)


def test_bad_offsets_rejected():
    X = np.zeros((4, 2))
    P = np.zeros((2, 2))
    for off in ([0, 3], [1, 4], [0, 3, 2, 4]):
        with pytest.raises(ValueError):
            sa_forward_ref(np.array(off), X, P)
