"""Pins for the oracle with one prototype table per user (no GPU).

SequenceO1 reading notes, section 3.3 (stacked refinement), Eq. (12)-(14): in
the refinement layers the queries of the sketch attention are the user's own
sketch, so each user has its own k x d table.  The oracle takes P as [B, k, d] then, and the
gradient dP[u] is user u's alone.  Pinned against the pure-Python scalar
loops (brute.py) and central finite differences of their loss.
"""

import numpy as np
import pytest

from oracle.brute import brute_forward, brute_loss
from oracle.sa_ref import sa_backward_ref, sa_forward_ref


def _case(seed, lengths, k=3, d=2):
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    X = rng.standard_normal((int(off[-1]), d))
    P = rng.standard_normal((len(lengths), k, d)) * 1.3
    return off, X, P


@pytest.mark.parametrize("mass_norm", [False, True])
def test_forward_matches_scalar_loops(mass_norm):
    off, X, P = _case(0, [3, 0, 4, 1])
    S, lse, mass = sa_forward_ref(off, X, P, mass_norm)
    Sb, lseb, massb = brute_forward(off.tolist(), X.tolist(), P.tolist(), mass_norm)
    assert np.max(np.abs(S - np.array(Sb))) < 1e-12
    assert np.max(np.abs(lse - np.array(lseb))) < 1e-12
    assert np.max(np.abs(mass - np.array(massb))) < 1e-12


def test_each_user_sees_only_its_table():
    off, X, P = _case(1, [2, 3, 2])
    S, lse, _ = sa_forward_ref(off, X, P)
    P2 = P.copy()
    # (adding one vector to every row of a table would shift all of a token's
    # affinities equally and change nothing: perturb the rows differently)
    P2[1] += np.random.default_rng(9).standard_normal(P[1].shape)
    S2, lse2, _ = sa_forward_ref(off, X, P2)
    assert np.array_equal(S[0], S2[0]) and np.array_equal(S[2], S2[2])
    assert not np.allclose(S[1], S2[1])
    assert np.array_equal(lse[:2], lse2[:2]) and np.array_equal(lse[5:], lse2[5:])


def test_one_prototype_gives_user_sums():
    # k = 1: every weight is 1, whatever the table, so S[u] is the sum of the
    # user's rows and no gradient reaches the tables.
    off, X, P = _case(2, [2, 0, 3], k=1)
    S, _, mass = sa_forward_ref(off, X, P)
    for u in range(3):
        lo, hi = off[u], off[u + 1]
        assert np.allclose(S[u, 0], X[lo:hi].sum(axis=0), atol=1e-14)
        assert mass[u, 0] == hi - lo
    dS = np.ones((3, 1, 2))
    _, dP = sa_backward_ref(off, X, P, dS)
    assert dP.shape == (3, 1, 2) and np.max(np.abs(dP)) < 1e-14


def test_identical_tables_reduce_to_the_shared_table():
    off, X, P = _case(3, [3, 2, 4])
    shared = P[0]
    stack = np.stack([shared] * 3)
    S1, lse1, m1 = sa_forward_ref(off, X, shared)
    S2, lse2, m2 = sa_forward_ref(off, X, stack)
    assert np.array_equal(S1, S2) and np.array_equal(lse1, lse2) and np.array_equal(m1, m2)


@pytest.mark.parametrize("mass_norm", [False, True])
def test_backward_finite_differences(mass_norm):
    off, X, P = _case(4, [2, 0, 3], k=3, d=2)
    rng = np.random.default_rng(5)
    dS = rng.standard_normal((3, 3, 2))
    dX, dP = sa_backward_ref(off, X, P, dS, mass_norm)
    assert dP.shape == P.shape

    def loss(X_, P_):
        return brute_loss(off.tolist(), X_.tolist(), P_.tolist(), dS.tolist(), mass_norm)

    h = 1e-6
    for idx in np.ndindex(P.shape):
        Pp, Pm = P.copy(), P.copy()
        Pp[idx] += h
        Pm[idx] -= h
        num = (loss(X, Pp) - loss(X, Pm)) / (2 * h)
        assert abs(num - dP[idx]) < 1e-6 * max(1.0, abs(num)), idx
    for idx in np.ndindex(X.shape):
        Xp, Xm = X.copy(), X.copy()
        Xp[idx] += h
        Xm[idx] -= h
        num = (loss(Xp, P) - loss(Xm, P)) / (2 * h)
        assert abs(num - dX[idx]) < 1e-6 * max(1.0, abs(num)), idx
    # the empty user's table gets no gradient
    assert np.array_equal(dP[1], np.zeros((3, 2)))
