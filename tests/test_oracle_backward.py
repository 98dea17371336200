"""Pins for the float64 backward oracle (no GPU).

The pages give no backward formulas (the reading notes, section 3.1, only say
the sketch is fully differentiable), so the oracle's chain rule is pinned by
central finite differences of the brute-force forward, by torch float64
autograd through the plain definition, and by identities that hold exactly.
"""

import math

import numpy as np
import pytest
import torch

from oracle.brute import brute_loss
from oracle.sa_ref import sa_backward_ref, sa_forward_ref


def _prob(seed, lengths, k, d, p_std=1.0):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    X = rng.standard_normal((T, d))
    P = rng.standard_normal((k, d)) * p_std
    dS = rng.standard_normal((len(lengths), k, d))
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return off, X, P, dS


@pytest.mark.parametrize("mass_norm", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_finite_differences(seed, mass_norm):
    off, X, P, dS = _prob(seed, [3, 0, 4], 3, 2, p_std=1.2)
    dX, dP = sa_backward_ref(off, X, P, dS, mass_norm)
    h = 1e-6
    ol = off.tolist()
    dSl = dS.tolist()

    def loss(Xa, Pa):
        return brute_loss(ol, Xa.tolist(), Pa.tolist(), dSl, mass_norm)

    for (i, e) in np.ndindex(*X.shape):
        Xp = X.copy(); Xp[i, e] += h
        Xm = X.copy(); Xm[i, e] -= h
        fd = (loss(Xp, P) - loss(Xm, P)) / (2 * h)
        assert abs(fd - dX[i, e]) <= 1e-6 * max(1.0, abs(fd)), (i, e, fd, dX[i, e])
    for (j, e) in np.ndindex(*P.shape):
        Pp = P.copy(); Pp[j, e] += h
        Pm = P.copy(); Pm[j, e] -= h
        fd = (loss(X, Pp) - loss(X, Pm)) / (2 * h)
        assert abs(fd - dP[j, e]) <= 1e-6 * max(1.0, abs(fd)), (j, e, fd, dP[j, e])


@pytest.mark.parametrize("mass_norm", [False, True])
def test_torch_autograd_of_definition(mass_norm):
    off, X, P, dS = _prob(7, [40, 1, 25], 9, 6, p_std=0.8)
    dX, dP = sa_backward_ref(off, X, P, dS, mass_norm)
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Pt = torch.tensor(P, dtype=torch.float64, requires_grad=True)
    loss = torch.zeros((), dtype=torch.float64)
    for u in range(len(off) - 1):
        xs = Xt[off[u]:off[u + 1]]
        Z = Pt @ xs.T / math.sqrt(X.shape[1])
        A = torch.softmax(Z, dim=0)
        S = A @ xs
        if mass_norm:
            S = S / A.sum(dim=1, keepdim=True)
        loss = loss + (S * torch.tensor(dS[u])).sum()
    loss.backward()
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dP, Pt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_uniform_dS_gives_zero_dP_and_constant_dX():
    # Plain sum: L = sum_j v . S_j = v . sum_i x_i, independent of P.
    off, X, P, _ = _prob(3, [30, 12], 7, 5, p_std=2.0)
    v = np.array([0.5, -1.0, 2.0, 0.25, 3.0])
    dS = np.broadcast_to(v, (2, 7, 5)).copy()
    dX, dP = sa_backward_ref(off, X, P, dS, False)
    np.testing.assert_allclose(dP, 0.0, atol=1e-12)
    np.testing.assert_allclose(dX, np.broadcast_to(v, X.shape), rtol=1e-12, atol=1e-12)


def test_linear_in_dS():
    off, X, P, dS1 = _prob(4, [20], 5, 4)
    dS2 = np.random.default_rng(99).standard_normal(dS1.shape)
    for mn in (False, True):
        a = sa_backward_ref(off, X, P, dS1, mn)
        b = sa_backward_ref(off, X, P, dS2, mn)
        c = sa_backward_ref(off, X, P, 2.0 * dS1 - 0.5 * dS2, mn)
        for t in range(2):
            np.testing.assert_allclose(c[t], 2.0 * a[t] - 0.5 * b[t], rtol=1e-11, atol=1e-12)


def test_directional_derivative_mass_norm_larger_problem():
    # A larger case than the brute-force finite differences can afford: the
    # derivative of L along one random direction of X and of P, by central
    # differences of the numpy forward, equals <grad, direction>.
    off, X, P, dS = _prob(5, [60, 33], 12, 8, p_std=1.5)
    dX, dP = sa_backward_ref(off, X, P, dS, True)
    rng = np.random.default_rng(55)
    vX = rng.standard_normal(X.shape)
    vP = rng.standard_normal(P.shape)
    h = 1e-6
    L = lambda Xa, Pa: float(np.sum(sa_forward_ref(off, Xa, Pa, True)[0] * dS))
    fdX = (L(X + h * vX, P) - L(X - h * vX, P)) / (2 * h)
    fdP = (L(X, P + h * vP) - L(X, P - h * vP)) / (2 * h)
    assert fdX == pytest.approx(float(np.sum(dX * vX)), rel=1e-6, abs=1e-8)
    assert fdP == pytest.approx(float(np.sum(dP * vP)), rel=1e-6, abs=1e-8)


def test_empty_user_contributes_nothing():
    off, X, P, dS = _prob(6, [10, 0, 5], 3, 4)
    dX, dP = sa_backward_ref(off, X, P, dS, True)
    keep = [0, 2]
    off2 = np.array([0, 10, 15])
    dX2, dP2 = sa_backward_ref(off2, X, P, dS[keep], True)
    np.testing.assert_allclose(dX, dX2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dP, dP2, rtol=1e-14, atol=1e-15)
