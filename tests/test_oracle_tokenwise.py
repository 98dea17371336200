"""Pins for the float64 oracle of the token-wise normalised sketch (the
vanilla-attention baseline of Table 1; SequenceO1 reading notes, sections 3.5
and 7.1).  No GPU."""

import math

import numpy as np
import pytest

from oracle.tokenwise import tokenwise_backward_ref, tokenwise_forward_brute, tokenwise_forward_ref


def _case(seed, lengths, k=3, d=2, p_scale=1.3):
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return off, rng.standard_normal((int(off[-1]), d)), rng.standard_normal((k, d)) * p_scale


def test_matches_scalar_loops():
    off, X, P = _case(0, [4, 0, 3, 1])
    S, lse = tokenwise_forward_ref(off, X, P)
    Sb, lseb = tokenwise_forward_brute(off.tolist(), X.tolist(), P.tolist())
    assert np.max(np.abs(S - Sb)) < 1e-12
    fin = np.isfinite(lseb)
    assert np.array_equal(fin, np.isfinite(lse)) and np.max(np.abs(lse[fin] - lseb[fin])) < 1e-12


def test_closed_forms():
    # one token: every prototype's distribution is that token, S_j = x
    off, X, P = _case(1, [1, 2], k=4, d=3)
    S, lse = tokenwise_forward_ref(off, X, P)
    assert np.allclose(S[0], np.repeat(X[:1], 4, axis=0), atol=1e-15)
    assert np.allclose(lse[0], (P @ X[0]) / math.sqrt(3), atol=1e-14)
    # P = 0: uniform weights, S_j = the user's mean row, lse = log n
    S0, lse0 = tokenwise_forward_ref(off, X, np.zeros_like(P))
    assert np.allclose(S0[1], np.repeat(X[1:3].mean(axis=0, keepdims=True), 4, axis=0), atol=1e-15)
    assert np.allclose(lse0[1], math.log(2), atol=1e-15)
    # an empty user
    off2 = np.array([0, 0, 3])
    S2, lse2 = tokenwise_forward_ref(off2, X, P)
    assert np.array_equal(S2[0], np.zeros((4, 3))) and np.all(np.isneginf(lse2[0]))


def test_token_permutation_invariance():
    off, X, P = _case(2, [6, 5])
    perm = np.concatenate([np.random.default_rng(3).permutation(6), 6 + np.arange(5)[::-1]])
    S1, l1 = tokenwise_forward_ref(off, X, P)
    S2, l2 = tokenwise_forward_ref(off, X[perm], P)
    assert np.allclose(S1, S2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


def test_weights_are_distributions_over_tokens():
    # S_j is a convex combination of the user's rows: inside their bounding box
    off, X, P = _case(4, [7])
    S, _ = tokenwise_forward_ref(off, X, P * 3)
    assert np.all(S[0] <= X.max(axis=0) + 1e-12) and np.all(S[0] >= X.min(axis=0) - 1e-12)


def test_backward_finite_differences():
    off, X, P = _case(5, [3, 0, 4], k=3, d=2)
    dS = np.random.default_rng(6).standard_normal((3, 3, 2))
    dX, dP = tokenwise_backward_ref(off, X, P, dS)

    def loss(X_, P_):
        return float(np.sum(dS * tokenwise_forward_ref(off, X_, P_)[0]))

    h = 1e-6
    for arr, grad in ((X, dX), (P, dP)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss(X, P)
            arr[idx] = old - h
            lm = loss(X, P)
            arr[idx] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - grad[idx]) < 1e-7 * max(1.0, abs(num))


def test_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    off, X, P = _case(7, [5, 1, 0, 8], k=4, d=4)
    dS = np.random.default_rng(8).standard_normal((4, 4, 4))
    dX, dP = tokenwise_backward_ref(off, X, P, dS)
    Xt = torch.tensor(X, requires_grad=True)
    Pt = torch.tensor(P, requires_grad=True)
    outs = []
    for u in range(4):
        xu = Xt[int(off[u]):int(off[u + 1])]
        if xu.shape[0] == 0:
            outs.append(torch.zeros(4, 4, dtype=torch.float64))
            continue
        A = torch.softmax(Pt @ xu.T / 2.0, dim=1)       # over tokens
        outs.append(A @ xu)
    (torch.stack(outs) * torch.tensor(dS)).sum().backward()
    assert np.allclose(Xt.grad.numpy(), dX, atol=1e-12)
    assert np.allclose(Pt.grad.numpy(), dP, atol=1e-12)
