"""Pins for the float64 oracle of the action-side SwiGLU fusion (SequenceO1
reading notes, section 3.6, Eq. (20)), with the readings of
oracle/action_fusion.py.  No GPU."""

import math

import numpy as np
import pytest

from oracle.action_fusion import action_fusion_backward_ref, action_fusion_ref


def _case(seed, T=7, d=3, n_types=4, scale=0.7):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, d)), rng.integers(0, n_types, T),
            rng.standard_normal((n_types, d)), rng.standard_normal((2 * d, 2 * d)) * scale,
            rng.standard_normal((2 * d, 2 * d)) * scale, rng.standard_normal((2 * d, d)) * scale)


def test_scalar_loops():
    e, t, A, W1, W3, W2 = _case(0, T=3, d=2, n_types=3)
    x = action_fusion_ref(e, t, A, W1, W3, W2)
    d = 2
    for i in range(3):
        v = list(e[i]) + list(A[t[i]])
        u1 = [math.fsum(v[a] * W1[a][c] for a in range(2 * d)) for c in range(2 * d)]
        u3 = [math.fsum(v[a] * W3[a][c] for a in range(2 * d)) for c in range(2 * d)]
        g = [u1[c] / (1.0 + math.exp(-u1[c])) * u3[c] for c in range(2 * d)]
        for o in range(d):
            want = e[i][o] + math.fsum(g[c] * W2[c][o] for c in range(2 * d))
            assert abs(x[i][o] - want) < 1e-12


def test_special_cases():
    e, t, A, W1, W3, W2 = _case(1)
    # no FFN output: the rows are the item embeddings
    assert np.array_equal(action_fusion_ref(e, t, A, W1, W3, np.zeros_like(W2)), e)
    assert np.array_equal(action_fusion_ref(e, t, A, W1, np.zeros_like(W3), W2), e)
    # the same item under two action types gives two rows unless the action
    # half of the weights is zero
    e2 = np.repeat(e[:1], 2, axis=0)
    t2 = np.array([0, 1])
    x = action_fusion_ref(e2, t2, A, W1, W3, W2)
    assert not np.allclose(x[0], x[1])
    W1z, W3z = W1.copy(), W3.copy()
    W1z[3:], W3z[3:] = 0.0, 0.0
    x = action_fusion_ref(e2, t2, A, W1z, W3z, W2)
    assert np.array_equal(x[0], x[1])


def test_backward_finite_differences():
    e, t, A, W1, W3, W2 = _case(2, T=5, d=2, n_types=3)
    dx = np.random.default_rng(3).standard_normal((5, 2))
    grads = action_fusion_backward_ref(e, t, A, W1, W3, W2, dx)
    h = 1e-6
    arrs = [e, A, W1, W3, W2]
    for which, (arr, g) in enumerate(zip(arrs, grads)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = float(np.sum(dx * action_fusion_ref(e, t, A, W1, W3, W2)))
            arr[idx] = old - h
            lm = float(np.sum(dx * action_fusion_ref(e, t, A, W1, W3, W2)))
            arr[idx] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - g[idx]) < 1e-7 * max(1.0, abs(num)), (which, idx)


def test_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    e, t, A, W1, W3, W2 = _case(4, T=9, d=4, n_types=5)
    dx = np.random.default_rng(5).standard_normal((9, 4))
    grads = action_fusion_backward_ref(e, t, A, W1, W3, W2, dx)
    ts = [torch.tensor(a, requires_grad=True) for a in (e, A, W1, W3, W2)]
    et, At, W1t, W3t, W2t = ts
    v = torch.cat([et, At[torch.tensor(t)]], dim=1)
    x = et + (torch.nn.functional.silu(v @ W1t) * (v @ W3t)) @ W2t
    (x * torch.tensor(dx)).sum().backward()
    for tt, g in zip(ts, grads):
        assert np.allclose(tt.grad.numpy(), g, atol=1e-12)
