"""Pins for the float64 oracle of the stacked Sketch Attention block (no GPU).

SequenceO1 reading notes, section 3.3 (stacked refinement), Eq. (12)-(16),
with the readings stated in oracle/block.py (SwiGLU FFN of hidden width 2d,
layer norm with scale and shift, eps 1e-5).  Pinned by:
  - a pure-Python scalar-loop evaluation of the block with the projections
    applied as printed;
  - layer-norm identities (zero mean, unit variance, affine) and SwiGLU
    special cases (W3 = 0 gives 0, silu at known points);
  - central finite differences of the whole block's loss for every input;
  - torch float64 autograd of an independently written torch forward.
"""

import math

import numpy as np
import pytest

from oracle.block import (LAYER_KEYS, block_backward_ref, block_forward_brute, block_forward_ref,
                          layer_norm_ref, silu, swiglu_ffn_ref)


def _layers(rng, n, d, scale=0.6):
    out = []
    for _ in range(n):
        out.append(dict(
            Wq=rng.standard_normal((d, d)) * scale, Wk=rng.standard_normal((d, d)) * scale,
            g1=1.0 + 0.3 * rng.standard_normal(d), b1=0.2 * rng.standard_normal(d),
            W1=rng.standard_normal((d, 2 * d)) * scale, W3=rng.standard_normal((d, 2 * d)) * scale,
            W2=rng.standard_normal((2 * d, d)) * scale,
            g2=1.0 + 0.3 * rng.standard_normal(d), b2=0.2 * rng.standard_normal(d)))
    return out


def _case(seed, lengths, k=3, d=2, n_layers=2):
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    X = rng.standard_normal((int(off[-1]), d))
    P0 = rng.standard_normal((k, d))
    return off, X, P0, _layers(rng, n_layers, d)


def test_layer_norm_identities():
    rng = np.random.default_rng(0)
    v = rng.standard_normal((5, 6)) * 3 + 1
    y, xh, _ = layer_norm_ref(v, np.ones(6), np.zeros(6))
    assert np.allclose(y.mean(axis=-1), 0, atol=1e-12)
    # biased variance with eps: var(y) = var(v) / (var(v) + eps)
    var = v.var(axis=-1)
    assert np.allclose(y.var(axis=-1), var / (var + 1e-5), atol=1e-12)
    g, b = rng.standard_normal(6), rng.standard_normal(6)
    y2, _, _ = layer_norm_ref(v, g, b)
    assert np.allclose(y2, xh * g + b, atol=1e-14)
    # shifting a row leaves it unchanged
    assert np.allclose(layer_norm_ref(v + 7.0, g, b)[0], y2, atol=1e-12)


def test_swiglu_special_cases():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 3))
    W1, W3, W2 = rng.standard_normal((3, 6)), rng.standard_normal((3, 6)), rng.standard_normal((6, 3))
    assert np.array_equal(swiglu_ffn_ref(x, W1, np.zeros((3, 6)), W2)[0], np.zeros((4, 3)))
    assert silu(0.0) == 0.0
    assert abs(silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(silu(40.0) - 40.0) < 1e-12 and abs(silu(-40.0)) < 1e-15
    # one hidden unit, written out
    w1, w3, w2 = rng.standard_normal((3, 1)), rng.standard_normal((3, 1)), rng.standard_normal((1, 3))
    u1, u3 = float(x[0] @ w1[:, 0]), float(x[0] @ w3[:, 0])
    want = (u1 / (1.0 + math.exp(-u1))) * u3 * w2[0]
    assert np.allclose(swiglu_ffn_ref(x[:1], w1, w3, w2)[0][0], want, atol=1e-13)


@pytest.mark.parametrize("n_layers", [1, 2])
def test_forward_matches_scalar_loops(n_layers):
    off, X, P0, layers = _case(2, [3, 0, 4], k=3, d=2, n_layers=n_layers)
    out, _ = block_forward_ref(off, X, P0, layers)
    ref = block_forward_brute(off.tolist(), X.tolist(), P0.tolist(), layers)
    assert np.max(np.abs(out - ref)) < 1e-11


def test_empty_user_keeps_layer_norms_of_the_table():
    # a user without history: X^ = 0, so layer 0 gives LN(P0) through the FFN
    off, X, P0, layers = _case(3, [0, 2], k=2, d=3, n_layers=1)
    out, saved = block_forward_ref(off, X, P0, layers)
    L = layers[0]
    xbar, _, _ = layer_norm_ref(P0, L["g1"], L["b1"])
    F, _, _ = swiglu_ffn_ref(xbar, L["W1"], L["W3"], L["W2"])
    want, _, _ = layer_norm_ref(xbar + F, L["g2"], L["b2"])
    assert np.allclose(out[0], want, atol=1e-13)


def _loss(off, X, P0, layers, dout):
    return float(np.sum(dout * block_forward_ref(off, X, P0, layers)[0]))


@pytest.mark.parametrize("n_layers", [1, 2])
def test_backward_finite_differences(n_layers):
    off, X, P0, layers = _case(4, [2, 0, 3], k=3, d=2, n_layers=n_layers)
    dout = np.random.default_rng(5).standard_normal((3, 3, 2))
    dX, dP0, grads = block_backward_ref(off, X, P0, layers, dout)
    h = 1e-6

    def check(arr, grad, name):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(off, X, P0, layers, dout)
            arr[idx] = old - h
            lm = _loss(off, X, P0, layers, dout)
            arr[idx] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - grad[idx]) < 1e-6 * max(1.0, abs(num)), (name, idx, num, grad[idx])

    check(X, dX, "X")
    check(P0, dP0, "P0")
    for li, L in enumerate(layers):
        for key in LAYER_KEYS:
            check(L[key], grads[li][key], f"layer {li} {key}")


def test_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    off, X, P0, layers = _case(6, [5, 1, 0, 4], k=4, d=4, n_layers=2)
    dout = np.random.default_rng(7).standard_normal((4, 4, 4))
    dX, dP0, grads = block_backward_ref(off, X, P0, layers, dout)

    # An independent forward in torch float64: per user, Eq. (12) unfolded.
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    Xt, P0t = t(X), t(P0)
    Lt = [{key: t(L[key]) for key in LAYER_KEYS} for L in layers]
    d = X.shape[1]

    def ln(v, g, b):
        mu = v.mean(-1, keepdim=True)
        var = ((v - mu) ** 2).mean(-1, keepdim=True)
        return (v - mu) / torch.sqrt(var + 1e-5) * g + b

    outs = []
    for u in range(len(off) - 1):
        xu = Xt[int(off[u]):int(off[u + 1])]
        q = P0t
        for L in Lt:
            z = (q @ L["Wq"]) @ (xu @ L["Wk"]).T / math.sqrt(d)        # k x n
            A = torch.softmax(z, dim=0)
            xbar = ln(q + A @ xu, L["g1"], L["b1"])
            u1, u3 = xbar @ L["W1"], xbar @ L["W3"]
            q = ln(xbar + (torch.nn.functional.silu(u1) * u3) @ L["W2"], L["g2"], L["b2"])
        outs.append(q)
    loss = (torch.stack(outs) * torch.tensor(dout)).sum()
    loss.backward()
    assert np.allclose(Xt.grad.numpy(), dX, atol=1e-10)
    assert np.allclose(P0t.grad.numpy(), dP0, atol=1e-10)
    for li in range(2):
        for key in LAYER_KEYS:
            assert np.allclose(Lt[li][key].grad.numpy(), grads[li][key], atol=1e-10), (li, key)
