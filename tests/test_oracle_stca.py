"""Pins for the float64 oracle of the reordered single-query STCA attention
(SequenceO1 reading notes, section 5.1, Eq. (24)-(25)).  No GPU."""

import math

import numpy as np

from oracle.stca import stca_attention_ref, stca_attention_unreordered, stca_layer_ref


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


def test_lse_two_rows_closed_form():
    # One head (d_h = D = 2), W_Q = W_K = I: the scores of rows a e1 and b e1
    # for query c e1 are a c / sqrt(2) and b c / sqrt(2).  Their log-sum-exp
    # is s_max + log(1 + exp(-delta)), delta = |s1 - s2|.
    a, b, c = 3.0, -1.5, 2.0
    X = np.array([[a, 0.0], [b, 0.0]])
    Q = np.array([[c, 0.0]])
    eye = np.eye(2)
    _, lse = stca_attention_ref(np.array([0, 2]), X, np.array([0, 1]), Q, eye, eye, eye, 1)
    s1, s2 = a * c / math.sqrt(2), b * c / math.sqrt(2)
    want = max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2)))
    assert abs(max(s1, s2)) > 4.0          # the maximum is far from zero
    assert abs(lse[0, 0] - want) < 1e-13


def test_lse_matches_library_logsumexp_per_head():
    from scipy.special import logsumexp

    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(4, [9, 3], [2, 2], D=8, h=4)
    Q = Q * 3.0                            # scores of several units
    _, lse = stca_attention_ref(x_off, X, t_off, Q, Wq, Wk, Wv, 4)
    # standard (unreordered) scores K q / sqrt(d_h) with K = X W_K per head
    for r in range(4):
        u = 0 if r < 2 else 1
        Xu = X[x_off[u]:x_off[u + 1]]
        for j in range(4):
            cols = slice(2 * j, 2 * j + 2)
            s = (Xu @ Wk[:, cols]) @ (Q[r] @ Wq[:, cols]) / math.sqrt(2)
            assert abs(np.max(s)) > 0.5
            assert abs(lse[r, j] - logsumexp(s)) < 1e-12


def _layer_weights(seed, D):
    rng = np.random.default_rng(seed)
    Wo = rng.standard_normal((D, D)) * 0.4
    W1 = rng.standard_normal((D, 2 * D)) * 0.4
    W3 = rng.standard_normal((D, 2 * D)) * 0.4
    W2 = rng.standard_normal((2 * D, D)) * 0.4
    return Wo, W1, W3, W2


def test_layer_against_torch_attention_and_silu():
    # Independent form of Eq. (26): K = X W_K and V = X W_V materialised per
    # head, torch's scaled_dot_product_attention (scale 1/sqrt(d_h)), torch's
    # silu, float64 on the CPU.
    import torch
    import torch.nn.functional as F

    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(5, [6, 0, 9], [2, 1, 3], D=8, h=2)
    Wo, W1, W3, W2 = _layer_weights(6, 8)
    y, o, _ = stca_layer_ref(x_off, X, t_off, Q, Wq, Wk, Wv, Wo, W1, W3, W2, 2)
    t = lambda a: torch.as_tensor(a, dtype=torch.float64)
    yt = torch.zeros(Q.shape[0], 8, dtype=torch.float64)
    for u in range(3):
        Xu = t(X[x_off[u]:x_off[u + 1]])
        for r in range(t_off[u], t_off[u + 1]):
            heads = []
            for j in range(2):
                cols = slice(4 * j, 4 * j + 4)
                if Xu.shape[0] == 0:
                    heads.append(torch.zeros(4, dtype=torch.float64))
                    continue
                q = (t(Q[r]) @ t(Wq)[:, cols])[None, None]
                k = (Xu @ t(Wk)[:, cols])[None]
                v = (Xu @ t(Wv)[:, cols])[None]
                heads.append(F.scaled_dot_product_attention(q, k, v)[0, 0])
            a = t(Q[r]) + torch.cat(heads) @ t(Wo)
            yt[r] = a + (F.silu(a @ t(W1)) * (a @ t(W3))) @ t(W2)
    assert np.max(np.abs(y - yt.numpy())) < 1e-12


def test_layer_special_cases():
    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(7, [5, 3], [2, 2], D=8, h=4)
    Wo, W1, W3, W2 = _layer_weights(8, 8)
    _, o, _ = stca_layer_ref(x_off, X, t_off, Q, Wq, Wk, Wv, Wo, W1, W3, W2, 4)
    # W2 = 0: the FFN adds nothing, y = q + o W_O (the attention path alone)
    y0, _, _ = stca_layer_ref(x_off, X, t_off, Q, Wq, Wk, Wv, Wo, W1, W3, np.zeros((16, 8)), 4)
    assert np.max(np.abs(y0 - (Q + o @ Wo))) < 1e-12
    # W_O = 0: the FFN acts on q itself, y = q + FFN(q), FFN by scipy's expit
    from scipy.special import expit

    yq, _, _ = stca_layer_ref(x_off, X, t_off, Q, Wq, Wk, Wv, np.zeros((8, 8)), W1, W3, W2, 4)
    u1 = Q @ W1
    want = Q + (u1 * expit(u1) * (Q @ W3)) @ W2
    assert np.max(np.abs(yq - want)) < 1e-12
    # both zero: y = q
    yz, _, _ = stca_layer_ref(x_off, X, t_off, Q, Wq, Wk, Wv, np.zeros((8, 8)), W1, W3,
                              np.zeros((16, 8)), 4)
    assert np.array_equal(yz, Q)
