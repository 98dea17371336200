"""GPU parity of the reordered single-query STCA attention (SequenceO1 reading
notes, section 5.1, Eq. (24)) through the C-ABI against the float64 oracle
(oracle/stca.py): max|gpu - ref| / max|ref| over o, <= 2e-2 (bf16 history
rows and query rows on the matrix cores, fp32 accumulation); lse absolute."""

import numpy as np
import pytest
import torch

from oracle.stca import stca_attention_ref
from recommender_ultra_long_amd import sa, synth
from sa_testutil import TOL_BF16, TOL_LSE_ABS, record, rel_err, say

pytestmark = pytest.mark.gpu


def _case(seed, x_lens, t_lens, D, h):
    g = torch.Generator().manual_seed(seed)
    x_off = np.concatenate([[0], np.cumsum(x_lens)]).astype(np.int64)
    t_off = np.concatenate([[0], np.cumsum(t_lens)]).astype(np.int64)
    X = torch.randn(int(x_off[-1]), D, generator=g).to(torch.bfloat16)
    Q = torch.randn(int(t_off[-1]), D, generator=g)
    s = D ** -0.5
    W = [torch.randn(D, D, generator=g) * s for _ in range(3)]
    return x_off, X, t_off, Q, W


@pytest.mark.parametrize("D,h", [(256, 4), (256, 8), (256, 16), (512, 8), (512, 64), (1024, 1),
                                 (1024, 8), (1024, 16)])
def test_stca_attention(D, h):
    x_lens = [700, 0, 1, 33, 1024, 90]
    t_lens = [3, 2, 1, 0, 5, 4]
    say(f"case stca D={D} h={h}")
    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(D + h, x_lens, t_lens, D, h)
    o, lse = sa.stca_attention(torch.as_tensor(x_off, device="cuda"), X.cuda(),
                               torch.as_tensor(t_off, device="cuda"), Q.cuda(), Wq.cuda(),
                               Wk.cuda(), Wv.cuda(), h)
    torch.cuda.synchronize()
    ro, rl = stca_attention_ref(x_off, synth.to_f64(X), t_off, Q.double().numpy(),
                                Wq.double().numpy(), Wk.double().numpy(), Wv.double().numpy(), h)
    og = o.cpu().numpy()
    # per target: a target whose outputs are small must still be right
    for r in range(ro.shape[0]):
        if np.any(ro[r] != 0):
            e = rel_err(og[r], ro[r])
            assert e <= TOL_BF16, f"target {r}: o rel err {e:.3e}"
        else:
            assert not np.any(og[r]), f"target {r}: o should be zero"
    lg = lse.cpu().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lg), fin)
    assert float(np.max(np.abs(lg[fin] - rl[fin]))) <= 5 * TOL_LSE_ABS * max(1.0, float(np.max(np.abs(rl[fin]))))


def test_stca_many_targets_sharp_scores():
    # 10,000-row history (the recent branch), 300 targets, scores sharp
    # enough that the running maxima rise past the rescale threshold
    say("case stca recent branch 10k rows x 300 targets")
    D, h = 1024, 16
    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(7, [10000], [300], D, h)
    Q = Q * 6.0
    o, _ = sa.stca_attention(torch.as_tensor(x_off, device="cuda"), X.cuda(),
                             torch.as_tensor(t_off, device="cuda"), Q.cuda(), Wq.cuda(), Wk.cuda(),
                             Wv.cuda(), h)
    torch.cuda.synchronize()
    sel = np.arange(0, 300, 37)                    # sampled targets, checked one by one
    ro, _ = stca_attention_ref(np.array([0, 10000]), synth.to_f64(X), np.array([0, len(sel)]),
                               Q[sel].double().numpy(), Wq.double().numpy(), Wk.double().numpy(),
                               Wv.double().numpy(), h)
    og = o.cpu().numpy()[sel]
    for r in range(len(sel)):
        e = rel_err(og[r], ro[r])
        assert e <= TOL_BF16, f"target {sel[r]}: o rel err {e:.3e}"


def test_stca_users_without_history():
    # every target's user has no rows: o = 0 and lse = -inf throughout
    say("case stca no history rows")
    D, h = 512, 8
    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(11, [0, 0, 0], [2, 0, 3], D, h)
    X = torch.zeros(16, D, dtype=torch.bfloat16)              # L = 0: no row is read
    o, lse = sa.stca_attention(torch.as_tensor(x_off, device="cuda"), X.cuda(),
                               torch.as_tensor(t_off, device="cuda"), Q.cuda(), Wq.cuda(),
                               Wk.cuda(), Wv.cuda(), h)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
    assert bool(torch.all(torch.isneginf(lse)).item())


def test_stca_is_deterministic():
    # no atomics anywhere: two calls on the same inputs agree bit for bit
    say("case stca determinism")
    D, h = 1024, 16
    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(5, [3000, 17, 900], [7, 3, 40], D, h)
    args = (torch.as_tensor(x_off, device="cuda"), X.cuda(), torch.as_tensor(t_off, device="cuda"),
            Q.cuda(), Wq.cuda(), Wk.cuda(), Wv.cuda(), h)
    o1, l1 = sa.stca_attention(*args)
    o2, l2 = sa.stca_attention(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("D,h", [(256, 4), (256, 16), (1024, 16)])
def test_stca_layer_eq26(D, h):
    """The whole layer of Eq. (26): attention, a = q + o W_O, y = a + SwiGLU(a)
    (hidden width 2D).  Checked per target on y and on y - q (the part the
    products make), and on o."""
    from oracle.stca import stca_layer_ref

    x_lens = [700, 0, 33, 1024, 5]
    t_lens = [3, 2, 0, 5, 4]
    say(f"case stca layer D={D} h={h}")
    x_off, X, t_off, Q, (Wq, Wk, Wv) = _case(3 * D + h, x_lens, t_lens, D, h)
    g = torch.Generator().manual_seed(D + 7 * h)
    Wo = torch.randn(D, D, generator=g) * D ** -0.5
    W1 = torch.randn(D, 2 * D, generator=g) * D ** -0.5
    W3 = torch.randn(D, 2 * D, generator=g) * D ** -0.5
    W2 = torch.randn(2 * D, D, generator=g) * (2 * D) ** -0.5
    c = lambda t: t.cuda()
    y, o, lse = sa.stca_layer(torch.as_tensor(x_off, device="cuda"), c(X),
                              torch.as_tensor(t_off, device="cuda"), c(Q), c(Wq), c(Wk), c(Wv),
                              c(Wo), c(W1), c(W3), c(W2), h)
    torch.cuda.synchronize()
    f64 = lambda t: t.double().numpy()
    ry, ro, rl = stca_layer_ref(x_off, synth.to_f64(X), t_off, f64(Q), f64(Wq), f64(Wk), f64(Wv),
                                f64(Wo), f64(W1), f64(W3), f64(W2), h)
    yg, og, q = y.cpu().numpy(), o.cpu().numpy(), f64(Q)
    worst = {"y": 0.0, "y_minus_q": 0.0, "o": 0.0}
    for r in range(ry.shape[0]):
        for name, got, ref in (("y", yg[r], ry[r]), ("y_minus_q", yg[r] - q[r], ry[r] - q[r])):
            e = rel_err(got, ref)
            assert e <= TOL_BF16, f"target {r}: {name} rel err {e:.3e}"
            worst[name] = max(worst[name], e)
        if np.any(ro[r] != 0):
            e = rel_err(og[r], ro[r])
            assert e <= TOL_BF16, f"target {r}: o rel err {e:.3e}"
            worst["o"] = max(worst["o"], e)
        else:
            assert not np.any(og[r])
    record(f"stca layer (Eq. 26) D={D} h={h}", **worst)
