"""GPU parity of the token-wise normalised sketch (SA_FLAG_TOKEN_WISE, the
vanilla-attention baseline of Table 1; SequenceO1 reading notes, sections 3.5
and 7.1) against the float64 oracle (oracle/tokenwise.py): max|gpu - ref| /
max|ref| per user for S and dX, over the tensor for dP, <= 1e-4 (fp32) and
<= 2e-2 (bf16); lse absolute."""

import numpy as np
import pytest
import torch

from oracle.tokenwise import tokenwise_backward_ref, tokenwise_forward_ref
from recommender_ultra_long_amd import sa, synth
from sa_testutil import TOL_BF16, TOL_F32, TOL_LSE_ABS, rel_err, say

pytestmark = pytest.mark.gpu


def _check(prob, S, lse, tol):
    X64, P64 = synth.to_f64(prob.X), synth.to_f64(prob.P)
    Sr, lr = tokenwise_forward_ref(prob.offsets, X64, P64)
    for u in range(len(prob.offsets) - 1):
        e = rel_err(S[u].cpu().numpy(), Sr[u])
        assert e <= tol, f"user {u}: S rel err {e:.3e}"
        lg = lse[u].cpu().numpy()
        if prob.offsets[u + 1] == prob.offsets[u]:
            assert np.all(np.isneginf(lg)), f"empty user {u}: lse not -inf"
        else:
            el = float(np.max(np.abs(lg - lr[u])))
            assert el <= TOL_LSE_ABS * max(1.0, float(np.max(np.abs(lr[u])))), f"user {u}: lse {el:.3e}"


@pytest.mark.parametrize("dtype,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("k", [1, 100, 300])
def test_tokenwise_forward(dtype, tol, d, k):
    lengths = [0, 1, 31, 33, 700, 0, 2500, 5]
    say(f"case tokenwise dtype={dtype} d={d} k={k}")
    prob = synth.make_inputs(lengths, k, d, dtype, device="cuda", seed=k + d, wid=500)
    S, lse = sa.tokenwise_forward(torch.as_tensor(prob.offsets, device="cuda"), prob.X, prob.P)
    torch.cuda.synchronize()
    _check(prob, S, lse, tol)


@pytest.mark.parametrize("dtype,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
def test_tokenwise_growing_maxima(dtype, tol):
    # sharp logits on rows whose norm grows along the history: the running
    # maxima keep rising past the rescale threshold, tile after tile
    say(f"case tokenwise growing maxima dtype={dtype}")
    lengths = [6000, 40]
    prob = synth.make_inputs(lengths, 256, 128, dtype, device="cuda", seed=3, wid=510, p_std=2.0)
    ramp = torch.linspace(0.5, 6.0, prob.X.shape[0], device="cuda")[:, None]
    prob.X = (prob.X.float() * ramp).to(prob.X.dtype)
    S, lse = sa.tokenwise_forward(torch.as_tensor(prob.offsets, device="cuda"), prob.X, prob.P)
    torch.cuda.synchronize()
    _check(prob, S, lse, tol)


def test_tokenwise_long_user_many_segments():
    say("case tokenwise 100k user")
    prob = synth.make_inputs([100000], 1024, 128, "bf16", device="cuda", seed=1, wid=520)
    S, lse = sa.tokenwise_forward(torch.as_tensor(prob.offsets, device="cuda"), prob.X, prob.P)
    torch.cuda.synchronize()
    _check(prob, S, lse, TOL_BF16)


def _check_backward(prob, dS, dX, dP, tol):
    X64, P64 = synth.to_f64(prob.X), synth.to_f64(prob.P)
    dXr, dPr = tokenwise_backward_ref(prob.offsets, X64, P64, synth.to_f64(dS))
    e = rel_err(dP.cpu().numpy(), dPr)
    assert e <= tol, f"dP rel err {e:.3e}"
    for u in range(len(prob.offsets) - 1):
        lo, hi = int(prob.offsets[u]), int(prob.offsets[u + 1])
        if hi > lo:
            e = rel_err(dX[lo:hi].cpu().numpy(), dXr[lo:hi])
            assert e <= tol, f"user {u}: dX rel err {e:.3e}"


@pytest.mark.parametrize("dtype,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("k", [1, 100, 300])
def test_tokenwise_backward(dtype, tol, d, k):
    lengths = [0, 1, 31, 33, 700, 0, 2500, 5]
    say(f"case tokenwise backward dtype={dtype} d={d} k={k}")
    prob = synth.make_inputs(lengths, k, d, dtype, device="cuda", seed=k + d, wid=530, with_dS=True)
    off = torch.as_tensor(prob.offsets, device="cuda")
    S, lse = sa.tokenwise_forward(off, prob.X, prob.P)
    dX, dP = sa.tokenwise_backward(off, prob.X, prob.P, prob.dS, S, lse)
    torch.cuda.synchronize()
    _check_backward(prob, prob.dS, dX, dP, tol)


def test_tokenwise_backward_long_user():
    say("case tokenwise backward 100k user")
    prob = synth.make_inputs([100000, 3000], 1024, 128, "bf16", device="cuda", seed=2, wid=540,
                             with_dS=True)
    off = torch.as_tensor(prob.offsets, device="cuda")
    S, lse = sa.tokenwise_forward(off, prob.X, prob.P)
    dX, dP = sa.tokenwise_backward(off, prob.X, prob.P, prob.dS, S, lse)
    torch.cuda.synchronize()
    _check_backward(prob, prob.dS, dX, dP, TOL_BF16)
