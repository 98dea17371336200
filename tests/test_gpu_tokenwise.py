"""GPU parity of the token-wise normalised sketch (SA_FLAG_TOKEN_WISE, the
vanilla-attention baseline of Table 1; SequenceO1 reading notes, sections 3.5
and 7.1) against the float64 oracle (oracle/tokenwise.py): max|gpu - ref| /
max|ref| per user for S, <= 1e-4 (fp32) and <= 2e-2 (bf16); lse absolute."""

import numpy as np
import pytest
import torch

from oracle.tokenwise import tokenwise_forward_ref
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
