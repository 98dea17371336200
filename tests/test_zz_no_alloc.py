"""sa_forward_noalloc (the forward on the library's own workspace array, for
callers that cannot allocate) against sa_forward with a caller workspace:
bitwise the same outputs, on two calls in a row, the second with a smaller
problem; a problem whose workspace exceeds the array is refused before
anything is enqueued."""

import pytest
import torch

from recommender_ultra_long_amd import sa, synth
from sa_testutil import say

pytestmark = pytest.mark.gpu


def _outputs(prob):
    B = len(prob.offsets) - 1
    T, d = prob.X.shape
    k = prob.P.shape[-2]
    dev = "cuda"
    return (torch.full((B, k, d), float("nan"), device=dev),
            torch.full((T,), float("nan"), device=dev),
            torch.full((B, k), float("nan"), device=dev))


def _check(prob):
    off = torch.as_tensor(prob.offsets, device="cuda")
    S, lse, mass = _outputs(prob)
    sa.sa_forward_noalloc(off, prob.X, prob.P, S, lse, mass, prob.mass_norm)
    Sr, lr, mr = sa.sa_forward(off, prob.X, prob.P, prob.mass_norm)
    torch.cuda.synchronize()
    assert torch.equal(S, Sr) and torch.equal(lse, lr) and torch.equal(mass, mr)
    # without lse and mass (the array then also holds lse)
    S2 = torch.full_like(S, float("nan"))
    sa.sa_forward_noalloc(off, prob.X, prob.P, S2, None, None, prob.mass_norm)
    torch.cuda.synchronize()
    assert torch.equal(S2, Sr)


def test_noalloc_forward_matches_sa_forward_twice_then_smaller():
    say("case noalloc: 4 users up to 40000 tokens, k=1024, d=128, bf16, mass-normalised")
    big = synth.make_inputs([40000, 0, 25000, 17], 1024, 128, "bf16", device="cuda", seed=1,
                            wid=800, mass_norm=True)
    _check(big)
    say("case noalloc: the same again")
    _check(big)
    say("case noalloc: smaller, 2 users, k=300, d=64, fp32")
    small = synth.make_inputs([3000, 41], 300, 64, "f32", device="cuda", seed=2, wid=801)
    _check(small)


def test_noalloc_refuses_problems_beyond_its_array():
    # 64 users at k = 2048: 95 partial sketches of 1 MiB each, more than the
    # library's 64 MiB array.
    pr = sa.make_problem(64, 2048, 128, 64 * 1000, sa.SA_BF16)
    assert sa.workspace_size(pr, sa.SA_OP_FORWARD) > sa.SA_NOALLOC_SCRATCH_BYTES
    prob = synth.make_inputs([1000] * 64, 2048, 128, "bf16", device="cuda", seed=3, wid=802)
    off = torch.as_tensor(prob.offsets, device="cuda")
    S = torch.zeros(64, 2048, 128, device="cuda")
    with pytest.raises(sa.SAError) as err:
        sa.sa_forward_noalloc(off, prob.X, prob.P, S)
    assert err.value.status == sa.SA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(S)) == 0      # nothing ran
