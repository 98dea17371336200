"""GPU parity with one prototype table per user (SA_FLAG_PER_USER_PROTOTYPES:
the refinement layers of the SequenceO1 reading notes, section 3.3,
Eq. (12)-(14), whose queries are each user's own sketch).  Forward S, lse and
mass, and backward dX and the per-user dP, through the C-ABI against the
float64 oracle, with the forward's tolerances: max|gpu - ref| / max|ref| per
user (over the whole tensor for dP), <= 1e-4 (fp32 path) and <= 2e-2 (bf16
inputs)."""

import numpy as np
import pytest
import torch

from oracle.sa_ref import sa_backward_ref, sa_forward_ref
from recommender_ultra_long_amd import sa, synth
from sa_testutil import TOL_BF16, TOL_F32, TOL_LSE_ABS, rel_err, say

pytestmark = pytest.mark.gpu

# Length mixes: users inside one 256-token block, users straddling blocks and
# 32-token tiles, empty users, one user over many segments.
MIXES = {
    "short": [5, 0, 31, 33, 1, 64, 100, 0, 17],
    "mixed": [300, 7, 0, 513, 1, 255, 257, 40],
    "long": [3000, 12, 4500, 0, 700],
}


def _prob(mix, k, d, dtype, mass_norm, seed=0):
    return synth.make_inputs(MIXES[mix], k, d, dtype, device="cuda", seed=seed, wid=300 + seed,
                             with_dS=True, mass_norm=mass_norm, per_user_p=True)


def _run(prob):
    off = torch.as_tensor(prob.offsets, device="cuda")
    S, lse, mass = sa.sa_forward(off, prob.X, prob.P, prob.mass_norm)
    dX, dP = sa.sa_backward(off, prob.X, prob.P, prob.dS, lse, S, mass, prob.mass_norm)
    torch.cuda.synchronize()
    return S, lse, mass, dX, dP


@pytest.mark.parametrize("dtype,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mix", ["short", "mixed", "long"])
@pytest.mark.parametrize("mass_norm", [False, True])
def test_per_user_forward_backward(dtype, tol, d, mix, mass_norm):
    k = 300 if d == 128 else 64
    say(f"case per-user dtype={dtype} d={d} k={k} mix={mix} mass_norm={mass_norm}")
    prob = _prob(mix, k, d, dtype, mass_norm, seed=d + len(mix))
    S, lse, mass, dX, dP = _run(prob)
    X64, P64, dS64 = synth.to_f64(prob.X), synth.to_f64(prob.P), synth.to_f64(prob.dS)
    Sr, lr, mr = sa_forward_ref(prob.offsets, X64, P64, mass_norm)
    dXr, dPr = sa_backward_ref(prob.offsets, X64, P64, dS64, mass_norm)
    assert dP.shape == P64.shape
    # dP is measured over the whole tensor, as for a shared table: a user's
    # own dP can be exactly zero (one token under mass normalisation has
    # S_j = x for every prototype), where a per-user ratio is meaningless.
    dscale = float(np.max(np.abs(dPr)))
    dPg = dP.cpu().numpy()
    for u in range(len(prob.offsets) - 1):
        lo, hi = int(prob.offsets[u]), int(prob.offsets[u + 1])
        assert rel_err(S[u].cpu().numpy(), Sr[u]) <= tol, f"user {u}: S"
        assert rel_err(mass[u].cpu().numpy(), mr[u]) <= tol, f"user {u}: mass"
        if hi == lo:
            assert torch.count_nonzero(dP[u]) == 0, f"empty user {u}: dP not zero"
            continue
        assert float(np.max(np.abs(lse[lo:hi].cpu().numpy() - lr[lo:hi]))) <= TOL_LSE_ABS
        assert rel_err(dX[lo:hi].cpu().numpy(), dXr[lo:hi]) <= tol, f"user {u}: dX"
        eP = float(np.max(np.abs(dPg[u] - dPr[u]))) / dscale
        assert eP <= tol, f"user {u}: dP err {eP:.3e} of max |dP|"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identical_tables_give_the_shared_sketch(dtype):
    # Every user given the same table: the per-user path must reproduce the
    # shared-table forward bit for bit (same arithmetic, tables reloaded), and
    # its per-user dP must add up to the shared dP.
    say(f"case per-user identical tables dtype={dtype}")
    prob = _prob("mixed", 256, 128, dtype, False, seed=5)
    shared = prob.P[0].contiguous()
    stack = shared.unsqueeze(0).repeat(prob.P.shape[0], 1, 1).contiguous()
    off = torch.as_tensor(prob.offsets, device="cuda")
    S1, l1, m1 = sa.sa_forward(off, prob.X, shared, False)
    S2, l2, m2 = sa.sa_forward(off, prob.X, stack, False)
    _, dP1 = sa.sa_backward(off, prob.X, shared, prob.dS, l1)
    _, dP2 = sa.sa_backward(off, prob.X, stack, prob.dS, l2)
    torch.cuda.synchronize()
    assert torch.equal(S1, S2) and torch.equal(l1, l2) and torch.equal(m1, m2)
    e = rel_err(dP2.sum(dim=0).cpu().numpy(), dP1.cpu().numpy().astype(np.float64))
    assert e <= 1e-5, f"sum of per-user dP vs shared dP: {e:.3e}"


@pytest.mark.parametrize("dtype,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
def test_lse_recomputed_in_backward(dtype, tol):
    # lse not passed: the backward recomputes it with each user's own table
    say(f"case per-user backward recomputes lse dtype={dtype}")
    prob = _prob("short", 64, 64, dtype, True, seed=9)
    off = torch.as_tensor(prob.offsets, device="cuda")
    S, _, mass = sa.sa_forward(off, prob.X, prob.P, True)
    dX, dP = sa.sa_backward(off, prob.X, prob.P, prob.dS, None, S, mass, True)
    torch.cuda.synchronize()
    X64, P64, dS64 = synth.to_f64(prob.X), synth.to_f64(prob.P), synth.to_f64(prob.dS)
    dXr, dPr = sa_backward_ref(prob.offsets, X64, P64, dS64, True)
    for u in range(len(prob.offsets) - 1):
        lo, hi = int(prob.offsets[u]), int(prob.offsets[u + 1])
        if hi > lo:
            assert rel_err(dX[lo:hi].cpu().numpy(), dXr[lo:hi]) <= tol, f"user {u}: dX"
            eP = float(np.max(np.abs(dP[u].cpu().numpy() - dPr[u]))) / float(np.max(np.abs(dPr)))
            assert eP <= tol, f"user {u}: dP err {eP:.3e} of max |dP|"
