"""GPU parity of the folded query/key projections (SequenceO1 reading notes,
section 3.1, Eq. (6)): sa_fold_prototypes and its backward through the C-ABI
against the float64 oracle, alone and chained with the sketch's forward and
backward."""

import numpy as np
import pytest
import torch

from oracle.projections import fold_prototypes_backward_ref, fold_prototypes_ref
from oracle.sa_ref import sa_backward_ref, sa_forward_ref
from recommender_ultra_long_amd import sa
from sa_testutil import TOL_BF16, TOL_F32, rel_err, say

pytestmark = pytest.mark.gpu

TOL_FOLD_F32 = 1e-5   # fp32 products of k x d and d x d matrices
TOL_FOLD_BF16 = 1e-2  # one bf16 rounding of P_eff


def _inputs(seed, k, d, dtype):
    g = torch.Generator().manual_seed(seed)
    P = (torch.randn(k, d, generator=g) / np.sqrt(d)).to(dtype)
    Wq = torch.randn(d, d, generator=g) / np.sqrt(d)
    Wk = torch.randn(d, d, generator=g) / np.sqrt(d)
    return P, Wq, Wk


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("k,d", [(1, 32), (37, 64), (300, 128), (1024, 128), (2048, 32)])
def test_fold_parity(dtype, k, d):
    say(f"case fold dtype={dtype} k={k} d={d}")
    P, Wq, Wk = _inputs(k * 7 + d, k, d, dtype)
    Peff = sa.fold_prototypes(P.cuda(), Wq.cuda(), Wk.cuda())
    torch.cuda.synchronize()
    ref = fold_prototypes_ref(P.float().numpy(), Wq.numpy(), Wk.numpy())
    e = rel_err(Peff.float().cpu().numpy(), ref)
    assert e <= (TOL_FOLD_F32 if dtype == torch.float32 else TOL_FOLD_BF16), f"P_eff rel err {e:.3e}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("k,d", [(1, 32), (33, 32), (37, 64), (300, 128), (1024, 128), (2048, 64), (2048, 128)])
def test_fold_backward_parity(dtype, k, d):
    say(f"case fold backward dtype={dtype} k={k} d={d}")
    P, Wq, Wk = _inputs(k * 11 + d, k, d, dtype)
    G = torch.randn(k, d, generator=torch.Generator().manual_seed(k + d))
    dP, dWq, dWk = sa.fold_prototypes_backward(P.cuda(), Wq.cuda(), Wk.cuda(), G.cuda())
    torch.cuda.synchronize()
    rP, rWq, rWk = fold_prototypes_backward_ref(P.float().numpy(), Wq.numpy(), Wk.numpy(), G.numpy())
    for name, a, b in (("dP", dP, rP), ("dWq", dWq, rWq), ("dWk", dWk, rWk)):
        e = rel_err(a.cpu().numpy(), b)
        assert e <= TOL_FOLD_F32, f"{name} rel err {e:.3e}"


@pytest.mark.parametrize("rows", [32 * 1024, 40000])
def test_fold_of_stacked_user_tables(rows):
    # the refinement layers fold every user's table with one W_Q, W_K: B k rows
    # in one call (the gram slices then span several 128-row sub-chunks)
    say(f"case fold stacked rows={rows} d=128")
    P, Wq, Wk = _inputs(rows, rows, 128, torch.bfloat16)
    G = torch.randn(rows, 128, generator=torch.Generator().manual_seed(rows + 1))
    Peff = sa.fold_prototypes(P.cuda(), Wq.cuda(), Wk.cuda())
    dP, dWq, dWk = sa.fold_prototypes_backward(P.cuda(), Wq.cuda(), Wk.cuda(), G.cuda())
    torch.cuda.synchronize()
    P64 = P.float().numpy()
    assert rel_err(Peff.float().cpu().numpy(), fold_prototypes_ref(P64, Wq.numpy(), Wk.numpy())) <= TOL_FOLD_BF16
    rP, rWq, rWk = fold_prototypes_backward_ref(P64, Wq.numpy(), Wk.numpy(), G.numpy())
    for name, a, b in (("dP", dP, rP), ("dWq", dWq, rWq), ("dWk", dWk, rWk)):
        e = rel_err(a.cpu().numpy(), b)
        assert e <= TOL_F32, f"{name} rel err {e:.3e}"


def test_fold_backward_is_deterministic():
    # dW_Q and dW_K add the workgroups' partial sums in a fixed order
    say("case fold backward determinism k=2048 d=128")
    P, Wq, Wk = _inputs(5, 2048, 128, torch.bfloat16)
    G = torch.randn(2048, 128, generator=torch.Generator().manual_seed(6)).cuda()
    a = sa.fold_prototypes_backward(P.cuda(), Wq.cuda(), Wk.cuda(), G)
    b = sa.fold_prototypes_backward(P.cuda(), Wq.cuda(), Wk.cuda(), G)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("mass_norm", [False, True])
def test_projected_sketch_forward_and_backward(mass_norm):
    # fold -> sa_forward -> sa_backward -> fold backward, against the oracle
    # chain on unrounded float64 values.
    say(f"case projected sketch mass_norm={mass_norm}")
    k, d = 256, 64
    lengths = [700, 0, 1500, 33]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(off[-1])
    g = torch.Generator().manual_seed(5)
    X = torch.randn(T, d, generator=g).to(torch.bfloat16)
    P, Wq, Wk = _inputs(6, k, d, torch.bfloat16)
    dS = torch.randn(len(lengths), k, d, generator=g)
    offd = torch.as_tensor(off, device="cuda")
    Peff = sa.fold_prototypes(P.cuda(), Wq.cuda(), Wk.cuda())
    S, lse, mass = sa.sa_forward(offd, X.cuda(), Peff, mass_norm)
    dX, dPeff = sa.sa_backward(offd, X.cuda(), Peff, dS.cuda(), lse, S, mass, mass_norm)
    dP, dWq, dWk = sa.fold_prototypes_backward(P.cuda(), Wq.cuda(), Wk.cuda(), dPeff)
    torch.cuda.synchronize()
    X64, P64 = X.float().numpy(), P.float().numpy()
    Pe = fold_prototypes_ref(P64, Wq.numpy(), Wk.numpy())
    rS, _, _ = sa_forward_ref(off, X64, Pe, mass_norm)
    rdX, rdPe = sa_backward_ref(off, X64, Pe, dS.numpy(), mass_norm)
    rdP, rdWq, rdWk = fold_prototypes_backward_ref(P64, Wq.numpy(), Wk.numpy(), rdPe)
    for name, a, b in (("S", S, rS), ("dX", dX, rdX), ("dP", dP, rdP), ("dWq", dWq, rdWq),
                       ("dWk", dWk, rdWk)):
        e = rel_err(a.cpu().numpy(), b)
        assert e <= TOL_BF16, f"{name} rel err {e:.3e}"


def test_identity_projections_reproduce_plain_sketch():
    # W_Q = W_K = I: the folded table is P itself (fp32, exact products by 1
    # and 0), so the sketch matches the unprojected one bit for bit.
    say("case identity projections")
    k, d = 128, 32
    P, _, _ = _inputs(9, k, d, torch.float32)
    I = torch.eye(d)
    Peff = sa.fold_prototypes(P.cuda(), I.cuda(), I.cuda())
    torch.cuda.synchronize()
    assert torch.equal(Peff.cpu(), P)
