"""GPU parity of the action-side SwiGLU fusion (SequenceO1 reading notes,
section 3.6, Eq. (20)) through the C-ABI against the float64 oracle
(oracle/action_fusion.py): max|gpu - ref| / max|ref| over each tensor,
<= 1e-4 for fp32 histories and <= 2e-2 for bf16 ones (bf16 products on the
matrix cores, and x rounded to bf16)."""

import numpy as np
import pytest
import torch

from oracle.action_fusion import action_fusion_backward_ref, action_fusion_ref
from recommender_ultra_long_amd import sa
from sa_testutil import TOL_BF16, TOL_F32, rel_err, say

pytestmark = pytest.mark.gpu


def _inputs(seed, T, d, n_types, dtype):
    g = torch.Generator().manual_seed(seed)
    e = torch.randn(T, d, generator=g).to(dtype)
    types = torch.randint(0, n_types, (T,), generator=g, dtype=torch.int32)
    A = torch.randn(n_types, d, generator=g) * 0.7
    s = (2 * d) ** -0.5
    W1 = torch.randn(2 * d, 2 * d, generator=g) * s
    W3 = torch.randn(2 * d, 2 * d, generator=g) * s
    W2 = torch.randn(2 * d, d, generator=g) * s
    return e, types, A, W1, W3, W2


@pytest.mark.parametrize("dtype,tol", [(torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("T", [1, 1000, 4133])
def test_action_fusion_forward_backward(dtype, tol, d, T):
    n_types = 8
    say(f"case action fusion dtype={dtype} d={d} T={T}")
    e, types, A, W1, W3, W2 = _inputs(T + d, T, d, n_types, dtype)
    dx = torch.randn(T, d, generator=torch.Generator().manual_seed(T))
    dev = [t.cuda() for t in (e, types, A, W1, W3, W2)]
    x = sa.action_fusion_forward(*dev)
    grads = sa.action_fusion_backward(*dev, dx.cuda())
    torch.cuda.synchronize()
    e64 = e.double().numpy()
    ref = action_fusion_ref(e64, types.numpy(), A.double().numpy(), W1.double().numpy(),
                            W3.double().numpy(), W2.double().numpy())
    ex = rel_err(x.double().cpu().numpy(), ref)
    assert ex <= tol, f"x rel err {ex:.3e}"
    rg = action_fusion_backward_ref(e64, types.numpy(), A.double().numpy(), W1.double().numpy(),
                                    W3.double().numpy(), W2.double().numpy(), dx.double().numpy())
    for name, a, b in zip(("de", "dA", "dW1", "dW3", "dW2"), grads, rg):
        eg = rel_err(a.cpu().numpy(), b)
        # fp32 histories: fp32 throughout; bf16 histories: the backward's
        # products take bf16 operands with fp32 accumulation
        assert eg <= tol, f"{name} rel err {eg:.3e}"


def test_action_fusion_one_type_equals_shared_row():
    # with one action type every event sees the same action row
    say("case action fusion single type")
    e, types, A, W1, W3, W2 = _inputs(1, 500, 64, 1, torch.bfloat16)
    x = sa.action_fusion_forward(*(t.cuda() for t in (e, types, A, W1, W3, W2)))
    torch.cuda.synchronize()
    ref = action_fusion_ref(e.double().numpy(), np.zeros(500, dtype=np.int64), A.double().numpy(),
                            W1.double().numpy(), W3.double().numpy(), W2.double().numpy())
    assert rel_err(x.double().cpu().numpy(), ref) <= TOL_BF16


def test_action_fusion_backward_is_deterministic():
    # the weight gradients are split over the events and summed in slice
    # order: two calls agree bit for bit
    say("case action fusion determinism")
    e, types, A, W1, W3, W2 = _inputs(3, 40000, 128, 8, torch.bfloat16)
    dx = torch.randn(40000, 128, generator=torch.Generator().manual_seed(4))
    dev = [t.cuda() for t in (e, types, A, W1, W3, W2)]
    g1 = sa.action_fusion_backward(*dev, dx.cuda())
    g2 = sa.action_fusion_backward(*dev, dx.cuda())
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("n_types", [1, 16])
@pytest.mark.parametrize("dtype,tol", [(torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)])
def test_action_fusion_backward_type_counts(n_types, dtype, tol):
    # the per-type sums behind dA and the action rows of dW1, dW3, at one type
    # and at the largest table (16 types), on a ragged event count
    say(f"case action fusion backward n_types={n_types} dtype={dtype}")
    d, T = 64, 2077
    e, types, A, W1, W3, W2 = _inputs(50 + n_types, T, d, n_types, dtype)
    dx = torch.randn(T, d, generator=torch.Generator().manual_seed(n_types))
    grads = sa.action_fusion_backward(*(t.cuda() for t in (e, types, A, W1, W3, W2)), dx.cuda())
    torch.cuda.synchronize()
    rg = action_fusion_backward_ref(e.double().numpy(), types.numpy(), A.double().numpy(),
                                    W1.double().numpy(), W3.double().numpy(), W2.double().numpy(),
                                    dx.double().numpy())
    for name, a, b in zip(("de", "dA", "dW1", "dW3", "dW2"), grads, rg):
        eg = rel_err(a.cpu().numpy(), b)
        assert eg <= tol, f"{name} rel err {eg:.3e}"
