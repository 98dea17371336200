"""The ctypes binding rejects tensors whose dtype, shape, contiguity or device
does not match what the C-ABI reads, before any library call (no GPU needed:
the checks run on host tensors, and the device check comes last)."""

import pytest
import torch

from recommender_ultra_long_amd import sa

B, T, K, D = 2, 10, 8, 32
OFF = torch.tensor([0, 4, 10])


def _x(dtype=torch.bfloat16):
    return torch.zeros(T, D, dtype=dtype)


def _p(dtype=torch.bfloat16, k=K, d=D):
    return torch.zeros(k, d, dtype=dtype)


@pytest.mark.parametrize("X,P,match", [
    (_x(torch.float32), _p(torch.bfloat16), "P must be torch.float32"),
    (_x(torch.bfloat16), _p(torch.float32), "P must be torch.bfloat16"),
    (_x(torch.float16), _p(torch.float16), "X must be one of"),
    (_x(), _p(d=16), "last dimension"),
    (torch.zeros(T, 2 * D, dtype=torch.bfloat16)[:, ::2], _p(), "X must be contiguous"),
    (_x(), torch.zeros(3, K, D, dtype=torch.bfloat16), r"P must be \[k, d\] or \[2, k, d\]"),
    (torch.zeros(T, D, 1, dtype=torch.bfloat16), _p(), r"X must be \[T, d\]"),
])
def test_forward_rejects_mismatched_inputs(X, P, match):
    with pytest.raises(ValueError, match=match):
        sa.sa_forward(OFF, X, P)


def test_forward_rejects_wrong_outputs_and_offsets():
    X, P = _x(), _p()
    with pytest.raises(ValueError, match="S must have shape"):
        sa.sa_forward(OFF, X, P, S=torch.zeros(B, K, D + 1))
    with pytest.raises(ValueError, match="lse must be torch.float32"):
        sa.sa_forward(OFF, X, P, lse=torch.zeros(T, dtype=torch.float64))
    with pytest.raises(ValueError, match="mass must be contiguous"):
        sa.sa_forward(OFF, X, P, mass=torch.zeros(K, B).t())
    with pytest.raises(ValueError, match="offsets must be"):
        sa.sa_forward(torch.tensor([[0, 10]]), X, P)
    with pytest.raises(ValueError, match="offsets must be an integer"):
        sa.sa_forward(OFF.float(), X, P)
    with pytest.raises(ValueError, match="workspace must be torch.uint8"):
        sa.sa_forward(OFF, X, P, workspace=torch.zeros(64))


def test_forward_rejects_host_tensors():
    with pytest.raises(ValueError, match="must be on a GPU"):
        sa.sa_forward(OFF, _x(), _p())


def test_backward_rejects_mismatched_inputs():
    X, P = _x(), _p()
    dS = torch.zeros(B, K, D)
    with pytest.raises(ValueError, match="dS must be torch.float32"):
        sa.sa_backward(OFF, X, P, dS.bfloat16())
    with pytest.raises(ValueError, match="dS must have shape"):
        sa.sa_backward(OFF, X, P, torch.zeros(B, K, D - 1))
    with pytest.raises(ValueError, match="lse must have shape"):
        sa.sa_backward(OFF, X, P, dS, lse=torch.zeros(T + 1))
    with pytest.raises(ValueError, match="S is required"):
        sa.sa_backward(OFF, X, P, dS, mass=torch.zeros(B, K), mass_norm=True)
    with pytest.raises(ValueError, match="dP must have shape"):
        sa.sa_backward(OFF, X, P, dS, dP=torch.zeros(B, K, D))
    with pytest.raises(ValueError, match="dX must be contiguous"):
        sa.sa_backward(OFF, X, P, dS, dX=torch.zeros(D, T).t())
    with pytest.raises(ValueError, match="must be on a GPU"):
        sa.sa_backward(OFF, X, P, dS)


def test_autograd_wrapper_rejects_mixed_dtypes():
    with pytest.raises(ValueError, match="P must be torch.bfloat16"):
        sa.SketchAttention.apply(_x(), _p(torch.float32), OFF, False)


def test_token_wise_rejects_per_user_tables():
    with pytest.raises(ValueError, match="shared"):
        sa.tokenwise_forward(OFF, _x(), torch.zeros(B, K, D, dtype=torch.bfloat16))


def test_other_entry_points_check_their_tensors():
    with pytest.raises(ValueError, match="Wq must have shape"):
        sa.fold_prototypes(_p(), torch.zeros(D, D + 1), torch.zeros(D, D))
    with pytest.raises(ValueError, match="dP_eff must be torch.float32"):
        sa.fold_prototypes_backward(_p(), torch.zeros(D, D), torch.zeros(D, D),
                                    torch.zeros(K, D, dtype=torch.bfloat16))
    e = torch.zeros(T, D, dtype=torch.bfloat16)
    W = (torch.zeros(2 * D, 2 * D), torch.zeros(2 * D, 2 * D), torch.zeros(2 * D, D))
    with pytest.raises(ValueError, match="types must be torch.int32"):
        sa.action_fusion_forward(e, torch.zeros(T, dtype=torch.int64), torch.zeros(8, D), *W)
    with pytest.raises(ValueError, match="W2 must have shape"):
        sa.action_fusion_forward(e, torch.zeros(T, dtype=torch.int32), torch.zeros(8, D),
                                 W[0], W[1], torch.zeros(D, D))
    with pytest.raises(ValueError, match="X must be torch.bfloat16"):
        sa.stca_attention(OFF, torch.zeros(T, 256), torch.tensor([0, 1, 2]), torch.zeros(2, 256),
                          *(torch.zeros(256, 256) for _ in range(3)), 4)
    layer = {k: torch.zeros(s) for k, s in sa._layer_shapes(D).items()}
    bad = dict(layer, W2=torch.zeros(D, D))
    with pytest.raises(ValueError, match=r"layers\[0\]\['W2'\] must have shape"):
        sa.block_forward(OFF, _x(), torch.zeros(K, D), [bad])
    with pytest.raises(ValueError, match="must be on a GPU"):
        sa.block_forward(OFF, _x(), torch.zeros(K, D), [layer])
