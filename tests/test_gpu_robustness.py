"""Robustness of the HIP path against its own buffers and against other work
on the GPU:

* poisoned buffers: every workspace (and every output) is filled with NaN
  bytes before the call; the results must equal, bit for bit, those of a call
  whose workspace and outputs start at zero.  A kernel that reads workspace
  it did not write in the same call, or leaves part of an output unwritten,
  fails this.
* a busy neighbour: the same calls on one stream while another stream keeps
  the GPU busy give bitwise the results of a quiet run (no atomics, no
  dependence on workgroup timing).
"""

import numpy as np
import pytest
import torch

from recommender_ultra_long_amd import sa, synth
from sa_testutil import say

pytestmark = pytest.mark.gpu

POISON = 0xFF     # every byte 0xFF: NaN as fp32 and as bf16


def _ws(nbytes, fill):
    return torch.full((max(int(nbytes), 256),), fill, dtype=torch.uint8, device="cuda")


def _nan_like(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _sketch_calls(prob, per_user=False, token_wise=False, pass_lse=True):
    """Forward then backward with caller-owned outputs and workspaces, each
    filled with `fill` first; returns every output."""
    off = torch.as_tensor(prob.offsets, device="cuda")
    B = len(prob.offsets) - 1
    T, d = prob.X.shape
    k = prob.P.shape[-2]
    mn = prob.mass_norm

    def run(fill):
        filled = (lambda s: _nan_like(s)) if fill == POISON else (
            lambda s: torch.zeros(s, dtype=torch.float32, device="cuda"))
        pr = sa.make_problem(B, k, d, T, prob.X.dtype, mn, per_user, token_wise)
        wsf = _ws(sa.workspace_size(pr, sa.SA_OP_FORWARD), fill)
        wsb = _ws(sa.workspace_size(pr, sa.SA_OP_BACKWARD), fill)
        S = filled((B, k, d))
        if token_wise:
            lse = filled((B, k))
            sa.tokenwise_forward(off, prob.X, prob.P, S=S, lse=lse, workspace=wsf)
            dX, dP = filled((T, d)), filled((k, d))
            sa.tokenwise_backward(off, prob.X, prob.P, prob.dS, S, lse, dX=dX, dP=dP, workspace=wsb)
            out = (S, lse, dX, dP)
        else:
            lse, mass = filled((T,)), filled((B, k))
            sa.sa_forward(off, prob.X, prob.P, mn, S=S, lse=lse, mass=mass, workspace=wsf)
            dX, dP = filled((T, d)), filled(tuple(prob.P.shape))
            sa.sa_backward(off, prob.X, prob.P, prob.dS, lse if pass_lse else None, S, mass, mn,
                           dX=dX, dP=dP, workspace=wsb)
            out = (S, lse, mass, dX, dP)
        torch.cuda.synchronize()
        assert sa.sa_get_device_status(wsf) == sa.SA_OK
        return [t.clone() for t in out]

    return run


def _assert_same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert not torch.isnan(x).any(), f"{what}: output {i} holds NaN"
        assert torch.equal(x, y), f"{what}: output {i} differs"


LENGTHS = [0, 700, 31, 0, 1300, 65, 1]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mass_norm", [False, True])
@pytest.mark.parametrize("pass_lse", [True, False])
def test_sketch_poisoned_workspace_and_outputs(dtype, mass_norm, pass_lse):
    k, d = (300, 128) if dtype == "bf16" else (37, 64)
    say(f"case poison sketch dtype={dtype} mass_norm={mass_norm} pass_lse={pass_lse}")
    prob = synth.make_inputs(LENGTHS, k, d, dtype, device="cuda", seed=2, wid=700, with_dS=True,
                             mass_norm=mass_norm)
    run = _sketch_calls(prob, pass_lse=pass_lse)
    _assert_same(run(POISON), run(0), "poisoned vs clean")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_per_user_and_token_wise_poisoned(dtype):
    k, d = 256, 128
    say(f"case poison per-user / token-wise dtype={dtype}")
    prob = synth.make_inputs(LENGTHS, k, d, dtype, device="cuda", seed=3, wid=701, with_dS=True,
                             mass_norm=True, per_user_p=True)
    run = _sketch_calls(prob, per_user=True)
    _assert_same(run(POISON), run(0), "per-user tables")
    prob = synth.make_inputs([40, 0, 900, 3], k, d, dtype, device="cuda", seed=4, wid=702,
                             with_dS=True)
    run = _sketch_calls(prob, token_wise=True)
    _assert_same(run(POISON), run(0), "token-wise")


def test_fold_block_action_stca_poisoned():
    g = torch.Generator().manual_seed(0)
    d, k = 128, 256
    P = (torch.randn(k, d, generator=g) / d ** 0.5).to(torch.bfloat16).cuda()
    Wq, Wk = (torch.randn(d, d, generator=g) / d ** 0.5).cuda(), (torch.randn(d, d, generator=g) / d ** 0.5).cuda()
    dPe = torch.randn(k, d, generator=g).cuda()
    nb = int(sa.load().sa_fold_workspace_size(k, d))
    say("case poison fold backward")
    outs = [sa.fold_prototypes_backward(P, Wq, Wk, dPe, workspace=_ws(nb, f)) for f in (POISON, 0)]
    _assert_same(outs[0], outs[1], "fold backward")

    say("case poison stacked block")
    lengths = [300, 0, 1200, 7]
    prob = synth.make_inputs(lengths, k, d, "bf16", device="cuda", seed=5, wid=703)
    s = d ** -0.5
    layers = [dict(Wq=torch.randn(d, d, generator=g) * s, Wk=torch.randn(d, d, generator=g) * s,
                   ln1_g=1 + 0.1 * torch.randn(d, generator=g), ln1_b=0.1 * torch.randn(d, generator=g),
                   W1=torch.randn(d, 2 * d, generator=g) * s, W3=torch.randn(d, 2 * d, generator=g) * s,
                   W2=torch.randn(2 * d, d, generator=g) * (2 * d) ** -0.5,
                   ln2_g=1 + 0.1 * torch.randn(d, generator=g), ln2_b=0.1 * torch.randn(d, generator=g))
              for _ in range(2)]
    layers = [{n: t.cuda() for n, t in L.items()} for L in layers]
    P0 = (torch.randn(k, d, generator=g) * s).cuda()
    dout = torch.randn(len(lengths), k, d, generator=g).cuda()
    off = torch.as_tensor(prob.offsets, device="cuda")
    res = []
    for f in (POISON, 0):
        ws = sa.block_workspace(len(lengths) + 1, k, d, prob.total_tokens, prob.X.dtype, 2, "cuda")
        ws.fill_(f)
        out, ws = sa.block_forward(off, prob.X, P0, layers, workspace=ws)
        dX, dP0, grads = sa.block_backward(off, prob.X, P0, layers, dout, ws)
        torch.cuda.synchronize()
        res.append([out.clone(), dX.clone(), dP0.clone()] + [gr[n].clone() for gr in grads
                                                             for n in sa.BLOCK_LAYER_KEYS])
    _assert_same(res[0], res[1], "stacked block")

    say("case poison action fusion")
    T = 3000
    e = torch.randn(T, d, generator=g).to(torch.bfloat16).cuda()
    types = torch.randint(0, 8, (T,), generator=g, dtype=torch.int32).cuda()
    A = (torch.randn(8, d, generator=g) * 0.7).cuda()
    sw = (2 * d) ** -0.5
    W1, W3 = (torch.randn(2 * d, 2 * d, generator=g) * sw).cuda(), (torch.randn(2 * d, 2 * d, generator=g) * sw).cuda()
    W2 = (torch.randn(2 * d, d, generator=g) * sw).cuda()
    dx = torch.randn(T, d, generator=g).cuda()
    lib = sa.load()
    res = []
    for f in (POISON, 0):
        wf = _ws(lib.sa_action_fusion_workspace_size(d, sa.SA_BF16, T, 8, 0), f)
        wb = _ws(lib.sa_action_fusion_workspace_size(d, sa.SA_BF16, T, 8, 1), f)
        x = sa.action_fusion_forward(e, types, A, W1, W3, W2, workspace=wf)
        grads = sa.action_fusion_backward(e, types, A, W1, W3, W2, dx, workspace=wb)
        torch.cuda.synchronize()
        res.append([x.float()] + [t.clone() for t in grads])
    _assert_same(res[0], res[1], "action fusion")

    say("case poison stca")
    D, h = 512, 8
    x_off = torch.tensor([0, 500, 500, 1533], device="cuda")
    t_off = torch.tensor([0, 3, 5, 9], device="cuda")
    X = torch.randn(1533, D, generator=g).to(torch.bfloat16).cuda()
    Q = torch.randn(9, D, generator=g).cuda()
    Ws = [(torch.randn(D, D, generator=g) * D ** -0.5).cuda() for _ in range(3)]
    nb = int(lib.sa_stca_workspace_size(D, h, 9))
    res = []
    for f in (POISON, 0):
        o, lse = sa.stca_attention(x_off, X, t_off, Q, *Ws, h, o=_nan_like((9, D)),
                                   lse=_nan_like((9, h)), workspace=_ws(nb, f))
        torch.cuda.synchronize()
        res.append([o.clone(), torch.nan_to_num(lse, neginf=-1e30)])
    _assert_same(res[0], res[1], "stca")


def test_bitwise_equal_with_a_busy_neighbour_stream():
    """Forward + backward on one stream while a second stream runs large
    matrix products: bitwise the results of a quiet run."""
    say("case busy neighbour stream")
    prob = synth.make_inputs([20000, 17, 9000, 0, 3000], 1024, 128, "bf16", device="cuda", seed=6,
                             wid=704, with_dS=True, mass_norm=True)
    off = torch.as_tensor(prob.offsets, device="cuda")

    def step():
        S, lse, mass = sa.sa_forward(off, prob.X, prob.P, True)
        dX, dP = sa.sa_backward(off, prob.X, prob.P, prob.dS, lse, S, mass, True)
        return S, lse, mass, dX, dP

    quiet = [t.clone() for t in step()]
    torch.cuda.synchronize()
    busy = torch.cuda.Stream()
    a = torch.randn(4096, 4096, device="cuda")
    main = torch.cuda.current_stream()
    for trial in range(3):
        with torch.cuda.stream(busy):
            acc = a
            for _ in range(12):
                acc = torch.tanh(acc @ a * 1e-2)
        loud = step()            # queued while the neighbour's products run
        main.synchronize()
        busy.synchronize()
        for i, (x, y) in enumerate(zip(quiet, loud)):
            assert torch.equal(x, y), f"trial {trial}: output {i} differs next to a busy stream"
    assert np.isfinite(float(acc.sum()))
