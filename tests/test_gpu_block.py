"""GPU parity of the stacked Sketch Attention block (SequenceO1 reading notes,
section 3.3, Eq. (12)-(16)): sa_block_forward / sa_block_backward through the
C-ABI against the float64 oracle (oracle/block.py), with the sketch's
tolerances: max|gpu - ref| / max|ref| per user for the output and dX, over
the tensor for dP0 and every parameter gradient; <= 1e-4 (fp32) and <= 2e-2
(bf16 history and folded tables, fp32 elsewhere)."""

import numpy as np
import pytest
import torch

from oracle.block import block_backward_ref, block_forward_ref
from recommender_ultra_long_amd import sa, synth
from sa_testutil import TOL_BF16, TOL_F32, record, rel_err, say

pytestmark = pytest.mark.gpu

# oracle key -> C-ABI key
KEYMAP = dict(Wq="Wq", Wk="Wk", g1="ln1_g", b1="ln1_b", W1="W1", W3="W3", W2="W2", g2="ln2_g",
              b2="ln2_b")


def _layers(seed, n, d):
    g = torch.Generator().manual_seed(seed)
    s = d ** -0.5
    out = []
    for _ in range(n):
        out.append(dict(
            Wq=torch.randn(d, d, generator=g) * s, Wk=torch.randn(d, d, generator=g) * s,
            ln1_g=1.0 + 0.1 * torch.randn(d, generator=g), ln1_b=0.1 * torch.randn(d, generator=g),
            W1=torch.randn(d, 2 * d, generator=g) * s, W3=torch.randn(d, 2 * d, generator=g) * s,
            W2=torch.randn(2 * d, d, generator=g) * (2 * d) ** -0.5,
            ln2_g=1.0 + 0.1 * torch.randn(d, generator=g), ln2_b=0.1 * torch.randn(d, generator=g)))
    return out


def _run(lengths, k, d, dtype, n_layers, seed):
    prob = synth.make_inputs(lengths, k, d, dtype, device="cuda", seed=seed, wid=400 + seed)
    g = torch.Generator().manual_seed(seed + 1)
    P0 = torch.randn(k, d, generator=g) * d ** -0.5
    layers = _layers(seed + 2, n_layers, d)
    dout = torch.randn(len(lengths), k, d, generator=g)
    off = torch.as_tensor(prob.offsets, device="cuda")
    lay_dev = [{key: v.cuda() for key, v in L.items()} for L in layers]
    out, ws = sa.block_forward(off, prob.X, P0.cuda(), lay_dev)
    dX, dP0, grads = sa.block_backward(off, prob.X, P0.cuda(), lay_dev, dout.cuda(), ws)
    torch.cuda.synchronize()
    ref_layers = [{ok: L[ck].double().numpy() for ok, ck in KEYMAP.items()} for L in layers]
    X64 = synth.to_f64(prob.X)
    return prob, out, dX, dP0, grads, X64, P0.double().numpy(), ref_layers, dout.double().numpy()


@pytest.mark.parametrize("dtype,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("n_layers", [1, 2])
def test_block_forward_backward(dtype, tol, d, n_layers):
    lengths = [300, 0, 77, 1000, 1]
    k = 64 if d < 128 else 96
    say(f"case block dtype={dtype} d={d} k={k} layers={n_layers}")
    prob, out, dX, dP0, grads, X64, P064, ref_layers, dout = _run(lengths, k, d, dtype, n_layers,
                                                                  seed=d + n_layers)
    ref_out, _ = block_forward_ref(prob.offsets, X64, P064, ref_layers)
    rdX, rdP0, rgrads = block_backward_ref(prob.offsets, X64, P064, ref_layers, dout)
    for u in range(len(lengths)):
        e = rel_err(out[u].cpu().numpy(), ref_out[u])
        assert e <= tol, f"user {u}: out rel err {e:.3e}"
        lo, hi = int(prob.offsets[u]), int(prob.offsets[u + 1])
        if hi > lo:
            e = rel_err(dX[lo:hi].cpu().numpy(), rdX[lo:hi])
            assert e <= tol, f"user {u}: dX rel err {e:.3e}"
    e = rel_err(dP0.cpu().numpy(), rdP0)
    assert e <= tol, f"dP0 rel err {e:.3e}"
    for li in range(n_layers):
        for ok, ck in KEYMAP.items():
            e = rel_err(grads[li][ck].cpu().numpy(), rgrads[li][ok])
            assert e <= tol, f"layer {li} d{ck} rel err {e:.3e}"


def test_block_backward_is_deterministic():
    say("case block determinism")
    lengths = [2000, 500, 0, 3000]
    prob = synth.make_inputs(lengths, 128, 128, "bf16", device="cuda", seed=3, wid=450)
    P0 = (torch.randn(128, 128, generator=torch.Generator().manual_seed(4)) / 128 ** 0.5).cuda()
    layers = [{key: v.cuda() for key, v in L.items()} for L in _layers(5, 2, 128)]
    dout = torch.randn(len(lengths), 128, 128, generator=torch.Generator().manual_seed(6)).cuda()
    off = torch.as_tensor(prob.offsets, device="cuda")
    res = []
    for _ in range(2):
        out, ws = sa.block_forward(off, prob.X, P0, layers)
        res.append((out,) + sa.block_backward(off, prob.X, P0, layers, dout, ws)[:2])
    torch.cuda.synchronize()
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


def test_block_two_layers_k1024_long_user():
    """The configuration the benchmark times (k = 1024, d = 128, bf16, two
    layers) with users of 12,000 and 3,000 tokens and an empty one."""
    lengths = [12000, 0, 3000]
    say("case block k=1024 d=128 bf16 2 layers, users 12000/0/3000")
    prob, out, dX, dP0, grads, X64, P064, ref_layers, dout = _run(lengths, 1024, 128, "bf16", 2,
                                                                  seed=31)
    ref_out, _ = block_forward_ref(prob.offsets, X64, P064, ref_layers)
    rdX, rdP0, rgrads = block_backward_ref(prob.offsets, X64, P064, ref_layers, dout)
    worst = {"out": 0.0, "dX": 0.0}
    for u in range(len(lengths)):
        e = rel_err(out[u].cpu().numpy(), ref_out[u])
        assert e <= TOL_BF16, f"user {u}: out rel err {e:.3e}"
        worst["out"] = max(worst["out"], e)
        lo, hi = int(prob.offsets[u]), int(prob.offsets[u + 1])
        if hi > lo:
            e = rel_err(dX[lo:hi].cpu().numpy(), rdX[lo:hi])
            assert e <= TOL_BF16, f"user {u}: dX rel err {e:.3e}"
            worst["dX"] = max(worst["dX"], e)
    worst["dP0"] = rel_err(dP0.cpu().numpy(), rdP0)
    assert worst["dP0"] <= TOL_BF16
    wg = 0.0
    for li in range(2):
        for ok, ck in KEYMAP.items():
            e = rel_err(grads[li][ck].cpu().numpy(), rgrads[li][ok])
            assert e <= TOL_BF16, f"layer {li} d{ck} rel err {e:.3e}"
            wg = max(wg, e)
    record("stacked block, 2 layers, k=1024, users 12000/0/3000", **worst, params=wg)
