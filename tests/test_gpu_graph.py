"""The sketch step captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must give bitwise the eager results.  The library
records no memset and allocates nothing inside an entry point, so
sa_forward, sa_backward and sa_forward_noalloc (whose purpose is code under
graph capture) can be captured once their outputs and workspaces exist.
Outputs are poisoned with NaN between replays, and unrelated eager work runs
in between, so a replay that skipped or repeated a kernel would show."""

import pytest
import torch

from recommender_ultra_long_amd import sa, synth
from sa_testutil import say

pytestmark = pytest.mark.gpu


def _setup(mass_norm):
    prob = synth.make_inputs([3000, 0, 5000, 77, 1], 1024, 128, "bf16", device="cuda", seed=3,
                             wid=97, with_dS=True, mass_norm=mass_norm)
    B, T, k, d = len(prob.offsets) - 1, prob.total_tokens, 1024, 128
    off = torch.as_tensor(prob.offsets, device="cuda")
    pr = sa.make_problem(B, k, d, T, prob.X.dtype, mass_norm)
    bufs = dict(
        S=torch.empty((B, k, d), device="cuda"), lse=torch.empty((T,), device="cuda"),
        mass=torch.empty((B, k), device="cuda"), dX=torch.empty((T, d), device="cuda"),
        dP=torch.empty((k, d), device="cuda"), S2=torch.empty((B, k, d), device="cuda"),
        wsf=torch.empty(sa.workspace_size(pr, sa.SA_OP_FORWARD), dtype=torch.uint8, device="cuda"),
        wsb=torch.empty(sa.workspace_size(pr, sa.SA_OP_BACKWARD), dtype=torch.uint8,
                        device="cuda"))
    return prob, off, bufs


def _step(prob, off, b):
    sa.sa_forward(off, prob.X, prob.P, prob.mass_norm, S=b["S"], lse=b["lse"], mass=b["mass"],
                  workspace=b["wsf"])
    sa.sa_backward(off, prob.X, prob.P, prob.dS, b["lse"], b["S"], b["mass"], prob.mass_norm,
                   dX=b["dX"], dP=b["dP"], workspace=b["wsb"])
    sa.sa_forward_noalloc(off, prob.X, prob.P, b["S2"], mass_norm=prob.mass_norm)


OUTS = ("S", "lse", "mass", "dX", "dP", "S2")


@pytest.mark.parametrize("mass_norm", [False, True])
def test_step_replayed_from_a_graph_matches_eager(mass_norm):
    prob, off, b = _setup(mass_norm)
    say(f"case graph replay mass_norm={mass_norm}")
    _step(prob, off, b)
    torch.cuda.synchronize()
    ref = {n: b[n].clone() for n in OUTS}
    assert torch.equal(ref["S"], ref["S2"])

    # capture (torch runs the capture on a stream of its own)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(prob, off, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(prob, off, b)
    torch.cuda.synchronize()

    junk = torch.randn(512, 512, device="cuda")
    for r in range(3):
        for n in OUTS:
            b[n].fill_(float("nan"))
        junk = junk @ junk.t() / 512.0            # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for n in OUTS:
            assert torch.equal(b[n], ref[n]), f"replay {r}: {n} differs from the eager result"
        assert sa.sa_get_device_status(b["wsf"]) == sa.SA_OK
        assert sa.sa_get_device_status(b["wsb"]) == sa.SA_OK
