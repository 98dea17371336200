"""GPU parity of the forward pass against the float64 oracle.

Every case calls the C-ABI through the ctypes binding and compares element by
element with oracle.sa_ref on the same seeded inputs.  Tolerances: max
abs error / max |ref| per user <= 1e-4 (fp32 path) and <= 2e-2 (bf16 inputs,
fp32 accumulation); per-token lse within 1e-3 absolute.
"""

import numpy as np
import pytest
import torch

from oracle.sa_ref import sa_forward_ref
from recommender_ultra_long_amd import sa, synth
from sa_testutil import (TOL_BF16, TOL_F32, check_forward_all_users, check_forward_users,
                         gpu_forward, record, rel_err, say)

pytestmark = pytest.mark.gpu


def _small(lengths, k, d, dtype, seed=0, mass_norm=False, p_std=None, x_kind="normal"):
    return synth.make_inputs(lengths, k, d, dtype, device="cuda", seed=seed, wid=90 + seed,
                             x_kind=x_kind, p_std=p_std, mass_norm=mass_norm)


def test_fp32_workload_n4096_k64_d32():
    prob = synth.make_workload("fp32_n4096_k64_d32", device="cuda")
    say("case fp32_n4096_k64_d32")
    S, lse, mass = gpu_forward(prob)
    eS, em, el = check_forward_all_users(prob, S, lse, mass, TOL_F32)
    record("fp32_n4096_k64_d32", S=eS, mass=em, lse_abs=el)


@pytest.mark.parametrize("dtype,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mass_norm", [False, True])
def test_ragged_edge_lengths(dtype, tol, d, mass_norm):
    # empty users (first, middle, last), single tokens, tile-1/tile/tile+1,
    # and one longer user spanning several segments.
    lengths = [0, 1, 31, 32, 33, 0, 64, 65, 1000, 3, 0]
    for k in (1, 37, 256, 300):
        prob = _small(lengths, k, d, dtype, seed=k, mass_norm=mass_norm)
        say(f"case ragged_edges dtype={dtype} d={d} k={k} mass_norm={mass_norm}")
        S, lse, mass = gpu_forward(prob)
        check_forward_users(prob, S, lse, mass, range(len(lengths)), tol)
        for u in (0, 5, 10):
            assert torch.all(S[u] == 0) and torch.all(mass[u] == 0)


@pytest.mark.parametrize("k,mass_norm,per_user", [(1024, False, False), (1024, True, False),
                                                  (1024, True, True), (256, True, False)])
def test_many_short_users_stale_workspace(k, mass_norm, per_user):
    """300 short users (up to 200 tokens).  k=1024: 64 segments of about 470
    tokens, users outnumber them four to one, so a user inside one segment
    has its row of S written by the aggregation pass and skipped by the
    reduction; k=256: 256 segments, every row goes through a partial.  About
    one user per segment boundary crosses it; three users are empty.  The
    workspace starts as all-ones bytes (NaN as float32), so a row of S or
    mass taken from a partial that this call did not write shows."""
    rng = np.random.default_rng(11)
    lengths = rng.integers(0, 200, size=300)
    lengths[[0, 7, 299]] = 0
    prob = synth.make_inputs([int(x) for x in lengths], k, 64, "bf16", device="cuda", seed=11,
                             wid=101, mass_norm=mass_norm, per_user_p=per_user)
    pr = sa.make_problem(len(lengths), k, 64, prob.total_tokens, sa.SA_BF16, mass_norm,
                         per_user)
    ws = torch.full((sa.workspace_size(pr, sa.SA_OP_FORWARD),), 255, dtype=torch.uint8,
                    device="cuda")
    off = torch.as_tensor(prob.offsets, device="cuda")
    say(f"case many_short_users k={k} mass_norm={mass_norm} per_user={per_user}")
    S, lse, mass = sa.sa_forward(off, prob.X, prob.P, mass_norm, workspace=ws)
    torch.cuda.synchronize()
    assert sa.sa_get_device_status(ws) == sa.SA_OK
    assert bool(torch.isfinite(S).all()) and bool(torch.isfinite(mass).all())
    check_forward_users(prob, S, lse, mass, range(len(lengths)), TOL_BF16)
    for u in (0, 7, 299):
        assert torch.all(S[u] == 0) and torch.all(mass[u] == 0)


@pytest.mark.parametrize("dtype,mass_norm", [("bf16", False), ("bf16", True), ("f32", True)])
def test_three_thousand_users(dtype, mass_norm):
    """3000 users of 0-40 tokens at k=256, d=32: each block row of the
    reduction walks about 190 users, three 64-user votes, and with bf16 most
    rows come straight from the aggregation pass (users outnumber the 256
    segments four to one); the fp32 path reduces every user."""
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(0, 41, size=3000)]
    lengths[0] = lengths[1500] = lengths[2999] = 0
    prob = synth.make_inputs(lengths, 256, 32, dtype, device="cuda", seed=31, wid=131,
                             mass_norm=mass_norm)
    say(f"case 3000 users dtype={dtype} mass_norm={mass_norm}")
    S, lse, mass = gpu_forward(prob)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    worst = check_forward_users(prob, S, lse, mass, range(len(lengths)), tol)
    for u in (0, 1500, 2999):
        assert torch.all(S[u] == 0) and torch.all(mass[u] == 0)
    say(f"3000 users dtype={dtype} mass_norm={mass_norm}: worst S rel err {worst:.2e}")


@pytest.mark.parametrize("dtype,tol", [("f32", TOL_F32), ("bf16", TOL_BF16)])
def test_sharp_logits_exercise_max_shift(dtype, tol):
    # P scaled so that affinities reach |z| ~ 30: exp without the max shift
    # would overflow in fp32 for the larger ones.
    prob = _small([500, 77], 96, 64, dtype, seed=3, p_std=12.0)
    say(f"case sharp dtype={dtype}")
    S, lse, mass = gpu_forward(prob)
    assert float(lse.abs().max()) > 20.0
    check_forward_users(prob, S, lse, mass, [0, 1], tol)


@pytest.mark.parametrize("per_user", [False, True])
def test_bf16_stats_reference_overflow_takes_exact_path(per_user):
    # The bf16 statistics pass keeps each token's first-tile maximum as a fixed
    # reference; a later affinity more than 128 / alpha above it (here ~800
    # against ~0, with 128 / alpha ~ 710 at d = 64) overflows the fast sum and
    # the block redoes its pass with the running maximum.
    prob = _small([300, 45, 0, 200], 300, 64, "bf16", seed=21)
    X = prob.X.float()
    P = prob.P.float().clone()
    P[:32] *= 0.01                                   # the first tile: z ~ 0
    for j, t in ((200, 7), (299, 320)):              # one huge affinity per chosen token
        P[j] = 100.0 * X[t] / X[t].norm()
    if per_user:
        P = P.unsqueeze(0).repeat(4, 1, 1)
        P[2:] *= -1.0                                # users 2 and 3: a different table
    prob.P = P.to(torch.bfloat16)
    say(f"case stats overflow per_user={per_user}")
    S, lse, mass = gpu_forward(prob)
    assert float(lse.max()) > 90.0                   # z / sqrt(d) of the aligned tokens
    assert bool(torch.isfinite(lse).all()) and bool(torch.isfinite(S).all())
    check_forward_users(prob, S, lse, mass, [0, 1, 2, 3], TOL_BF16)


@pytest.mark.parametrize("k", [512, 1000, 1024, 2048])
def test_bf16_large_k(k):
    prob = _small([4000, 2500, 1], k, 128, "bf16", seed=k)
    say(f"case bf16 k={k}")
    S, lse, mass = gpu_forward(prob)
    check_forward_users(prob, S, lse, mass, [0, 1, 2], TOL_BF16)


def test_bf16_workload_n100k_k1024_d128():
    prob = synth.make_workload("bf16_n100k_k1024_d128", device="cuda")
    say("case bf16_n100k_k1024_d128")
    S, lse, mass = gpu_forward(prob)
    eS, em, el = check_forward_all_users(prob, S, lse, mass, TOL_BF16)
    record("bf16_n100k_k1024_d128", S=eS, mass=em, lse_abs=el)


def test_ragged64_massnorm_every_user():
    """The 64-user mass-normalised batch: every user against the oracle."""
    prob = synth.make_workload("ragged64_k1024_massnorm", device="cuda")
    say(f"case ragged64_k1024_massnorm T={prob.total_tokens}")
    S, lse, mass = gpu_forward(prob)
    eS, em, el = check_forward_all_users(prob, S, lse, mass, TOL_BF16)
    record("ragged64_k1024_massnorm, all 64 users", S=eS, mass=em, lse_abs=el)


def test_ragged256_lognormal_every_user():
    """The 256-user lognormal batch (k = 512, item + action rows): every user
    against the oracle, plus a property that holds at any size: each user's
    masses add up to its token count (the columns of A sum to one)."""
    prob = synth.make_workload("ragged256_lognormal_k512", device="cuda")
    say(f"case ragged256_lognormal_k512 T={prob.total_tokens}")
    S, lse, mass = gpu_forward(prob)
    lens = np.diff(prob.offsets)
    tot = mass.double().sum(dim=1).cpu().numpy()
    np.testing.assert_allclose(tot, lens, rtol=1e-3)
    eS, em, el = check_forward_all_users(prob, S, lse, mass, TOL_BF16)
    record("ragged256_lognormal_k512, all 256 users", S=eS, mass=em, lse_abs=el)


def test_sum_over_prototypes_is_sum_of_tokens():
    prob = _small([3000, 20, 700], 1024, 128, "bf16", seed=11)
    S, _, _ = gpu_forward(prob)
    for u in range(3):
        lo, hi = int(prob.offsets[u]), int(prob.offsets[u + 1])
        ref = synth.to_f64(prob.X[lo:hi]).sum(axis=0)
        got = S[u].double().sum(dim=0).cpu().numpy()
        assert rel_err(got, ref) < 2e-2


def test_bitwise_deterministic():
    prob = _small([5000, 17, 12000], 1024, 128, "bf16", seed=5, mass_norm=True)
    out1 = gpu_forward(prob)
    for _ in range(3):
        out2 = gpu_forward(prob)
        for a, b in zip(out1, out2):
            assert torch.equal(a, b)


def test_token_permutation_invariance():
    prob = _small([4096], 256, 128, "bf16", seed=6)
    S1, _, _ = gpu_forward(prob)
    perm = torch.randperm(4096, generator=torch.Generator().manual_seed(0)).cuda()
    prob.X = prob.X[perm].contiguous()
    S2, _, _ = gpu_forward(prob)
    assert rel_err(S2.cpu().numpy(), S1.cpu().numpy()) < 2e-2


def test_bad_offsets_flagged_on_device():
    prob = _small([50, 50], 64, 32, "f32", seed=7)
    bad = torch.tensor([0, 70, 40], dtype=torch.int64, device="cuda")   # decreasing
    ws = torch.zeros(sa.workspace_size(sa.make_problem(2, 64, 32, 100, sa.SA_F32), 0),
                     dtype=torch.uint8, device="cuda")
    sa.sa_forward(bad, prob.X, prob.P, workspace=ws)
    assert sa.sa_get_device_status(ws) == sa.SA_ERR_BAD_OFFSETS
    good = torch.tensor([0, 50, 100], dtype=torch.int64, device="cuda")
    sa.sa_forward(good, prob.X, prob.P, workspace=ws)
    assert sa.sa_get_device_status(ws) == sa.SA_OK


def test_autograd_wrapper_forward_matches():
    prob = _small([300, 200], 64, 64, "f32", seed=8)
    off = torch.as_tensor(prob.offsets, device="cuda")
    S = sa.SketchAttention.apply(prob.X, prob.P, off, False)
    S2, _, _ = gpu_forward(prob)
    assert torch.equal(S, S2)


@pytest.mark.parametrize("mass_norm", [False, True])
@pytest.mark.parametrize("k,d", [(1024, 128), (300, 64), (2048, 32), (37, 128)])
def test_single_pass_and_two_pass_forward_agree(monkeypatch, k, d, mass_norm):
    """The single-pass forward (statistics exchanged between the workgroups
    of a segment) and the two-pass forward (statistics pass first) against
    the oracle and against each other; the exchange reports no timeout."""
    lengths = [0, 1, 31, 33, 4000, 0, 700, 65]
    prob = _small(lengths, k, d, "bf16", seed=k + d, mass_norm=mass_norm)
    off = torch.as_tensor(prob.offsets, device="cuda")
    say(f"case single vs two pass k={k} d={d} mass_norm={mass_norm}")
    pr = sa.make_problem(len(lengths), k, d, prob.total_tokens, sa.SA_BF16, mass_norm)
    ws = torch.empty(sa.workspace_size(pr, sa.SA_OP_FORWARD), dtype=torch.uint8, device="cuda")
    monkeypatch.setenv("SA_FORWARD_PATH", "single_pass")
    t = sa.KernelTimer()
    one = [x.clone() for x in sa.sa_forward(off, prob.X, prob.P, mass_norm, workspace=ws, timer=t)]
    assert sa.sa_get_device_status(ws) == sa.SA_OK
    assert [n for n, _ in t.times()] == ["sa_fused_clear", "sa_fused_bf16", "sa_reduce"]
    monkeypatch.delenv("SA_FORWARD_PATH")
    two = [x.clone() for x in sa.sa_forward(off, prob.X, prob.P, mass_norm, workspace=ws)]
    torch.cuda.synchronize()
    check_forward_users(prob, *one, range(len(lengths)), TOL_BF16)
    check_forward_users(prob, *two, range(len(lengths)), TOL_BF16)
    # same arithmetic up to the order of the per-token statistics merge
    assert float((one[1] - two[1]).abs().max()) < 1e-4
    for a, b in zip(one, two):
        assert rel_err(a.cpu().numpy(), b.cpu().numpy()) < 1e-2
