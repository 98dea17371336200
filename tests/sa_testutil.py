"""Shared helpers for the GPU parity tests: run the HIP path and the float64
oracle on the same seeded inputs and compare them."""

import sys

import numpy as np
import torch

from oracle.sa_ref import sa_backward_ref, sa_forward_ref
from recommender_ultra_long_amd import sa, synth

TOL_F32 = 1e-4      # max|gpu - ref| / max|ref|, fp32 path
TOL_BF16 = 2e-2     # same measure, bf16 in / fp32 accumulate
TOL_LSE_ABS = 1e-3  # per-token log-sum-exp, absolute


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# Achieved parity errors of the full-size cases, printed at the end of the
# test session (tests/conftest.py), so that a passing run still shows them.
PARITY_LOG = []


def record(case, **errors):
    line = case + ": " + ", ".join(f"{k} {v:.2e}" for k, v in errors.items())
    PARITY_LOG.append(line)
    say("  " + line)


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(gpu - ref)) if gpu.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def gpu_forward(prob, mass_norm=None):
    mn = prob.mass_norm if mass_norm is None else mass_norm
    off = torch.as_tensor(prob.offsets, device="cuda")
    S, lse, mass = sa.sa_forward(off, prob.X, prob.P, mn)
    torch.cuda.synchronize()
    return S, lse, mass


def check_forward_users(prob, S, lse, mass, users, tol, mass_norm=None):
    """Oracle on the listed users only (each user is independent)."""
    mn = prob.mass_norm if mass_norm is None else mass_norm
    P64 = synth.to_f64(prob.P)
    worst = 0.0
    for u in users:
        lo, hi = int(prob.offsets[u]), int(prob.offsets[u + 1])
        X64 = synth.to_f64(prob.X[lo:hi])
        Pu = P64[u] if P64.ndim == 3 else P64          # one table per user, or shared
        Sr, lr, mr = sa_forward_ref(np.array([0, hi - lo]), X64, Pu, mn)
        e = rel_err(S[u].cpu().numpy(), Sr[0])
        assert e <= tol, f"user {u} (n={hi - lo}): S rel err {e:.3e} > {tol}"
        em = rel_err(mass[u].cpu().numpy(), mr[0])
        assert em <= tol, f"user {u}: mass rel err {em:.3e}"
        if hi > lo:
            el = float(np.max(np.abs(lse[lo:hi].cpu().numpy().astype(np.float64) - lr)))
            assert el <= TOL_LSE_ABS, f"user {u}: lse abs err {el:.3e}"
        worst = max(worst, e)
    return worst


def _gpu_checksum(X):
    x = X.double()
    return float(x.sum().item()), float((x * x).sum().item())


def _same_rows(prob, u, lo, hi, ref_sum):
    """The rows a worker regenerated are the rows the GPU consumed."""
    got = _gpu_checksum(prob.X[lo:hi])
    for a, b in zip(got, ref_sum):
        assert abs(a - b) <= 1e-9 * max(1.0, abs(b)), f"user {u}: regenerated rows differ"


def check_forward_all_users(prob, S, lse, mass, tol, mass_norm=None):
    """Every user of the batch against the oracle, run in worker processes
    that regenerate each user's rows from the seeded recipe.  Returns the
    worst (S, mass, lse) errors."""
    from oracle_pool import forward_user, pool

    mn = prob.mass_norm if mass_norm is None else mass_norm
    B = len(prob.offsets) - 1
    lens = np.diff(prob.offsets)
    jobs = [(prob.gen, u, int(lens[u]), mn) for u in range(B)]
    # longest users first, so the pool drains evenly
    jobs.sort(key=lambda j: -j[2])
    worst = [0.0, 0.0, 0.0]
    Sg, mg = S.cpu().numpy(), mass.cpu().numpy()
    with pool() as p:
        for done, (u, Sr, lr, mr, cs) in enumerate(p.imap_unordered(forward_user, jobs), 1):
            if done % 32 == 0:
                say(f"  oracle: {done}/{B} users checked")
            lo, hi = int(prob.offsets[u]), int(prob.offsets[u + 1])
            _same_rows(prob, u, lo, hi, cs)
            e = rel_err(Sg[u], Sr)
            assert e <= tol, f"user {u} (n={hi - lo}): S rel err {e:.3e} > {tol}"
            em = rel_err(mg[u], mr)
            assert em <= tol, f"user {u}: mass rel err {em:.3e}"
            el = 0.0
            if hi > lo:
                el = float(np.max(np.abs(lse[lo:hi].cpu().numpy().astype(np.float64) - lr)))
                assert el <= TOL_LSE_ABS, f"user {u}: lse abs err {el:.3e}"
            worst = [max(worst[0], e), max(worst[1], em), max(worst[2], el)]
    return worst


def check_backward_all_users(prob, dX, dP, tol):
    """dX of every user, and dP over the whole batch (the sum of the oracle's
    per-user dP, since the table is shared), against the oracle in worker
    processes.  Returns the worst (dX, dP) errors."""
    from oracle_pool import backward_user, pool

    B = len(prob.offsets) - 1
    lens = np.diff(prob.offsets)
    jobs = [(prob.gen, u, int(lens[u]), prob.mass_norm) for u in range(B)]
    jobs.sort(key=lambda j: -j[2])
    dP_ref = np.zeros(tuple(dP.shape))
    worst_dx = 0.0
    with pool() as p:
        for done, (u, dXr, dPu, cs) in enumerate(p.imap_unordered(backward_user, jobs), 1):
            if done % 8 == 0:
                say(f"  oracle: {done}/{B} users checked")
            lo, hi = int(prob.offsets[u]), int(prob.offsets[u + 1])
            _same_rows(prob, u, lo, hi, cs)
            if dP_ref.ndim == 3:
                dP_ref[u] = dPu
            else:
                dP_ref += dPu
            if hi > lo:
                e = rel_err(dX[lo:hi].cpu().numpy(), dXr)
                assert e <= tol, f"user {u} (n={hi - lo}): dX rel err {e:.3e} > {tol}"
                worst_dx = max(worst_dx, e)
    edp = rel_err(dP.cpu().numpy(), dP_ref)
    assert edp <= tol, f"dP rel err {edp:.3e} > {tol}"
    return worst_dx, edp
