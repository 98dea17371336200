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
        Sr, lr, mr = sa_forward_ref(np.array([0, hi - lo]), X64, P64, mn)
        e = rel_err(S[u].cpu().numpy(), Sr[0])
        assert e <= tol, f"user {u} (n={hi - lo}): S rel err {e:.3e} > {tol}"
        em = rel_err(mass[u].cpu().numpy(), mr[0])
        assert em <= tol, f"user {u}: mass rel err {em:.3e}"
        if hi > lo:
            el = float(np.max(np.abs(lse[lo:hi].cpu().numpy().astype(np.float64) - lr)))
            assert el <= TOL_LSE_ABS, f"user {u}: lse abs err {el:.3e}"
        worst = max(worst, e)
    return worst
