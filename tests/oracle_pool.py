"""Runs the float64 oracle over many users at once in worker processes.

Test infrastructure.  Every user of a Sketch Attention batch is independent,
so a full-size workload is checked user by user: each worker regenerates the
user's inputs from the seeded recipe (``synth.GenSpec``, numpy only) and runs
``oracle.sa_ref`` on them, single-threaded; the parent process compares the
results with the GPU's.  The workers never touch the GPU or the HIP library.
"""

from __future__ import annotations

import contextlib
import multiprocessing as mp
import os

import numpy as np

_WORKER_ENV = {"OPENBLAS_NUM_THREADS": "1", "OMP_NUM_THREADS": "1", "MKL_NUM_THREADS": "1"}


def n_workers():
    """At most 16 worker processes (one GPU's share of the host cores)."""
    return max(1, min(16, os.cpu_count() or 1))


@contextlib.contextmanager
def pool(workers=None):
    """A spawn-context process pool whose workers run BLAS single-threaded
    (the environment is read when a worker starts)."""
    saved = {k: os.environ.get(k) for k in _WORKER_ENV}
    os.environ.update(_WORKER_ENV)
    try:
        p = mp.get_context("spawn").Pool(workers or n_workers())
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    try:
        yield p
    finally:
        p.terminate()
        p.join()


def _inputs(spec, u, n):
    X = spec.rows(u, n).astype(np.float64)
    P = spec.table(u if spec.per_user_p else None).astype(np.float64)
    return X, P


def checksum(X):
    """Sum and sum of squares of a user's rows, float64."""
    X = np.asarray(X, dtype=np.float64)
    return float(X.sum()), float((X * X).sum())


def forward_user(job):
    """job = (spec, u, n, mass_norm) -> (u, S [k, d], lse [n], mass [k],
    checksum of the rows)."""
    from oracle.sa_ref import sa_forward_ref

    spec, u, n, mass_norm = job
    X, P = _inputs(spec, u, n)
    S, lse, mass = sa_forward_ref(np.array([0, n]), X, P, mass_norm)
    return u, S[0], lse, mass[0], checksum(X)


def backward_user(job):
    """job = (spec, u, n, mass_norm) -> (u, dX [n, d], dP_u [k, d], checksum
    of the rows): the gradients of sum(dS_u * S_u) for user u alone."""
    from oracle.sa_ref import sa_backward_ref

    spec, u, n, mass_norm = job
    X, P = _inputs(spec, u, n)
    dS = spec.dS(u).astype(np.float64)[None]
    dX, dP = sa_backward_ref(np.array([0, n]), X, P, dS, mass_norm)
    return u, dX, dP, checksum(X)
