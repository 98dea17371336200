"""Seeded synthetic inputs for Sketch Attention workloads.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic, so both the HIP path and the CPU oracle may consume
what it produces.

Workload shapes follow the SequenceO1 pages: histories of up to 100K events
(reading notes section 2.1), an average of 85K events at 100K truncation
(Fig. 1(c) discussion of the paper's HTML page), k = 512-1024 prototypes of
width d = 128 (reading notes section 5.4 and Table 2), and events built from an
item embedding plus an action-type embedding (reading notes Eq. (20); the
additive form here is a stand-in for the SwiGLU fusion).

Conventions
  * Every tensor comes from numpy's PCG64 seeded with
    SeedSequence(seed, spawn_key=(workload id, tensor tag, index)), where the
    index is the user for per-user tensors (history rows, action ids, dS, a
    per-user prototype table) and 0 for shared ones.  Any user's rows can be
    regenerated on the host alone, without the rest of the batch and without
    a GPU.
  * N(0, s2) means variance s2 (so P ~ N(0, 1/d) has standard deviation
    d**-0.5).  Samples are drawn in float64, cast to float32, then rounded
    to bfloat16 (round to nearest, ties to even) for bf16 workloads.
  * Lengths come from PCG64 seeded with SeedSequence(seed, spawn_key=(workload
    id, 0)).

The numpy half (``user_rows``, ``prototype_table``, ``user_dS``) imports no
torch, so worker processes of the test-suite oracle can regenerate a user's
inputs cheaply; ``make_inputs`` and ``make_workload`` assemble torch tensors
from it.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    k: int
    d: int
    dtype: str            # "f32" or "bf16": dtype of X and P
    mass_norm: bool
    lengths_kind: str     # "fixed", "uniform", "lognormal"
    len_lo: int
    len_hi: int
    x_kind: str = "normal"        # "normal" or "item_action"
    backward: bool = False
    description: str = ""


# The five workloads, in order: small fp32 parity case, the single-user 100K
# bf16 forward, a 64-user ragged forward with mass normalisation, a 256-user
# lognormal throughput batch, and a 32-user backward.
WORKLOADS = {
    "fp32_n4096_k64_d32": Workload(
        1, "fp32_n4096_k64_d32", 1, 64, 32, "f32", False, "fixed", 4096, 4096,
        description="single user, n=4096, k=64, d=32, fp32, plain sum"),
    "bf16_n100k_k1024_d128": Workload(
        2, "bf16_n100k_k1024_d128", 1, 1024, 128, "bf16", False, "fixed", 100000, 100000,
        description="single user, n=100000, k=1024, d=128, bf16 in / fp32 out"),
    "ragged64_k1024_massnorm": Workload(
        3, "ragged64_k1024_massnorm", 64, 1024, 128, "bf16", True, "uniform", 1000, 100000,
        description="64 users, n~U[1000,100000], k=1024, d=128, bf16, mass-normalised"),
    "ragged256_lognormal_k512": Workload(
        4, "ragged256_lognormal_k512", 256, 512, 128, "bf16", False, "lognormal", 512, 100000,
        x_kind="item_action",
        description="256 users, lognormal lengths mean 85000 clipped [512,100000], k=512, d=128, bf16, "
                    "X = item N(0,1) + action-type embedding (8 types, N(0,0.5))"),
    "backward32_k1024": Workload(
        5, "backward32_k1024", 32, 1024, 128, "bf16", False, "uniform", 10000, 100000,
        backward=True,
        description="backward, 32 users, n~U[10000,100000], k=1024, d=128, dS~N(0,1) fp32"),
}

WORKLOAD_ORDER = list(WORKLOADS)

# Lognormal location for the 256-user batch: with sigma = 0.5 this mu makes the
# mean of the lengths clipped to [512, 100000] equal 85000 (solved numerically;
# about half of the users sit at the 100000 cap).
LOGNORMAL_MU = 11.514
LOGNORMAL_SIGMA = 0.5
N_ACTION_TYPES = 8

TAGS = {"X": 1, "P": 2, "dS": 3, "act_table": 4, "act_ids": 5}

# Host threads drawing a batch's rows (numpy's generators release the GIL
# while filling arrays).
_THREADS = max(1, min(16, os.cpu_count() or 1))


def rng_for(seed, wid, tag, index=0):
    """The generator of one tensor (tag) of workload wid, for one user or
    shared (index 0)."""
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(int(seed), spawn_key=(int(wid), TAGS[tag], int(index)))))


def round_bf16(a):
    """float32 array -> float32 array of the nearest bfloat16 values (ties to
    even).  Finite inputs only (normal samples never hold NaN or inf)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def _to_dtype_values(a32, dtype):
    return round_bf16(a32) if dtype == "bf16" else a32


def action_table(seed, wid, d):
    """8 x d action-type embeddings, N(0, 0.5), float32."""
    g = rng_for(seed, wid, "act_table", 0)
    return (g.standard_normal((N_ACTION_TYPES, d)) * math.sqrt(0.5)).astype(np.float32)


def user_rows(seed, wid, u, n, d, dtype, x_kind="normal"):
    """History rows of user u: float32 values exactly representable in dtype.

    x_kind "normal": x_i ~ N(0, I).  "item_action": x_i = e_i + a[t_i] with
    e_i ~ N(0, I), t_i ~ U{0..7} and the action table of ``action_table``,
    summed in float32 and then rounded to dtype."""
    g = rng_for(seed, wid, "X", u)
    e = g.standard_normal((int(n), d)).astype(np.float32)
    if x_kind == "item_action":
        ids = rng_for(seed, wid, "act_ids", u).integers(0, N_ACTION_TYPES, size=int(n))
        e += action_table(seed, wid, d)[ids]
    elif x_kind != "normal":
        raise ValueError(x_kind)
    return _to_dtype_values(e, dtype)


def prototype_table(seed, wid, k, d, dtype, p_std, index=0):
    """k x d prototypes ~ N(0, p_std^2): the shared table (index 0) or user
    index - 1's own table (index = u + 1)."""
    g = rng_for(seed, wid, "P", index)
    return _to_dtype_values((g.standard_normal((k, d)) * p_std).astype(np.float32), dtype)


def user_dS(seed, wid, u, k, d):
    """Upstream gradient of user u's sketch, k x d, N(0, 1), float32."""
    return rng_for(seed, wid, "dS", u).standard_normal((k, d)).astype(np.float32)


def workload_lengths(w: Workload, seed: int = 0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(w.wid, 0))))
    if w.lengths_kind == "fixed":
        return np.full(w.batch, w.len_lo, dtype=np.int64)
    if w.lengths_kind == "uniform":
        return rng.integers(w.len_lo, w.len_hi, size=w.batch, endpoint=True).astype(np.int64)
    if w.lengths_kind == "lognormal":
        raw = rng.lognormal(LOGNORMAL_MU, LOGNORMAL_SIGMA, size=w.batch)
        return np.clip(np.rint(raw), w.len_lo, w.len_hi).astype(np.int64)
    raise ValueError(w.lengths_kind)


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


@dataclasses.dataclass(frozen=True)
class GenSpec:
    """Everything needed to regenerate a problem's tensors user by user."""
    seed: int
    wid: int
    k: int
    d: int
    dtype: str
    x_kind: str
    p_std: float
    per_user_p: bool

    def rows(self, u, n):
        return user_rows(self.seed, self.wid, u, n, self.d, self.dtype, self.x_kind)

    def table(self, u=None):
        """The shared table (u None) or user u's own table."""
        return prototype_table(self.seed, self.wid, self.k, self.d, self.dtype, self.p_std,
                               0 if u is None else u + 1)

    def dS(self, u):
        return user_dS(self.seed, self.wid, u, self.k, self.d)


@dataclasses.dataclass
class Problem:
    workload: Workload
    offsets: np.ndarray          # int64 [B+1], host
    X: "torch.Tensor"            # [T, d] f32 or bf16
    P: "torch.Tensor"            # [k, d] (or [B, k, d] per user), same dtype as X
    dS: "torch.Tensor | None"    # [B, k, d] f32
    mass_norm: bool
    gen: GenSpec | None = None

    @property
    def total_tokens(self):
        return int(self.offsets[-1])


def _torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(lengths, k, d, dtype="bf16", device="cpu", seed=0, wid=0,
                x_kind="normal", p_std=None, with_dS=False, mass_norm=False,
                workload=None, per_user_p=False) -> Problem:
    """Build a Problem for arbitrary lengths.

    p_std defaults to d**-0.5 (P ~ N(0, 1/d)); a larger value gives sharper
    logits (the standard deviation of each affinity is p_std when X ~ N(0, 1)).
    per_user_p draws one k x d table per user (P is then [B, k, d]).
    """
    import torch

    lengths = np.asarray(lengths, dtype=np.int64)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    B = int(lengths.size)
    tdt = _torch_dtype(dtype)
    if p_std is None:
        p_std = 1.0 / math.sqrt(d)
    spec = GenSpec(int(seed), int(wid), int(k), int(d), dtype, x_kind, float(p_std),
                   bool(per_user_p))
    X = torch.empty((T, d), dtype=tdt, device=device)
    # Users are drawn in parallel host threads and copied in user order.
    with concurrent.futures.ThreadPoolExecutor(_THREADS) as ex:
        futs = [ex.submit(spec.rows, u, int(lengths[u])) for u in range(B)]
        for u, f in enumerate(futs):
            lo, hi = int(off[u]), int(off[u + 1])
            rows = f.result()
            futs[u] = None
            if hi > lo:
                X[lo:hi].copy_(torch.from_numpy(rows).to(tdt))
    if per_user_p:
        P = torch.from_numpy(np.stack([spec.table(u) for u in range(B)])).to(tdt).to(device)
    else:
        P = torch.from_numpy(spec.table()).to(tdt).to(device)
    dS = None
    if with_dS:
        dS = torch.from_numpy(np.stack([spec.dS(u) for u in range(B)]).reshape(B, k, d)).to(device)
    if workload is None:
        workload = Workload(wid, "custom", B, k, d, dtype, mass_norm,
                            "custom", int(lengths.min()) if lengths.size else 0,
                            int(lengths.max()) if lengths.size else 0, x_kind, with_dS)
    return Problem(workload, off, X, P, dS, mass_norm, spec)


def make_workload(name: str, device="cpu", seed=0, with_dS=None) -> Problem:
    w = WORKLOADS[name]
    lengths = workload_lengths(w, seed)
    if with_dS is None:
        with_dS = w.backward
    return make_inputs(lengths, w.k, w.d, w.dtype, device, seed, w.wid, w.x_kind,
                       None, with_dS, w.mass_norm, w)


def to_f64(t) -> np.ndarray:
    """Exact upcast of a float32 / bfloat16 tensor to a float64 numpy array."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()
