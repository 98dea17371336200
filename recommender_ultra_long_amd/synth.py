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
  * N(0, s2) means variance s2 (so P ~ N(0, 1/d) has standard deviation
    d**-0.5).
  * Floating-point samples are drawn in float32 by torch, then rounded to
    bfloat16 (round-to-nearest-even) for bf16 workloads.
  * Lengths come from numpy's PCG64 seeded with SeedSequence(seed,
    spawn_key=(workload id, 0)); tensors from torch generators seeded with a
    value derived from (seed, workload id, tensor tag), so every tensor is
    independent and reproducible on a given device type.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


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

_TAGS = {"X": 1, "P": 2, "dS": 3, "act_table": 4, "act_ids": 5}


def _seed_for(seed, wid, tag):
    return (int(seed) * 1_000_003 + int(wid) * 10_007 + _TAGS[tag] * 101) & 0x7FFFFFFFFFFFFFFF


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


def _torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal_rows(T, d, std, dtype, device, seed, chunk_rows=1 << 22):
    """T x d samples of N(0, std^2), drawn in float32 and cast to dtype in
    row chunks so that the float32 staging stays bounded."""
    out = torch.empty((T, d), dtype=dtype, device=device)
    g = _gen(device, seed)
    for r0 in range(0, T, chunk_rows):
        r1 = min(T, r0 + chunk_rows)
        tmp = torch.randn((r1 - r0, d), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        out[r0:r1] = tmp.to(dtype)
    return out


@dataclasses.dataclass
class Problem:
    workload: Workload
    offsets: np.ndarray          # int64 [B+1], host
    X: torch.Tensor              # [T, d] f32 or bf16
    P: torch.Tensor              # [k, d] (or [B, k, d] per user), same dtype as X
    dS: torch.Tensor | None      # [B, k, d] f32
    mass_norm: bool

    @property
    def total_tokens(self):
        return int(self.offsets[-1])


def make_inputs(lengths, k, d, dtype="bf16", device="cpu", seed=0, wid=0,
                x_kind="normal", p_std=None, with_dS=False, mass_norm=False,
                workload=None, per_user_p=False) -> Problem:
    """Build a Problem for arbitrary lengths.

    p_std defaults to d**-0.5 (P ~ N(0, 1/d)); a larger value gives sharper
    logits (the standard deviation of each affinity is p_std when X ~ N(0, 1)).
    per_user_p draws one k x d table per user (P is then [B, k, d]).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    tdt = _torch_dtype(dtype)
    if p_std is None:
        p_std = 1.0 / math.sqrt(d)
    if x_kind == "normal":
        X = _normal_rows(T, d, 1.0, tdt, device, _seed_for(seed, wid, "X"))
    elif x_kind == "item_action":
        g = _gen(device, _seed_for(seed, wid, "act_table"))
        table = torch.randn((N_ACTION_TYPES, d), generator=g, device=device,
                            dtype=torch.float32) * math.sqrt(0.5)
        gi = _gen(device, _seed_for(seed, wid, "act_ids"))
        X = torch.empty((T, d), dtype=tdt, device=device)
        gx = _gen(device, _seed_for(seed, wid, "X"))
        step = 1 << 22
        for r0 in range(0, T, step):
            r1 = min(T, r0 + step)
            ids = torch.randint(0, N_ACTION_TYPES, (r1 - r0,), generator=gi, device=device)
            e = torch.randn((r1 - r0, d), generator=gx, device=device, dtype=torch.float32)
            X[r0:r1] = (e + table[ids]).to(tdt)
    else:
        raise ValueError(x_kind)
    gp = _gen(device, _seed_for(seed, wid, "P"))
    pshape = (int(lengths.size), k, d) if per_user_p else (k, d)
    P = (torch.randn(pshape, generator=gp, device=device, dtype=torch.float32) * p_std).to(tdt)
    dS = None
    if with_dS:
        gd = _gen(device, _seed_for(seed, wid, "dS"))
        dS = torch.randn((lengths.size, k, d), generator=gd, device=device, dtype=torch.float32)
    if workload is None:
        workload = Workload(wid, "custom", int(lengths.size), k, d, dtype, mass_norm,
                            "custom", int(lengths.min()) if lengths.size else 0,
                            int(lengths.max()) if lengths.size else 0, x_kind, with_dS)
    return Problem(workload, off, X, P, dS, mass_norm)


def make_workload(name: str, device="cpu", seed=0, with_dS=None) -> Problem:
    w = WORKLOADS[name]
    lengths = workload_lengths(w, seed)
    if with_dS is None:
        with_dS = w.backward
    return make_inputs(lengths, w.k, w.d, w.dtype, device, seed, w.wid, w.x_kind,
                       None, with_dS, w.mass_norm, w)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a float32 / bfloat16 tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
