"""Analytic FLOP counts of the SequenceO1 reading notes, section 5
(appendix G), Eq. (23)-(36) — TEST INFRASTRUCTURE.

Convention of Eq. (23): a product of an m x r and an r x p matrix costs 2 m r p
FLOPs; element-wise work (softmax exponentials, normalisation, activations) is
not counted.  The pinned values are the ones the pages print for the
instantiation of section 5.4 (d = 128, one head, N_sa = 2, L_s = 1024, h = 16,
d_h = 64, D = 1024, N_stca = 4, p_hit 0.5 / 0.6, R 40 / 300).

The Sketch Attention kernel of this repository computes the two length-
dependent terms of Eq. (29): 2 L_s L d (affinities) + 2 L_s L d (aggregation),
i.e. 4 k d FLOPs per history token for the forward.
"""

from __future__ import annotations


def swiglu(T, w, wf=None):
    """Eq. (23): SwiGLU FFN over T tokens of width w, inner width wf (2w)."""
    if wf is None:
        wf = 2 * w
    return 6 * T * w * wf


def attn_reorder(L, D, h):
    """Eq. (25): reordered single-query attention, all heads."""
    return 4 * L * D * h + 6 * D * D


def stca_layer(L, D, h):
    """Eq. (26): one STCA layer per target (attention + W_O + query FFN)."""
    return 4 * L * D * h + 20 * D * D


def hist_ffn(L, D):
    """Eq. (27): history-side SwiGLU FFN over all L tokens."""
    return 12 * L * D * D


def stca(L, n_stca, D, h):
    """Eq. (28): total per-target STCA FLOPs."""
    return n_stca * (hist_ffn(L, D) + stca_layer(L, D, h))


def sa_layer(L, Ls, d):
    """Eq. (29): one SA layer, 2 L d^2 + 14 L_s d^2 + 4 L_s L d."""
    return 2 * L * d * d + 2 * Ls * d * d + 2 * Ls * L * d + 2 * Ls * L * d + 12 * Ls * d * d


def sa_kernel_forward(L, Ls, d):
    """The two length-dependent GEMM terms of Eq. (29) (affinities and
    aggregation): the work of one SA forward call on an L-token history."""
    return 2 * Ls * L * d + 2 * Ls * L * d


def sa(L, n_sa, Ls, d):
    """Eq. (30)."""
    return n_sa * sa_layer(L, Ls, d)


def adapt(Ls, d, D):
    """Adapter W_A of Eq. (18): 2 L_s d D."""
    return 2 * Ls * d * D


def flops_hit(Ls, d, D, n_stca, h):
    """Eq. (31), cache hit: adapter + STCA over the sketch."""
    return adapt(Ls, d, D) + stca(Ls, n_stca, D, h)


def expected_seqo1(L, p_hit, n_sa, Ls, d, D, n_stca, h):
    """Eq. (32): expected per-target FLOPs without MRLB."""
    return flops_hit(Ls, d, D, n_stca, h) + (1.0 - p_hit) * sa(L, n_sa, Ls, d)


def stca_mrlb(L, R, n_stca, D, h):
    """Eq. (33): direct STCA with the history FFN amortised over R targets."""
    return 12 * n_stca * L * D * D / R + n_stca * (4 * L * D * h + 20 * D * D)


def seqo1_mrlb(L, R, p_hit, n_sa, Ls, d, D, n_stca, h):
    """Eq. (34): SequenceO1 with SA, adapter and the sketch-side history FFN
    amortised over R targets."""
    shared = adapt(Ls, d, D) + 12 * n_stca * Ls * D * D + (1.0 - p_hit) * sa(L, n_sa, Ls, d)
    return n_stca * (4 * Ls * D * h + 20 * D * D) + shared / R


def miss_minus_hit_mrlb(L, R, n_sa, Ls, d):
    """Eq. (35): the MRLB miss penalty per target."""
    return sa(L, n_sa, Ls, d) / R


def delta_hit_rate(p1, p2, L, R, n_sa, Ls, d):
    """Eq. (36): change of expected FLOPs between hit rates p1 and p2."""
    return (p1 - p2) * sa(L, n_sa, Ls, d) / R
