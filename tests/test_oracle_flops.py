"""Pin the analytic FLOP formulas, Eq. (23)-(36) of the SequenceO1 reading
notes (section 5 / appendix G), to the values the pages print for the
instantiation of section 5.4 (no GPU)."""

import json
import os

import pytest

from oracle import flops as F

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "flops_instantiation.json")))
H = GOLD["hyperparameters"]
V = GOLD["printed_gflop_per_target"]
R = GOLD["printed_ratios"]


def _last_digit(printed):
    s = repr(printed)
    decimals = len(s.split(".")[1]) if "." in s else 0
    return 10 ** (-decimals)


def _check(value_flop, printed_gflop):
    # The printed values are truncated to 4-5 significant figures and one of
    # them (108.09 against 108.1008 computed) sits 1.0e-4 below the formula:
    # allow one unit of the last printed digit or 2e-4 relative, whichever is
    # larger.  The smallest term of any formula here moves its total by more
    # than 7e-4, so a dropped or doubled term still fails.
    tol = max(_last_digit(printed_gflop), 2e-4 * printed_gflop)
    assert abs(value_flop / 1e9 - printed_gflop) <= tol, (value_flop / 1e9, printed_gflop)


def test_printed_instantiation_values():
    L, Ls, d, D, h, N, Nsa = H["L"], H["L_s"], H["d"], H["D"], H["h"], H["n_stca"], H["n_sa"]
    stca_full = F.stca(L, N, D, h)
    _check(stca_full, V["direct_stca_train_no_mrlb"])
    _check(F.expected_seqo1(L, H["p_hit_train"], Nsa, Ls, d, D, N, h), V["seqo1_train_no_mrlb"])
    _check(F.stca_mrlb(L, H["R_train"], N, D, h), V["direct_stca_train_mrlb"])
    _check(F.seqo1_mrlb(L, H["R_train"], H["p_hit_train"], Nsa, Ls, d, D, N, h), V["seqo1_train_mrlb"])
    _check(F.stca_mrlb(L, H["R_infer"], N, D, h), V["direct_stca_infer_mrlb"])
    _check(F.seqo1_mrlb(L, H["R_infer"], H["p_hit_infer"], Nsa, Ls, d, D, N, h), V["seqo1_infer_mrlb"])
    _check(F.stca_mrlb(10000, H["R_infer"], N, D, h), V["recent_10k_branch_infer_mrlb"])


def test_printed_ratios():
    L, Ls, d, D, h, N, Nsa = H["L"], H["L_s"], H["d"], H["D"], H["h"], H["n_stca"], H["n_sa"]
    r1 = F.stca(L, N, D, h) / F.expected_seqo1(L, H["p_hit_train"], Nsa, Ls, d, D, N, h)
    r2 = F.stca_mrlb(L, H["R_train"], N, D, h) / F.seqo1_mrlb(L, H["R_train"], H["p_hit_train"], Nsa, Ls, d, D, N, h)
    r3 = F.stca_mrlb(L, H["R_infer"], N, D, h) / F.seqo1_mrlb(L, H["R_infer"], H["p_hit_infer"], Nsa, Ls, d, D, N, h)
    assert r1 == pytest.approx(R["train_no_mrlb"], abs=0.005)
    assert r2 == pytest.approx(R["train_mrlb"], abs=0.005)
    assert r3 == pytest.approx(R["infer_mrlb"], abs=0.005)


def test_sa_layer_terms():
    # Eq. (29) collects to 2 L d^2 + 14 L_s d^2 + 4 L_s L d.
    for L, Ls, d in [(100000, 1024, 128), (4096, 64, 32), (7, 3, 5)]:
        assert F.sa_layer(L, Ls, d) == 2 * L * d * d + 14 * Ls * d * d + 4 * Ls * L * d
        assert F.sa_kernel_forward(L, Ls, d) == 4 * Ls * L * d
    assert F.swiglu(10, 8) == 12 * 10 * 8 * 8     # Eq. (23), w_f = 2w
    assert F.sa(100000, 2, 1024, 128) / 1e9 == pytest.approx(111.88, abs=0.005)


def test_hit_rate_sensitivity():
    # Eq. (35)-(36): the MRLB miss penalty is SA / R; the change between hit
    # rates is linear in their difference.
    sa = F.sa(100000, 2, 1024, 128)
    assert F.miss_minus_hit_mrlb(100000, 40, 2, 1024, 128) == pytest.approx(sa / 40)
    d1 = F.seqo1_mrlb(100000, 40, 0.4, 2, 1024, 128, 1024, 4, 16) - F.seqo1_mrlb(100000, 40, 0.6, 2, 1024, 128, 1024, 4, 16)
    assert d1 == pytest.approx(F.delta_hit_rate(0.6, 0.4, 100000, 40, 2, 1024, 128))
