"""Host checks of the all-user parity harness (worker processes that
regenerate each user's inputs and run the oracle): it accepts results that
equal the oracle's and names the user whose result is wrong.  No GPU: the
"device" results here are the oracle's own, computed in this process."""

import numpy as np
import pytest
import torch

from oracle.sa_ref import sa_backward_ref, sa_forward_ref
from recommender_ultra_long_amd import synth
from sa_testutil import check_backward_all_users, check_forward_all_users


def _prob(mass_norm):
    return synth.make_inputs([300, 0, 45, 1000, 1], 64, 32, "bf16", device="cpu", seed=4, wid=900,
                             x_kind="item_action", with_dS=True, mass_norm=mass_norm)


def test_regenerated_rows_match_the_batch():
    prob = _prob(False)
    for u in range(5):
        lo, hi = int(prob.offsets[u]), int(prob.offsets[u + 1])
        rows = prob.gen.rows(u, hi - lo)
        assert np.array_equal(rows, prob.X[lo:hi].float().numpy())
    assert np.array_equal(prob.gen.table(), prob.P.float().numpy())
    assert np.array_equal(prob.gen.dS(3), prob.dS[3].numpy())


@pytest.mark.parametrize("mass_norm", [False, True])
def test_forward_harness_accepts_the_oracle_and_names_a_wrong_user(mass_norm):
    prob = _prob(mass_norm)
    S, lse, mass = sa_forward_ref(prob.offsets, synth.to_f64(prob.X), synth.to_f64(prob.P), mass_norm)
    S, lse, mass = (torch.from_numpy(a).float() for a in (S, lse, mass))
    worst = check_forward_all_users(prob, S, lse, mass, 1e-6)
    assert max(worst) < 1e-6
    S[3, 7, 1] += 0.05 * float(S[3].abs().max())
    with pytest.raises(AssertionError, match="user 3"):
        check_forward_all_users(prob, S, lse, mass, 2e-2)


def test_backward_harness_checks_every_user_and_the_summed_dP():
    prob = _prob(False)
    dX, dP = sa_backward_ref(prob.offsets, synth.to_f64(prob.X), synth.to_f64(prob.P),
                             synth.to_f64(prob.dS), False)
    dX, dP = torch.from_numpy(dX).float(), torch.from_numpy(dP).float()
    edx, edp = check_backward_all_users(prob, dX, dP, 1e-6)
    assert edx < 1e-6 and edp < 1e-6
    bad = dP.clone()
    bad[5, 2] += 0.05 * float(dP.abs().max())
    with pytest.raises(AssertionError, match="dP"):
        check_backward_all_users(prob, dX, bad, 2e-2)
