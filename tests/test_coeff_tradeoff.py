"""The schedule explorer against the oracle's exact Newton-Schulz iteration
(an independent implementation of the same map) and against calculus."""
import numpy as np

from oracle import muon_oracle as om
from optimizer_muon_step_amd import coeff_tradeoff as ct

SCHEDULE = [(3.4445, -4.7750, 2.0315), (3.0, -3.2, 1.2), (2.5, -2.0, 0.6), (2.0, -1.5, 0.5),
            (1.875, -1.25, 0.375)]


def test_composition_matches_the_iteration_on_a_diagonal_matrix():
    sig = np.array([1.0, 0.7, 0.31, 0.05, 0.004, 1e-5])
    X0 = np.zeros((6, 9))
    X0[np.arange(6), np.arange(6)] = sig
    for sch in (ct.as_schedule(ct.DEFAULT_TRIPLE, 5), SCHEDULE):
        X = om.newton_schulz(X0, len(sch), sch, mode="exact")
        assert np.allclose(np.diag(X[:, :6]), ct.compose(sch, sig), rtol=1e-13, atol=0)


def test_slope_at_zero_is_the_product_of_the_linear_coefficients():
    for sch in (ct.as_schedule(ct.DEFAULT_TRIPLE, 5), SCHEDULE):
        h = 1e-9
        fd = ct.compose(sch, [h])[0] / h
        assert abs(fd - ct.profile(sch)["slope0"]) < 1e-6 * fd


def test_profiles_of_known_schedules():
    d5 = ct.profile(ct.as_schedule(ct.DEFAULT_TRIPLE, 5), s_min=3e-3)
    assert abs(d5["slope0"] - 3.4445 ** 5) < 1e-9
    lo, hi = d5["band"]
    assert 0.6817 < lo < 0.6819 and 1.2023 < hi < 1.2025
    assert abs(d5["P(1)"] - 0.696436) < 1e-6
    tb = ct.profile(ct.as_schedule(ct.TEXTBOOK_TRIPLE, 5))
    assert abs(tb["P(1)"] - 1.0) < 1e-15 and tb["band"][1] <= 1.0 + 1e-15
