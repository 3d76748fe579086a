"""Pins for the analytic speedup model (oracle/model.py): Monte Carlo of the
round process, the explicit sum over acceptance lengths, limits, and
hand-worked values."""
import numpy as np
import pytest

from oracle.model import best_gamma, omega, round_time, speedup


@pytest.mark.parametrize("gamma,alpha", [(1, 0.5), (4, 0.8), (6, 0.93), (3, 0.0), (5, 1.0)])
def test_omega_is_the_mean_tokens_of_simulated_rounds(gamma, alpha):
    """Each draft is accepted with probability alpha until the first
    rejection; a round yields the accepted drafts plus one token."""
    rng = np.random.default_rng(gamma * 100 + int(alpha * 100))
    n = 400_000
    accept = rng.random((n, gamma)) < alpha
    first_reject = np.where(accept.all(axis=1), gamma, np.argmin(accept, axis=1))
    tokens = first_reject + 1
    se = tokens.std() / np.sqrt(n)
    assert abs(tokens.mean() - omega(gamma, alpha)) <= 5 * se + 1e-12


def test_omega_equals_the_sum_over_lengths_and_limits():
    for gamma in range(0, 9):
        for alpha in (0.0, 0.3, 0.77, 0.999, 1.0):
            # P(at least i drafts accepted) = alpha^i, i = 0..gamma
            assert np.isclose(omega(gamma, alpha), sum(alpha ** i for i in range(gamma + 1)), rtol=1e-12)
    assert omega(0, 0.6) == 1.0            # no drafts: one token per round
    assert omega(4, 0.0) == 1.0            # every draft rejected
    assert omega(4, 1.0) == 5.0            # every draft accepted
    assert omega(2, 0.5) == 1.75           # 1 + 1/2 + 1/4
    with pytest.raises(ValueError):
        omega(3, 1.5)


def test_speedup_hand_values_and_special_cases():
    # free draft, verification as cheap as decoding: the speedup is Omega
    assert np.isclose(speedup(1.0, 0.0, 1.0, 4, 0.8), omega(4, 0.8))
    # T_T = 10, T_D = 1, T_V = 12, gamma = 2, alpha = 0.5: 10 * 1.75 / (2 + 12) = 1.25
    assert np.isclose(speedup(10.0, 1.0, 12.0, 2, 0.5), 1.25)
    # a dynamic search of 0.5 per draft step adds gamma * 0.5 to the round
    assert np.isclose(speedup(10.0, 1.0, 12.0, 2, 0.5, t_select_step=0.5), 17.5 / 15.0)
    assert round_time(1.0, 12.0, 2, t_select_fixed=3.0) == 17.0
    # alpha = 0: every round yields one token at the cost of a round
    assert np.isclose(speedup(3.0, 0.5, 3.0, 3, 0.0), 3.0 / 4.5)


def test_best_gamma_minimises_time_per_token():
    t_v = [1.0 + 0.02 * g for g in range(1, 9)]
    g, s = best_gamma(1.0, 0.1, t_v, 0.9)
    per_token = [(g2 * 0.1 + t_v[g2 - 1]) / omega(g2, 0.9) for g2 in range(1, 9)]
    assert g == 1 + int(np.argmin(per_token)) and np.isclose(s, 1.0 / min(per_token))
    # a costlier draft pushes the optimum to shorter speculation
    g_costly, _ = best_gamma(1.0, 0.5, t_v, 0.9)
    assert g_costly < g
    # alpha = 0: speculation never pays; gamma = 1 is the least bad
    assert best_gamma(1.0, 0.1, t_v, 0.0)[0] == 1
    # exact ties (alpha = 0, free draft, flat verify cost) go to the smaller gamma
    assert best_gamma(1.0, 0.0, [2.0] * 4, 0.0) == (1, 0.5)
