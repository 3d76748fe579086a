"""The library's analytic speedup model (host code behind the C ABI) against
the oracle (oracle/model.py); runs on the CPU."""
import math

import numpy as np
import pytest

import long_context_kv_split_amd as sd
import oracle
from tests.gpu_helpers import ensure_lib


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def test_expected_tokens_matches_oracle():
    for gamma in range(0, 12):
        for alpha in (0.0, 0.1, 0.5, 0.8, 0.9, 0.97, 0.999999, 1.0):
            # the oracle's closed form (1 - a^(g+1)) / (1 - a) loses about
            # eps / (1 - a) to cancellation near a = 1; the library sums the series
            tol = 1e-12 if alpha == 1.0 else max(1e-12, 8 * 2.0 ** -52 / (1.0 - alpha))
            assert math.isclose(sd.sd_expected_tokens(gamma, alpha), oracle.omega(gamma, alpha), rel_tol=tol)
    assert math.isnan(sd.sd_expected_tokens(-1, 0.5))
    assert math.isnan(sd.sd_expected_tokens(3, 1.01))
    assert math.isnan(sd.sd_expected_tokens(3, float("nan")))


def test_speedup_matches_oracle_on_a_grid():
    rng = np.random.default_rng(3)
    for _ in range(300):
        tt, td, tv = rng.uniform(0.5, 5), rng.uniform(0, 1), rng.uniform(0.5, 6)
        fx, st = rng.uniform(0, 1) * (rng.random() < 0.5), rng.uniform(0, 2) * (rng.random() < 0.5)
        g, a = int(rng.integers(1, 9)), float(rng.uniform(0, 1))
        want = oracle.speedup(tt, td, tv, g, a, fx, st)
        assert math.isclose(sd.sd_speedup(tt, td, tv, g, a, fx, st), want, rel_tol=1e-12)


@pytest.mark.parametrize("args", [
    (0.0, 1.0, 1.0, 2, 0.5, 0.0, 0.0),       # t_target <= 0
    (1.0, -1.0, 1.0, 2, 0.5, 0.0, 0.0),      # negative time
    (1.0, 1.0, float("inf"), 2, 0.5, 0.0, 0.0),
    (1.0, 0.0, 0.0, 2, 0.5, 0.0, 0.0),       # round time 0
    (1.0, 1.0, 1.0, 2, 2.0, 0.0, 0.0),       # alpha > 1
])
def test_speedup_rejects_bad_arguments(args):
    assert math.isnan(sd.sd_speedup(*args))


def test_best_gamma_matches_oracle_including_ties():
    rng = np.random.default_rng(4)
    for _ in range(200):
        tt, td = rng.uniform(1, 4), rng.uniform(0, 0.6)
        tv = list(np.cumsum(rng.uniform(0, 0.2, 8)) + tt)
        a = float(rng.uniform(0, 1))
        fx, st = (rng.uniform(0, 1), 0.0) if rng.random() < 0.5 else (0.0, rng.uniform(0, 1))
        g, s = sd.sd_best_gamma(tt, td, tv, a, fx, st)
        g_ref, s_ref = oracle.best_gamma(tt, td, tv, a, fx, st)
        assert g == g_ref and math.isclose(s, s_ref, rel_tol=1e-12)
    assert sd.sd_best_gamma(1.0, 0.0, [2.0] * 4, 0.0) == (1, 0.5)  # exact ties
    with pytest.raises(sd.SdError):
        sd.sd_best_gamma(1.0, 0.1, [], 0.5)
    with pytest.raises(sd.SdError):
        sd.sd_best_gamma(1.0, 0.1, [1.0, -1.0], 0.5)
