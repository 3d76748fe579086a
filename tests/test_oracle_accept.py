"""Pins for the oracle's modified-rejection speculative sampling.

Hand-worked fixtures (tests/golden/accept_cases.json), Monte Carlo checks that
the procedure preserves the target distribution (the property the pages state),
closed-form acceptance probabilities and the expected number of tokens per
round, and the special cases q = p and disjoint supports.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "accept_cases.json")))["cases"]
    for c in cases:
        zt = np.array(c["target_logits"])[None]
        zd = np.array(c["draft_logits"])[None]
        n, out, fl = oracle.spec_accept(zt, zd, np.array(c["x"])[None], np.array(c["u_accept"])[None],
                                        np.array(c["u_sample"])[None])
        assert n[0] == c["n"], c["name"]
        assert out[0].tolist() == c["out"], c["name"]
        assert bool(fl[0]) == bool(c.get("flagged", False)), c["name"]


def _mc(p, q, trials, seed, gamma):
    """Run the oracle on `trials` independent rounds with fixed per-position
    distributions p [gamma+1, V], q [gamma, V]; draft tokens x_i ~ q_i."""
    rng = np.random.default_rng(seed)
    V = p.shape[1]
    zt = np.broadcast_to(np.log(np.maximum(p, 1e-300)), (trials, gamma + 1, V))
    zd = np.broadcast_to(np.log(np.maximum(q, 1e-300)), (trials, gamma, V))
    x = np.stack([rng.choice(V, size=trials, p=q[i]) for i in range(gamma)], axis=1)
    ua = rng.random((trials, gamma))
    us = rng.random((trials, gamma + 1))
    return oracle.spec_accept(zt, zd, x, ua, us)


def _chi2_ok(tokens, p):
    V = p.shape[0]
    counts = np.bincount(tokens, minlength=V)
    exp = p * counts.sum()
    keep = exp > 0
    assert counts[~keep].sum() == 0
    chi2 = ((counts[keep] - exp[keep]) ** 2 / exp[keep]).sum()
    return stats.chi2.sf(chi2, keep.sum() - 1)


def test_monte_carlo_preserves_target_distribution():
    """Among rounds that emit position i, the emitted token follows p_i."""
    rng = np.random.default_rng(11)
    V, gamma = 6, 3
    p = rng.dirichlet(np.ones(V), size=gamma + 1)
    q = rng.dirichlet(np.ones(V), size=gamma)
    n, out, _ = _mc(p, q, 60000, 12, gamma)
    for i in range(gamma + 1):
        emitted = out[n >= i, i]
        assert emitted.shape[0] > 2000
        assert _chi2_ok(emitted, p[i]) > 1e-3, i


def test_acceptance_probability_closed_form():
    """P(n >= k) = prod_{i<k} alpha_i, alpha_i = sum_x min(p_i(x), q_i(x))."""
    rng = np.random.default_rng(21)
    V, gamma = 5, 3
    p = rng.dirichlet(np.ones(V) * 2, size=gamma + 1)
    q = rng.dirichlet(np.ones(V) * 2, size=gamma)
    alpha = np.minimum(p[:gamma], q).sum(axis=1)
    trials = 60000
    n, _, _ = _mc(p, q, trials, 22, gamma)
    for k in range(1, gamma + 1):
        want = np.prod(alpha[:k])
        got = (n >= k).mean()
        assert abs(got - want) < 4.5 * math.sqrt(want * (1 - want) / trials) + 1e-3


def test_expected_tokens_per_round_constant_alpha():
    """At a constant acceptance rate alpha the mean number of emitted tokens per
    round is (1 - alpha^(gamma+1)) / (1 - alpha) (the expected-length formula
    the MagicDec notes cite for Eq. 1 in §3.1)."""
    V, gamma = 4, 4
    p1 = np.array([0.4, 0.3, 0.2, 0.1])
    q1 = np.array([0.1, 0.3, 0.2, 0.4])
    alpha = np.minimum(p1, q1).sum()                      # 0.7
    p = np.tile(p1, (gamma + 1, 1))
    q = np.tile(q1, (gamma, 1))
    trials = 60000
    n, _, _ = _mc(p, q, trials, 31, gamma)
    omega = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    emitted = n + 1
    assert abs(emitted.mean() - omega) < 4.5 * emitted.std() / math.sqrt(trials)


def test_identical_distributions_accept_everything_and_bonus_follows_target():
    rng = np.random.default_rng(41)
    V, gamma = 7, 3
    p = rng.dirichlet(np.ones(V), size=gamma + 1)
    q = p[:gamma].copy()
    zt = np.log(p)[None].repeat(20000, 0)
    zd = zt[:, :gamma].copy()                            # same logits: q == p bit for bit
    x = np.stack([rng.choice(V, size=20000, p=q[i]) for i in range(gamma)], axis=1)
    n, out, _ = oracle.spec_accept(zt, zd, x, rng.random((20000, gamma)), rng.random((20000, gamma + 1)))
    assert (n == gamma).all()
    assert _chi2_ok(out[:, gamma], p[gamma]) > 1e-3


def test_disjoint_supports_reject_at_once_and_correct_from_target():
    rng = np.random.default_rng(51)
    V, gamma, trials = 6, 2, 20000
    zt = np.full((trials, gamma + 1, V), -1e30)
    zd = np.full((trials, gamma, V), -1e30)
    pt = np.array([0.5, 0.3, 0.2])
    zt[:, :, :3] = np.log(pt)
    zd[:, :, 3:] = 0.0                                    # draft mass only on tokens 3..5
    x = rng.integers(3, 6, (trials, gamma))
    n, out, _ = oracle.spec_accept(zt, zd, x, rng.random((trials, gamma)), rng.random((trials, gamma + 1)))
    assert (n == 0).all()
    assert (out[:, 1:] == -1).all()
    assert _chi2_ok(out[:, 0], np.array([0.5, 0.3, 0.2, 0, 0, 0])) > 1e-3


@pytest.mark.parametrize("std_t,noise,independent,expected",
                         [(2.0, None, True, 2 * stats.norm.cdf(-2.0 / math.sqrt(2))),
                          (2.0, 0.5, False, 2 * stats.norm.cdf(-0.25))])
def test_large_vocab_acceptance_closed_forms(std_t, noise, independent, expected):
    """For large V with Gaussian logits: independent N(0, s^2) target and draft
    give alpha = 2 Phi(-s / sqrt 2); draft = target + N(0, e^2) gives
    alpha = 2 Phi(-e / 2), whatever the target's scale."""
    rng = np.random.default_rng(61)
    B, V = 400, 20000
    zt = rng.standard_normal((B, 2, V)) * std_t
    if independent:
        zd = rng.standard_normal((B, 1, V)) * std_t
    else:
        zd = zt[:, :1] + rng.standard_normal((B, 1, V)) * noise
    q = oracle.softmax(zd[:, 0])
    cdf = np.cumsum(q, axis=1)
    x = np.array([min(np.searchsorted(cdf[b], rng.random()), V - 1) for b in range(B)])[:, None]
    n, _, _ = oracle.spec_accept(zt, zd, x, rng.random((B, 1)), rng.random((B, 2)))
    # exact per-sequence alpha from the oracle's own distributions vs the closed form
    p = oracle.softmax(zt[:, 0])
    alpha = np.minimum(p, q).sum(axis=1)
    assert abs(alpha.mean() - expected) < 0.02
    assert abs(n.mean() - expected) < 4.5 * math.sqrt(expected * (1 - expected) / B) + 0.02


def test_temperature_scales_logits():
    rng = np.random.default_rng(71)
    zt = rng.standard_normal((50, 3, 9))
    zd = rng.standard_normal((50, 2, 9))
    x = rng.integers(0, 9, (50, 2))
    ua, us = rng.random((50, 2)), rng.random((50, 3))
    a = oracle.spec_accept(zt, zd, x, ua, us, temperature=0.5)
    b = oracle.spec_accept(zt * 2.0, zd * 2.0, x, ua, us, temperature=1.0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_gamma_zero_is_inverse_cdf_sampling_from_softmax():
    """With no drafts the round emits one token drawn from p_0 = softmax(z / T):
    the draft-token sampler. Hand-worked inverse CDF and Monte Carlo."""
    p = np.array([0.2, 0.5, 0.3])
    zt = np.log(p)[None, None, :].repeat(6, axis=0)
    us = np.array([0.0, 0.1, 0.25, 0.69, 0.71, 0.99])[:, None]  # off the CDF boundaries 0.2, 0.7
    none = np.zeros((6, 0))
    n, out, _ = oracle.spec_accept(zt, none.reshape(6, 0, 3), none.astype(int), none, us)
    assert (n == 0).all()
    assert list(out[:, 0]) == [0, 0, 1, 1, 2, 2]
    rng = np.random.default_rng(72)
    q = rng.dirichlet(np.ones(7))
    trials = 40000
    zt = np.log(q)[None, None, :].repeat(trials, axis=0)
    n, out, _ = oracle.spec_accept(zt, np.zeros((trials, 0, 7)), np.zeros((trials, 0), int),
                                   np.zeros((trials, 0)), rng.random((trials, 1)))
    assert _chi2_ok(out[:, 0], q) > 1e-3


# ---- the set of correct results when a uniform sits in the flag band ----

def test_golden_outcome_sets():
    """Hand-derived sets of correct results (each fixture's "outcomes")."""
    cases = json.load(open(os.path.join(GOLDEN, "accept_cases.json")))["cases"]
    for c in cases:
        zt = np.array(c["target_logits"])[None]
        zd = np.array(c["draft_logits"])[None]
        got = oracle.accept_outcomes(zt, zd, np.array(c["x"])[None], np.array(c["u_accept"])[None],
                                     np.array(c["u_sample"])[None], 0)
        want = {(n, tuple(o)) for n, o in c["outcomes"]}
        assert got == want, c["name"]


def _near_threshold_batch(seed, B, V, gamma):
    """Random distributions whose uniforms sit within 0.5e-6 of a decision
    threshold: the accept uniform of a random position next to p/q of its
    draft token, the sampling uniform next to a random CDF boundary of the
    weights the emitted token is drawn from."""
    rng = np.random.default_rng(seed)
    zt = rng.standard_normal((B, gamma + 1, V)) * 1.5
    zd = zt[:, :gamma] + rng.standard_normal((B, gamma, V)) * 0.7
    x = rng.integers(0, V, (B, gamma))
    ua = rng.random((B, gamma))
    us = rng.random((B, gamma + 1))
    for b in range(B):
        p = oracle.softmax(zt[b])
        q = oracle.softmax(zd[b])
        i = int(rng.integers(0, gamma))
        ratio = p[i, x[b, i]] / q[i, x[b, i]]
        if ratio < 0.999:
            ua[b, i] = ratio + rng.uniform(-0.5e-6, 0.5e-6)
        n, _, _ = oracle.spec_accept(zt[b:b + 1], zd[b:b + 1], x[b:b + 1], ua[b:b + 1], us[b:b + 1])
        n = int(n[0])
        r = np.maximum(0.0, p[n] - q[n]) if n < gamma else p[gamma]
        c = np.cumsum(r) / r.sum()
        t = int(rng.integers(0, V - 1))
        if 1e-3 < c[t] < 0.999:
            us[b, n] = c[t] + rng.uniform(-0.5e-6, 0.5e-6)
    return zt, zd, x, ua, us


def test_results_within_the_band_are_correct():
    """Moving every uniform by less than the band keeps the result in the set:
    the set holds what a slightly different rounding can return. Both sides of
    the planted thresholds are reached, so the set is not a single result."""
    B, V, gamma = 300, 40, 3
    zt, zd, x, ua, us = _near_threshold_batch(81, B, V, gamma)
    n0, out0, flagged = oracle.spec_accept(zt, zd, x, ua, us)
    valid, ambiguous = oracle.accept_valid(zt, zd, x, ua, us, n0, out0)
    assert valid.all()
    assert flagged.sum() > B // 2 and ambiguous.sum() > B // 2
    differ = 0
    for shift in (-0.45e-6, 0.45e-6):
        ua2 = np.clip(ua + shift, 0.0, 1.0 - 2 ** -24)
        us2 = np.clip(us + shift, 0.0, 1.0 - 2 ** -24)
        n2, out2, _ = oracle.spec_accept(zt, zd, x, ua2, us2)
        v2, _ = oracle.accept_valid(zt, zd, x, ua, us, n2, out2)
        assert v2.all(), np.nonzero(~v2)[0][:10]
        differ += int(((n2 != n0) | (out2 != out0).any(axis=1)).sum())
    assert differ > B // 4


def test_results_outside_the_band_are_rejected():
    """A result reached only by moving a uniform well past the band is not in
    the set, and an unflagged sequence has exactly one correct result: every
    other (n, token) pair, enumerated, is rejected."""
    B, V, gamma = 200, 12, 2
    rng = np.random.default_rng(91)
    zt = rng.standard_normal((B, gamma + 1, V)) * 1.5
    zd = zt[:, :gamma] + rng.standard_normal((B, gamma, V)) * 0.7
    x = rng.integers(0, V, (B, gamma))
    ua = rng.random((B, gamma))
    us = rng.random((B, gamma + 1))
    n0, out0, flagged = oracle.spec_accept(zt, zd, x, ua, us)
    _, ambiguous = oracle.accept_valid(zt, zd, x, ua, us, n0, out0)
    assert not (ambiguous & ~flagged).any()
    moved = 0
    for shift in (-3e-3, 3e-3):
        n2, out2, _ = oracle.spec_accept(zt, zd, x, np.clip(ua + shift, 0, 0.999),
                                         np.clip(us + shift, 0, 0.999))
        changed = (n2 != n0) | (out2 != out0).any(axis=1)
        v2, _ = oracle.accept_valid(zt, zd, x, ua, us, n2, out2)
        assert not (v2 & changed & ~ambiguous).any()
        moved += int((changed & ~ambiguous).sum())
    assert moved > 10
    for b in np.nonzero(~flagged)[0][:40]:
        count = 0
        for n in range(gamma + 1):
            for y in range(V):
                row = np.array([list(x[b, :n]) + [y] + [-1] * (gamma - n)])
                v, _ = oracle.accept_valid(zt[b:b + 1], zd[b:b + 1], x[b:b + 1], ua[b:b + 1],
                                           us[b:b + 1], np.array([n]), row)
                count += int(v[0])
        assert count == 1, b


def test_band_flags_are_rare_at_large_vocabulary():
    """At V = 128256 the band is reached mostly by the draw (about 2e-6 per
    interval of the drawn row); the share of sequences with more than one
    correct result stays near that expectation."""
    rng = np.random.default_rng(95)
    B, V, gamma = 48, 128256, 4
    zt = rng.standard_normal((B, gamma + 1, V)) * 2.0
    zd = zt[:, :gamma] + rng.standard_normal((B, gamma, V)) * 0.5
    x = np.array([[np.searchsorted(np.cumsum(oracle.softmax(zd[b, i])), rng.random())
                   for i in range(gamma)] for b in range(B)]).clip(0, V - 1)
    ua = rng.random((B, gamma))
    us = rng.random((B, gamma + 1))
    n0, out0, flagged = oracle.spec_accept(zt, zd, x, ua, us)
    valid, ambiguous = oracle.accept_valid(zt, zd, x, ua, us, n0, out0)
    assert valid.all()
    assert ambiguous.sum() <= flagged.sum() <= 20
