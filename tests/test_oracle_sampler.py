"""Pins of the oracle's sampler ("ember internals", section "sampler"): hand-derived
small cases, the greedy limit, float64 library re-derivations of each stage, and the
distribution the draw follows over a uniform grid of draws."""
import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
from oracle import sampler as S


def test_temperature_zero_is_greedy_lowest_index():
    logits = np.array([1.0, 5.0, 5.0, 2.0], np.float32)
    for r in (0.0, 0.5, 0.99):
        assert S.sample(logits, 0.0, 0, 1.0, r) == 1
        assert S.sample(logits, 0.0, 0, 1.0, r) == int(oracle.greedy_argmax(logits[None])[0])


def test_top_k_keeps_ties_with_the_threshold():
    # k = 2 on [1, 3, 2, 3]: the 2nd largest is 3, so indices 1 and 3 survive with equal
    # weight; a draw below 0.5 lands on 1, above on 3.
    logits = np.array([1.0, 3.0, 2.0, 3.0], np.float32)
    z = S.top_k_mask(logits, 2)
    assert np.isneginf(z[[0, 2]]).all() and (z[[1, 3]] == 3.0).all()
    assert S.sample(logits, 1.0, 2, 1.0, 0.25) == 1
    assert S.sample(logits, 1.0, 2, 1.0, 0.75) == 3
    # k = 1: the threshold is still 3, both tied maxima survive
    assert S.sample(logits, 1.0, 1, 1.0, 0.75) == 3
    # k = 0 and k >= V leave the row alone
    assert np.array_equal(S.top_k_mask(logits, 0), logits)
    assert np.array_equal(S.top_k_mask(logits, 4), logits)


def test_top_p_worked_example():
    # probabilities 0.5, 0.3, 0.2: with p = 0.6 the decreasing running sums are 0.5, 0.8,
    # so the nucleus is {0, 1} (cutoff 0.3) and renormalises to 0.625 / 0.375.
    logits = np.log(np.array([0.5, 0.3, 0.2])).astype(np.float32)
    z = S.top_p_mask(logits, 0.6)
    assert np.isneginf(z[2]) and np.isfinite(z[:2]).all()
    d = S.softmax(z)
    assert abs(d[0] - 0.625) < 1e-6 and abs(d[1] - 0.375) < 1e-6 and d[2] == 0
    assert S.sample(logits, 1.0, 0, 0.6, 0.6) == 0
    assert S.sample(logits, 1.0, 0, 0.6, 0.7) == 1
    # p = 0.4: the first probability alone exceeds p
    assert all(S.sample(logits, 1.0, 0, 0.4, r) == 0 for r in (0.0, 0.5, 0.999))
    # p outside (0, 1) switches the stage off
    assert np.array_equal(S.top_p_mask(logits, 1.0), logits)


def test_fully_masked_row_is_uniform():
    z = np.full(4, -np.inf, np.float32)
    d = S.softmax(z)
    assert np.allclose(d, 0.25)
    # running sums 0.25, 0.5, 0.75, 1: r = 0.5 is first exceeded at index 2
    assert S.categorical(d, 0.5) == 2


def test_rounding_fallback_takes_the_last_maximum():
    # total 0.9 < r: no running sum exceeds r, the last of the equal maxima is returned
    assert S.categorical(np.array([0.3, 0.3, 0.3], np.float32), 0.95) == 2
    assert S.categorical(np.array([0.1, 0.4, 0.4], np.float32), 0.95) == 2


def _ref_index(dist64, r):
    return int(np.searchsorted(np.cumsum(dist64), r, side="right"))


@pytest.mark.parametrize("t", [0.7, 1.3])
def test_plain_draw_matches_float64_inverse_cdf(t):
    rng = np.random.default_rng(3)
    logits = rng.normal(0, 3, 1000).astype(np.float32)
    d64 = sp_softmax(logits.astype(np.float64) / t)
    cdf = np.cumsum(d64)
    checked = 0
    for r in rng.random(200):
        if np.min(np.abs(cdf - r)) < 1e-5:
            continue                              # too close to a boundary for f32
        assert S.sample(logits, t, 0, 1.0, float(r)) == _ref_index(d64, r)
        checked += 1
    assert checked > 150


def test_top_k_keeps_exactly_the_k_largest():
    rng = np.random.default_rng(4)
    logits = rng.normal(0, 2, 5000).astype(np.float32)
    for k in (1, 10, 777):
        keep = np.isfinite(S.top_k_mask(logits, k))
        ref = np.zeros_like(keep)
        ref[np.argpartition(-logits.astype(np.float64), k - 1)[:k]] = True
        assert np.array_equal(keep, ref)


def test_top_p_nucleus_matches_float64_definition():
    rng = np.random.default_rng(5)
    for trial in range(20):
        logits = rng.normal(0, 2, 3000).astype(np.float32)
        p = float(rng.uniform(0.05, 0.95))
        d64 = sp_softmax(logits.astype(np.float64))
        order = np.argsort(-d64, kind="stable")
        cum = np.cumsum(d64[order])
        n = int(np.nonzero(cum > p)[0][0]) + 1    # shortest prefix exceeding p
        if abs(cum[n - 1] - p) < 1e-5 or (n > 1 and abs(cum[n - 2] - p) < 1e-5):
            continue
        ref = np.zeros(3000, bool)
        ref[order[:n]] = True
        assert np.array_equal(np.isfinite(S.top_p_mask(logits, p)), ref)


def test_draws_over_a_uniform_grid_follow_the_distribution():
    # r_j = (j + 0.5) / N: the share of draws landing on each token equals its final
    # probability to within 1/N (inverse-CDF sampling maps grid points to intervals).
    rng = np.random.default_rng(6)
    logits = rng.normal(0, 1.5, 64).astype(np.float32)
    N = 20000
    for t, k, p in [(1.0, 0, 1.0), (0.8, 20, 1.0), (1.2, 0, 0.7), (0.9, 16, 0.8)]:
        dist = S.final_distribution(logits, t, k, p).astype(np.float64)
        counts = np.bincount([S.sample(logits, t, k, p, (j + 0.5) / N) for j in range(N)],
                             minlength=64)
        assert np.abs(counts / N - dist).max() <= 1.0 / N + 1e-5


def test_large_temperature_tends_to_uniform():
    logits = np.linspace(-3, 3, 16).astype(np.float32)
    for i in range(16):
        assert S.sample(logits, 1e7, 0, 1.0, (i + 0.5) / 16) == i
