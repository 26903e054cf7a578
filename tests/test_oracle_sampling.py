"""Pins of the oracle's top-k / top-p sampling against what its definition fixes."""

import numpy as np
import pytest

from oracle import sampling as OS


def test_top1_is_the_first_largest_logit():
    z = np.array([0.5, 3.0, -1.0, 3.0, 2.0])
    for u in (0.0, 0.3, 0.999):
        assert OS.sample(z, 1.0, 1, 1.0, u).token == 1  # the lower index of the tied maximum


def test_tiny_nucleus_is_greedy():
    z = np.random.default_rng(0).normal(size=500)
    assert OS.sample(z, 0.7, 64, 1e-9, 0.99).token == int(np.argmax(z))


def test_equal_logits_split_the_unit_interval_in_index_order():
    z = np.zeros(100)
    for k in (1, 7, 64):
        for u in (0.0, 0.05, 0.5, 0.99):
            s = OS.sample(z, 1.0, k, 1.0, u)
            assert s.token == int(np.floor(u * k))  # candidates 0..k-1, equal weights


def test_two_candidates_closed_form():
    # P(first) = 1 / (1 + exp((b - a) / T)): draws below it pick the first candidate
    a, b, T = 2.0, 1.0, 0.5
    p0 = 1.0 / (1.0 + np.exp((b - a) / T))
    z = np.array([b, a, -30.0])
    assert OS.sample(z, T, 2, 1.0, p0 - 1e-9).token == 1
    assert OS.sample(z, T, 2, 1.0, p0 + 1e-9).token == 0


def test_draw_frequencies_equal_the_nucleus_probabilities():
    # the set of u in [0, 1) that draws candidate j has measure p_j: integrate on a grid
    rng = np.random.default_rng(1)
    z = rng.normal(size=300) * 2
    T, k, p = 0.8, 20, 0.9
    ref = OS.sample(z, T, k, p, 0.0)
    grid = (np.arange(200000) + 0.5) / 200000
    counts = {}
    for u in grid[::50]:
        t = OS.sample(z, T, k, p, float(u)).token
        counts[t] = counts.get(t, 0) + 1
    n = len(grid[::50])
    # brute force: softmax over the top k, nucleus cut, renormalize
    idx = np.argsort(-z, kind="stable")[:k]
    w = np.exp((z[idx] - z[idx].max()) / T)
    c = np.cumsum(w) / w.sum()
    m = int(np.nonzero(c >= p)[0][0])
    pr = w[: m + 1] / w[: m + 1].sum()
    for j in range(m + 1):
        assert abs(counts.get(int(idx[j]), 0) / n - pr[j]) < 2.0 / n + 1e-3
        assert abs(ref.probs[j] - pr[j]) < 1e-12
    assert set(counts) <= set(int(i) for i in idx[: m + 1])


def test_temperature_scales_the_logits():
    z = np.random.default_rng(2).normal(size=64)
    for u in (0.1, 0.6, 0.93):
        assert OS.sample(z, 0.5, 32, 0.8, u).token == OS.sample(z * 2.0, 1.0, 32, 0.8, u).token


def test_nan_ranks_last_and_arguments_are_checked():
    z = np.array([np.nan, 1.0, 0.0])
    assert OS.sample(z, 1.0, 1, 1.0, 0.5).token == 1
    assert OS.sample(z, 1.0, 3, 1.0, 0.999).token == 2  # NaN carries no weight
    with pytest.raises(ValueError):
        OS.sample(z, 0.0, 1, 1.0, 0.5)
    with pytest.raises(ValueError):
        OS.sample(z, 1.0, 1, 1.0, 1.0)


@pytest.mark.parametrize("planted", ["no_renormalize", "ties_high_index"])
def test_planted_mistakes_fail_a_pin(planted):
    """Variants with a plausible mistake must fail one of the pins above."""
    z = np.zeros(10)
    z[3] = z[7] = 1.0
    if planted == "ties_high_index":
        order = np.lexsort((-np.arange(z.size), -z))  # the higher index first on ties
        assert order[0] != OS.sample(z, 1.0, 1, 1.0, 0.0).token
    else:
        # drawing against the total weight instead of the nucleus weight
        rng = np.random.default_rng(3)
        zz = rng.normal(size=50)
        s = OS.sample(zz, 1.0, 10, 0.5, 0.95)
        idx = np.argsort(-zz, kind="stable")[:10]
        w = np.exp(zz[idx] - zz[idx].max())
        wrong = int(idx[int(np.nonzero(np.cumsum(w) > 0.95 * w.sum())[0][0])])
        assert wrong != s.token
