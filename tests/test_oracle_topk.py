"""Pins of the oracle's top-K (CPU only)."""
import numpy as np
import pytest

from oracle import topk


def _brute(s, n, K):
    if n <= K:
        return np.concatenate([np.arange(n), -np.ones(K - n, int)])
    return np.sort(np.argsort(-s[:n], kind="stable")[:K])


@pytest.mark.parametrize("seed", range(20))
def test_matches_stable_full_sort_with_planted_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 512))
    K = int(rng.integers(1, 64))
    s = rng.standard_normal(n)
    # planted exact ties, exact zeros and a ReLU-like floor
    s[rng.integers(0, n, n // 4)] = 0.0
    s[rng.integers(0, n, n // 8)] = s[rng.integers(0, n)]
    s = np.round(s, 1)
    got = topk.topk_row(np.concatenate([s, np.full(7, np.nan)]), n, K)
    assert np.array_equal(got, _brute(s, n, K))


def test_selection_property_and_padding():
    rng = np.random.default_rng(1)
    s = np.round(rng.standard_normal(300), 1)
    sel = topk.topk_row(s, 300, 40)
    assert np.all(np.diff(sel) > 0)
    rest = np.setdiff1d(np.arange(300), sel)
    for t in sel:                       # every selected token beats every other one
        assert np.all((s[t] > s[rest]) | ((s[t] == s[rest]) & (t < rest)))
    sel = topk.topk_row(s, 5, 8)
    assert list(sel) == [0, 1, 2, 3, 4, -1, -1, -1]
    assert list(topk.topk_row(s, 0, 3)) == [-1, -1, -1]
    assert list(topk.topk_row(s, -2, 2)) == [-1, -1]


def test_batch_limits_follow_positions():
    # P positions: position p of a request with T tokens sees T - P + p + 1 tokens
    S = np.zeros((1, 3, 64))
    out = topk.topk(S, [5], 4)
    assert list(out[0, 0]) == [0, 1, 2, -1]
    assert list(out[0, 1]) == [0, 1, 2, 3]
    assert list(out[0, 2]) == [0, 1, 2, 3]


def test_kth_score():
    s = np.array([3.0, 1.0, 2.0, 5.0])
    assert topk.kth_score(s, 4, 2) == 3.0
    assert topk.kth_score(s, 4, 4) == -np.inf
