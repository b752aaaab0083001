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


@pytest.mark.parametrize("seed", range(8))
def test_sharded_selection_equals_the_global_one(seed):
    # Every token of the global top-K is among its shard's top-K, so the merge
    # of the shards' selections is the global selection, ties included.
    from oracle import topk as ot
    rng = np.random.default_rng(900 + seed)
    for _ in range(20):
        shard = int(rng.choice([64, 128, 256]))
        n = int(rng.integers(0, 6 * shard))
        K = int(rng.integers(1, 3 * shard))
        # coarse scores: many exact ties across shards
        row = np.round(rng.standard_normal(6 * shard) * 3) / 2
        row[rng.random(row.shape) < 0.1] = -0.0
        got = ot.topk_sharded_row(row, n, K, shard)
        assert np.array_equal(got, ot.topk_row(row, n, K)), (n, K, shard)


def test_sharded_selection_brute_force_small():
    # exhaustive over every score pattern of 6 tokens with values in {0, 1, 2}
    import itertools
    from oracle import topk as ot
    for vals in itertools.product([0.0, 1.0, 2.0], repeat=6):
        row = np.array(vals)
        for K in (1, 2, 3, 5):
            for shard in (1, 2, 4):
                order = sorted(range(6), key=lambda t: (-row[t], t))[:K]
                want = np.full(K, -1)
                want[:min(K, 6)] = sorted(order)
                assert np.array_equal(ot.topk_sharded_row(row, 6, K, shard), want)
