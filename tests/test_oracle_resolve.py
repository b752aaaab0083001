"""Pins of the oracle's residency state machine (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import resolve

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_traced_example():
    g = json.load(open(os.path.join(GOLD, "resolve_tiny.json")))
    su = g["setup"]
    C, Ts = su["C"], su["T_stride"]
    t2s = np.full((1, Ts), -1, np.int32)
    s2t = np.full((1, C), -1, np.int32)
    stamp = np.zeros((1, C), np.int32)
    for v, (t, s) in enumerate([(10, 3), (20, 1), (30, 2)] + [(100 + i, 2) for i in range(61)]):
        s2t[0, v], t2s[0, t], stamp[0, v] = t, v, s
    st = resolve.ResidencyState(np.array([su["bt"]], np.int32), np.array([su["hot_blocks"]], np.int32),
                                t2s, s2t, stamp, np.array([su["host_bt"]], np.int64), su["step"])
    new, rr = resolve.resolve(np.array(su["topk"], np.int32), st)
    assert rr.row_ids.tolist() == g["row_ids"]
    assert rr.counts.tolist() == g["counts"]
    assert rr.faults[0].tolist() == g["faults"]
    assert rr.copies[0].tolist() == g["copies"]
    assert new.stamp[0, :4].tolist() == g["stamp_0_3"]
    for t, v in g["tok2slot"].items():
        assert new.tok2slot[0, int(t)] == v
    assert new.step == g["step_after"] and st.step == su["step"] and rr.err == 0


def _brute_resolve(topk, st):
    """Independent brute force: per fault, a linear scan for the least recently
    used slot among the slots not used in this step."""
    st = st.copy()
    B, P, K = topk.shape
    C = st.slot2tok.shape[1]
    s = st.step + 1
    st.step = s
    rows = np.full((B, P, K), -1, np.int64)
    counts = np.zeros((B, 4), np.int64)
    faults = []
    for b in range(B):
        seen = []
        for t in sorted(set(int(x) for x in topk[b].ravel() if x >= 0)):
            seen.append(t)
        used = [False] * C
        row_of = {}
        fl = []
        pend = []
        for t in seen:
            j = t // 64
            if st.bt[b, j] >= 0:
                counts[b, 0] += 1
                row_of[t] = st.bt[b, j] * 64 + t % 64
            elif st.tok2slot[b, t] >= 0:
                v = st.tok2slot[b, t]
                counts[b, 1] += 1
                st.stamp[b, v] = s
                used[v] = True
                row_of[t] = st.hot_blocks[b, v // 64] * 64 + v % 64
            else:
                pend.append(t)
        for t in pend:
            best = None
            for v in range(C):
                if used[v] or st.stamp[b, v] >= s:
                    continue
                if best is None or (st.stamp[b, v], v) < (st.stamp[b, best], best):
                    best = v
            assert best is not None
            old = st.slot2tok[b, best]
            if old >= 0:
                st.tok2slot[b, old] = -1
                counts[b, 3] += 1
            st.slot2tok[b, best] = t
            st.tok2slot[b, t] = best
            st.stamp[b, best] = s
            used[best] = True
            counts[b, 2] += 1
            row_of[t] = st.hot_blocks[b, best // 64] * 64 + best % 64
            fl.append((t, best))
        for p in range(P):
            for k in range(K):
                t = topk[b, p, k]
                rows[b, p, k] = -1 if t < 0 else row_of[int(t)]
        faults.append(fl)
    return st, rows, counts, faults


def _random_state(rng, B, T, C, n_res_pages):
    nb = -(-T // 64)
    bt = np.full((B, nb), -1, np.int32)
    hot = np.zeros((B, C // 64), np.int32)
    ids = rng.permutation(B * (n_res_pages + C // 64) + 10)
    k = 0
    for b in range(B):
        for j in range(nb - n_res_pages, nb):
            bt[b, j] = ids[k]; k += 1
        for i in range(C // 64):
            hot[b, i] = ids[k]; k += 1
    host_bt = np.arange(nb, dtype=np.int64)[None, :] * 64 + np.arange(B, dtype=np.int64)[:, None] * (nb * 64)
    t2s = np.full((B, nb * 64), -1, np.int32)
    s2t = np.full((B, C), -1, np.int32)
    stamp = np.zeros((B, C), np.int32)
    return resolve.ResidencyState(bt, hot, t2s, s2t, stamp, host_bt, 0)


@pytest.mark.parametrize("seed", range(6))
def test_multi_step_matches_brute_force_and_invariants(seed):
    rng = np.random.default_rng(seed)
    B, P, K = 2, int(rng.integers(1, 4)), 16
    T = 640
    C = 64 * int(np.ceil((P + 1) * K / 64))
    st = _random_state(rng, B, T, C, n_res_pages=2)
    for step in range(8):
        topk = np.full((B, P, K), -1, np.int32)
        for b in range(B):
            for p in range(P):
                # a drifting hot region so later steps hit and evict
                centre = 100 + 40 * step + 10 * p
                cand = np.unique(np.clip(rng.normal(centre, 60, 4 * K).astype(int), 0, T - 1))
                n = min(K, len(cand), int(rng.integers(K // 2, K + 1)))
                topk[b, p, :n] = np.sort(rng.choice(cand, n, replace=False))
        new, rr = resolve.resolve(topk, st)
        bst, brows, bcounts, bfaults = _brute_resolve(topk, st)
        assert np.array_equal(rr.row_ids, brows)
        assert np.array_equal(rr.counts, bcounts)
        for b in range(B):
            assert rr.faults[b].tolist() == [list(x) for x in bfaults[b]]
        for a in ("tok2slot", "slot2tok", "stamp"):
            assert np.array_equal(getattr(new, a), getattr(bst, a)), a
        assert rr.err == 0
        s = new.step
        for b in range(B):
            occ = np.nonzero(new.slot2tok[b] >= 0)[0]
            # mutual inverses
            assert np.all(new.tok2slot[b, new.slot2tok[b, occ]] == occ)
            assert np.sum(new.tok2slot[b] >= 0) == len(occ)
            # every slot stamped this step was a hit or a fault
            assert np.sum(new.stamp[b] == s) == rr.counts[b, 1] + rr.counts[b, 2]
            # resident tokens never occupy hot slots
            toks = new.slot2tok[b, occ]
            assert np.all(new.bt[b, toks // 64] < 0)
            # every token selected this step is resident or hot now
            U = np.unique(topk[b][topk[b] >= 0])
            assert np.all((new.bt[b, U // 64] >= 0) | (new.tok2slot[b, U] >= 0))
            # the copies read exactly the host row of the token
            for (t, v), (hr, pr) in zip(rr.faults[b], rr.copies[b]):
                assert hr == new.host_bt[b, t // 64] + t % 64
                assert pr == new.hot_blocks[b, v // 64] * 64 + v % 64
        st = new


def test_capacity_rule_never_short():
    # |U| <= P*K and C >= P*K: the victims always suffice (no error bit), even
    # when every selection of every step is a fresh fault.
    rng = np.random.default_rng(9)
    B, P, K = 1, 4, 16
    C = 64
    st = _random_state(rng, B, 64 * 200, C, n_res_pages=0)
    for step in range(20):
        topk = np.sort(rng.choice(np.arange(step * 64, step * 64 + 64 * 8), (1, P, K)), axis=2).astype(np.int32)
        st, rr = resolve.resolve(topk, st)
        assert rr.err == 0


def test_shortage_and_missing_host_row_set_error_bits():
    B, K = 1, 3
    st = resolve.ResidencyState(np.full((1, 4), -1, np.int32), np.zeros((1, 0), np.int32),
                                np.full((1, 256), -1, np.int32), np.zeros((1, 0), np.int32),
                                np.zeros((1, 0), np.int32), np.array([[0, 64, -1, 192]], np.int64), 0)
    new, rr = resolve.resolve(np.array([[[1, 130, 200]]], np.int32), st)
    assert rr.err == 3
    assert rr.row_ids.tolist() == [[[-1, -1, -1]]]
    assert rr.counts.tolist() == [[0, 0, 0, 0]]


def test_no_residency_first_step_all_faults():
    # empty hot buffers: step 1 hits nothing and evicts nothing
    rng = np.random.default_rng(3)
    st = _random_state(rng, 2, 64 * 64, 128, n_res_pages=0)
    topk = np.sort(np.stack([rng.choice(64 * 64, 64, replace=False) for _ in range(2)])[:, None], axis=2).astype(np.int32)
    new, rr = resolve.resolve(topk, st)
    assert rr.counts[:, 1].tolist() == [0, 0] and rr.counts[:, 3].tolist() == [0, 0]
    assert rr.counts[:, 2].tolist() == [64, 64]
    # and the same selection again is all hits
    new2, rr2 = resolve.resolve(topk, new)
    assert rr2.counts[:, 1].tolist() == [64, 64] and rr2.counts[:, 2].tolist() == [0, 0]
