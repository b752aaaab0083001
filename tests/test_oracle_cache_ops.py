"""Pins of the oracle's KV append, pre-copy and demotion (CPU only).

A hand-traced case (tests/golden/cache_ops_tiny.json), and random sequences of
the three operations checked against an independent record of what each
request's tokens must read (the rows appended, in order): whatever the
operations do with blocks, the logical cache may not change, no block may be
lost or held twice, host copies equal the pool, and the tail stays resident.
"""
import copy
import json
import os

import numpy as np
import pytest

from oracle import cache_ops as co

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _state(B, T_stride, L, D, Dk, n_blocks, n_idx, ctx, bt, idx_bt, free, idx_free, cap,
           rng=None):
    MB = T_stride // 64
    pool = np.zeros((L, n_blocks * 64, D), dtype=np.uint8)
    idx_pool = np.zeros((n_idx, 64, Dk), dtype=np.uint8)
    if rng is not None:
        pool[:] = rng.integers(0, 255, pool.shape)
        idx_pool[:] = rng.integers(0, 255, idx_pool.shape)
    return co.CacheState(
        ctx_len=np.array(ctx, dtype=np.int32), bt=np.array(bt, dtype=np.int32).reshape(B, MB),
        idx_bt=np.array(idx_bt, dtype=np.int32).reshape(B, MB),
        host_bt=np.full((B, MB), -1, dtype=np.int64), pool=pool,
        row_scale=np.ones((L, n_blocks * 64), dtype=np.float32), idx_pool=idx_pool,
        idx_scale=np.ones(n_idx, dtype=np.float32),
        host_rows=np.zeros((L, B * T_stride, D), dtype=np.uint8),
        host_scale=np.zeros((L, B * T_stride), dtype=np.float32),
        free=list(free), idx_free=list(idx_free), free_capacity=cap)


def test_hand_traced_append_precopy_demote():
    g = json.load(open(os.path.join(GOLD, "cache_ops_tiny.json")))
    ini = g["initial"]
    st = _state(2, g["T_stride"], 1, 2, 2, 8, 5, ini["ctx_len"], ini["bt"], ini["idx_bt"],
                ini["free"], ini["idx_free"], ini["free_capacity"])
    a = g["append"]
    P = max(a["n_new"])
    rows = np.arange(2 * P * 1 * 2, dtype=np.uint8).reshape(2, P, 1, 2) + 10
    keys = np.arange(2 * P * 2, dtype=np.uint8).reshape(2, P, 2) + 100
    assert co.append_tokens(st, a["n_new"], rows, np.full((2, P, 1), 0.5, np.float32), keys,
                            np.full((2, P), 0.25, np.float32)) == 0
    assert st.bt.tolist() == a["bt"] and st.idx_bt.tolist() == a["idx_bt"]
    assert st.ctx_len.tolist() == a["ctx_len"] and st.free == [] and st.idx_free == []
    for b, t, blk, r in a["rows_written"]:
        i = t - ini["ctx_len"][b]
        assert st.pool[0, blk * 64 + r].tolist() == rows[b, i, 0].tolist()
        assert st.row_scale[0, blk * 64 + r] == 0.5
        assert st.idx_pool[st.idx_bt[b, t // 64], t % 64].tolist() == keys[b, i].tolist()
    assert st.idx_scale[3] == 0.25 and st.idx_scale[4] == 0.25 and st.idx_scale[2] == 1.0
    before = (st.bt.copy(), st.ctx_len.copy(), list(st.free))
    a2 = g["append_again"]
    assert co.append_tokens(st, a2["n_new"], np.zeros((2, 64, 1, 2), np.uint8), None,
                            np.zeros((2, 64, 2), np.uint8), None) == a2["err"]
    assert np.array_equal(st.bt, before[0]) and np.array_equal(st.ctx_len, before[1])
    pc = g["precopy"]
    assert co.precopy_pages(st, pc["max_pages"]) == [tuple(x) for x in pc["copied"]]
    for b, p, row in pc["host_bt_set"]:
        assert st.host_bt[b, p] == row
        blk = st.bt[b, p]
        assert np.array_equal(st.host_rows[0, row:row + 64], st.pool[0, blk * 64:blk * 64 + 64])
    d = g["demote"]
    err, plan = co.demote_pages(st, d["n_demote"], d["tail_pages"])
    assert err == 0 and st.free == d["free"] and st.bt.tolist() == d["bt"]


def test_hand_traced_append_rejections():
    """Each append rejection rule on its own, with a control that differs from
    the rejected case only in the condition the rule tests."""
    g = json.load(open(os.path.join(GOLD, "append_reject_tiny.json")))
    P = g["P"]
    for case in g["cases"]:
        ini = dict(g["base"], **case["override"])
        st = _state(2, g["T_stride"], 1, 2, 2, 8, 8, ini["ctx_len"], ini["bt"], ini["idx_bt"],
                    ini["free"], ini["idx_free"], ini["free_capacity"])
        before = (st.pool.copy(), st.idx_pool.copy(), st.idx_bt.copy(), list(st.free),
                  list(st.idx_free))
        rows = np.full((2, P, 1, 2), 9, np.uint8)
        keys = np.full((2, P, 2), 7, np.uint8)
        err = co.append_tokens(st, case["n_new"], rows, np.ones((2, P, 1), np.float32), keys,
                               np.ones((2, P), np.float32))
        assert err == case["err"], case["name"]
        assert st.bt.tolist() == case["bt"], case["name"]
        assert st.ctx_len.tolist() == case["ctx_len"], case["name"]
        if err:
            assert np.array_equal(st.pool, before[0]) and np.array_equal(st.idx_pool, before[1])
            assert np.array_equal(st.idx_bt, before[2])
            assert st.free == before[3] and st.idx_free == before[4], case["name"]
        else:
            assert not np.array_equal(st.pool, before[0]), case["name"]


def _random_run(seed, steps=80):
    rng = np.random.default_rng(seed)
    B, T_stride, L, D, Dk, P = 3, 1024, 2, 3, 2, 8
    MB = T_stride // 64
    ctx = rng.integers(0, 300, B)
    in_use = sum(-(-int(t) // 64) for t in ctx)
    # few spare blocks, so that appends run the free lists dry
    n_blocks, n_idx = in_use + 3, in_use + 4
    # initial allocation: pages of every request from a shuffled block order
    order = list(rng.permutation(n_blocks))
    iorder = list(rng.permutation(n_idx))
    bt = np.full((B, MB), -1, np.int32)
    ibt = np.full((B, MB), -1, np.int32)
    for b in range(B):
        for p in range(-(-int(ctx[b]) // 64)):
            bt[b, p] = order.pop()
            ibt[b, p] = iorder.pop()
    # a free list that can overflow on demotion for odd seeds
    cap = n_blocks if seed % 2 == 0 else len(order) + 3
    st = _state(B, T_stride, L, D, Dk, n_blocks, n_idx, ctx, bt, ibt, order, iorder, cap, rng)
    # the record: what every token must read, built from the initial pool and the appends
    ref = [[st.pool[:, bt[b, t // 64] * 64 + t % 64].copy() for t in range(int(ctx[b]))]
           for b in range(B)]
    tail = 2
    for _ in range(steps):
        op = rng.integers(0, 3)
        snap = (st.bt.copy(), st.ctx_len.copy(), list(st.free), list(st.idx_free), st.host_bt.copy())
        if op == 0:
            n_new = rng.integers(0, P + 1, B)
            over = rng.random() < 0.15
            if over:
                # one request asks for more tokens than a step accepts
                n_new[int(rng.integers(0, B))] = P + 1
            rows = rng.integers(0, 255, (B, P, L, D)).astype(np.uint8)
            keys = rng.integers(0, 255, (B, P, Dk)).astype(np.uint8)
            err = co.append_tokens(st, n_new, rows, np.ones((B, P, L), np.float32), keys,
                                   np.ones((B, P), np.float32))
            if over:
                assert err & co.ERR_APPEND_RANGE
            if err:
                assert np.array_equal(st.bt, snap[0]) and np.array_equal(st.ctx_len, snap[1])
                assert st.free == snap[2] and st.idx_free == snap[3]
            else:
                for b in range(B):
                    ref[b].extend(rows[b, i].copy() for i in range(int(n_new[b])))
        elif op == 1:
            co.precopy_pages(st, int(rng.integers(1, 4)))
            _partial_page_rejection(st, rng, P, L, D, Dk)
        else:
            err, plan = co.demote_pages(st, rng.integers(0, 4, B), tail)
            if err:
                assert np.array_equal(st.bt, snap[0]) and st.free == snap[2]
        # logical content never changes
        for b in range(B):
            T = int(st.ctx_len[b])
            assert T == len(ref[b])
            for l in range(L):
                got, _ = co.logical_rows(st, b, range(T), l)
                if T:
                    assert np.array_equal(got, np.array([r[l] for r in ref[b]])), (b, l)
        # blocks: free + in use = every block, no duplicates
        used = [int(x) for x in st.bt.ravel() if x >= 0]
        assert sorted(used + st.free) == list(range(n_blocks))
        iused = [int(x) for x in st.idx_bt.ravel() if x >= 0]
        assert sorted(iused + st.idx_free) == list(range(n_idx))
        for b in range(B):
            T = int(st.ctx_len[b])
            if T:
                last = (T - 1) // 64
                assert all(st.bt[b, p] >= 0 for p in range(max(0, last - tail + 1), last + 1))
                assert all(st.idx_bt[b, p] >= 0 for p in range(last + 1))   # indexer stays
            # host copies equal the pool for resident pages
            for p in range(MB):
                if st.host_bt[b, p] >= 0 and st.bt[b, p] >= 0:
                    h, s = int(st.host_bt[b, p]), int(st.bt[b, p]) * 64
                    assert np.array_equal(st.host_rows[:, h:h + 64], st.pool[:, s:s + 64])
    return st


def _partial_page_rejection(st, rng, P, L, D, Dk):
    """On a copy of the state, take away the block of one request's partly
    filled last page (latent or indexer side): an append that would write into
    it must be refused and change nothing."""
    cand = [b for b in range(len(st.ctx_len)) if int(st.ctx_len[b]) % 64 != 0]
    if not cand:
        return
    b = cand[int(rng.integers(0, len(cand)))]
    c = copy.deepcopy(st)
    page = int(c.ctx_len[b]) // 64
    (c.bt if rng.random() < 0.5 else c.idx_bt)[b, page] = -1
    snap = copy.deepcopy(c)
    n_new = np.zeros(len(c.ctx_len), np.int64)
    n_new[b] = int(rng.integers(1, P + 1))
    err = co.append_tokens(c, n_new, np.zeros((len(n_new), P, L, D), np.uint8),
                           np.ones((len(n_new), P, L), np.float32),
                           np.zeros((len(n_new), P, Dk), np.uint8),
                           np.ones((len(n_new), P), np.float32))
    assert err & co.ERR_APPEND_RANGE
    assert np.array_equal(c.bt, snap.bt) and np.array_equal(c.idx_bt, snap.idx_bt)
    assert np.array_equal(c.ctx_len, snap.ctx_len) and np.array_equal(c.pool, snap.pool)
    assert c.free == snap.free and c.idx_free == snap.idx_free


@pytest.mark.parametrize("seed", range(6))
def test_random_sequences_keep_the_logical_cache(seed):
    _random_run(seed)


def test_random_sequences_reach_every_path():
    seen = {"append_err": 0, "demote_err": 0, "demoted": 0, "copied": 0, "appended": 0}
    oa, od, op = co.append_tokens, co.demote_pages, co.precopy_pages

    def a(st, n_new, *x):
        e = oa(st, n_new, *x)
        seen["append_err"] += bool(e)
        seen["appended"] += 0 if e else int(np.sum(n_new))
        return e

    def d(*x):
        e, p = od(*x)
        seen["demote_err"] += bool(e)
        seen["demoted"] += len(p)
        return e, p

    def c(*x):
        r = op(*x)
        seen["copied"] += len(r)
        return r
    try:
        co.append_tokens, co.demote_pages, co.precopy_pages = a, d, c
        for seed in range(6):
            _random_run(seed)
    finally:
        co.append_tokens, co.demote_pages, co.precopy_pages = oa, od, op
    assert all(v > 0 for v in seen.values()), seen
