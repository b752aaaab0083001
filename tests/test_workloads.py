"""The input generators: determinism, layout invariants, sizing rules (CPU only)."""
import numpy as np
import pytest

from oracle import indexer
from workloads import gen


def _eq(a, b):
    if a is None or b is None:
        return a is None and b is None
    return np.array_equal(a, b)


def test_same_seed_same_bytes():
    a, b = gen.tiny_fp32(), gen.tiny_fp32()
    for f in ("idx_pool", "idx_bt", "lat", "bt", "w"):
        assert _eq(getattr(a, f), getattr(b, f)), f
    assert np.array_equal(a.q, b.q) and np.array_equal(a.q_idx, b.q_idx)
    c = gen.tiny_fp32(seed=7)
    assert not np.array_equal(a.lat, c.lat)


def _check_layout(wl):
    # every resident page and every hot block is a distinct pool block
    used = np.concatenate([wl.bt[wl.bt >= 0].ravel(), wl.hot_blocks.ravel()])
    assert len(np.unique(used)) == len(used)
    assert used.min(initial=0) >= 0 and used.max(initial=-1) < wl.n_pool_blocks
    # the indexer cache covers every token, blocks distinct
    for b in range(wl.B):
        nb = -(-int(wl.ctx_len[b]) // 64)
        assert np.all(wl.idx_bt[b, :nb] >= 0) and np.all(wl.idx_bt[b, nb:] == -1)
    ib = wl.idx_bt[wl.idx_bt >= 0]
    assert len(np.unique(ib)) == len(ib)
    # hot tables are mutual inverses
    for b in range(wl.B):
        occ = np.nonzero(wl.slot2tok[b] >= 0)[0]
        assert np.all(wl.tok2slot[b, wl.slot2tok[b, occ]] == occ)
        assert np.sum(wl.tok2slot[b] >= 0) == len(occ)
        toks = wl.slot2tok[b, occ]
        assert np.all(wl.bt[b, toks // 64] < 0)           # never a resident token


def test_layouts_small_variants():
    _check_layout(gen.tiny_fp32())
    _check_layout(gen.resident_fp8(B=3))
    rng = np.random.default_rng(0)
    hot = np.sort(rng.choice(8192 - 1024, (2, 64), replace=False), axis=1)
    wl = gen.mixed_128k(B=2, T=8192, K=128, tail=1024, beta=1.0, hot_tokens=hot)
    _check_layout(wl)
    assert wl.C == 2 * wl.K and wl.step == 8
    assert np.all((wl.stamp >= 1) & (wl.stamp <= 8))
    assert np.all(wl.slot2tok >= 0)                       # pre-seeded buffers are full
    for b in range(2):
        assert np.all(wl.tok2slot[b, hot[b]] >= 0)        # the calibrated tokens are hot
    # pool contents: resident pages and hot slots hold the logical rows
    pool, rsc = gen.build_pool(wl)
    b, t = 1, 8192 - 3
    r = wl.bt[b, t // 64] * 64 + t % 64
    assert np.array_equal(pool[0, r], wl.lat[0, b, t]) and rsc[0, r] == wl.lat_scale[0, b, t // 64]
    v = 17
    t = wl.slot2tok[b, v]
    r = wl.hot_blocks[b, v // 64] * 64 + v % 64
    assert np.array_equal(pool[0, r], wl.lat[0, b, t])
    # host pool rows are the logical rows
    hb = wl.host_bt
    assert np.array_equal(wl.host_rows[0, hb[b, 3] + 5], wl.lat[0, b, 3 * 64 + 5])
    assert wl.host_scale[0, hb[b, 3] + 5] == wl.lat_scale[0, b, 3]


def test_hot_capacity_rule():
    # 2 x top-K rows per request, (num_speculative_tokens + 2) x top-K with MTP
    wl = gen.mtp3_agentic(B=2, K=64, steps=2, first_turn=4000, per_turn=100, turns=3, out_max=20)
    assert wl.P == 4 and wl.C == (3 + 2) * wl.K
    _check_layout(wl)
    assert wl.steps == 2 and not np.array_equal(wl.step_inputs(1)[0], wl.step_inputs(2)[0])
    wl5 = gen.norescache_1m(B=2, T=8192, K=64, L=2, steps=3)
    assert wl5.C == 2 * wl5.K and np.all(wl5.bt == -1) and wl5.L == 2
    _check_layout(wl5)


def test_ctx_lengths_follow_conversation_shape():
    T = gen.conversation_lengths(np.random.SeedSequence(1004).spawn(10)[0], 64)
    assert T.min() >= 74160 + 1 and T.max() <= 74160 + 12 * 973 + 220
    assert np.all(((T - 74160 - 1) % 973) < 220)


def test_sink_bias_sigma_closed_form_matches_scores():
    wl = gen.resident_fp8(B=2)
    S = indexer.indexer_scores(wl.q_idx, wl.q_dtype, wl.w, wl.idx_pool, wl.k_dtype,
                               wl.idx_scale, wl.idx_bt, wl.ctx_len, None, T_stride=wl.T_stride)
    for b in range(2):
        T = wl.ctx_len[b]
        emp = S[b, 0, :T].std()
        assert abs(emp / wl.info["sigma"][b] - 1) < 0.03
        assert wl.bias[b, 0] == np.float32(2 * wl.info["sigma"][b])
        assert wl.bias[b, T - 1] == wl.bias[b, 0] and wl.bias[b, 64] == 0 and wl.bias[b, T - 257] == 0


def test_append_loop_inputs():
    """The decode-loop variant: room for the appended tokens, spare blocks past the
    initial pools on two stacks, appended rows and scales taken from the latent's
    own rows past the context, one key scale per new page."""
    wl = gen.norescache_1m(B=2, T=8192, K=64, L=2, steps=70, append=True)
    base = gen.norescache_1m(B=2, T=8192, K=64, L=2, steps=70)
    assert not base.appends and base.T_stride == 8192
    assert wl.appends and wl.T_stride == 8192 + 128 and wl.ctx_len.tolist() == [8192, 8192]
    n_idx0 = wl.idx_pool.shape[0] - 4
    assert sorted(wl.free_blocks.tolist()) == list(range(wl.n_pool_blocks - 4, wl.n_pool_blocks))
    assert sorted(wl.idx_free_blocks.tolist()) == list(range(n_idx0, n_idx0 + 4))
    assert not wl.idx_pool[n_idx0:].any() and not wl.idx_scale[n_idx0:].any()
    for s in (1, 2, 64, 65, 69):
        n_new, rows, rsc, keys, ksc = wl.append_inputs(s)
        t = 8192 + s - 1
        assert n_new.tolist() == [1, 1]
        for b in range(2):
            assert np.array_equal(rows[b, 0], wl.lat[:, b, t])
            assert np.array_equal(rsc[b, 0], wl.lat_scale[:, b, t // 64])
            assert np.array_equal(keys[b, 0], wl.app_keys[b, s - 1])
            assert ksc[b, 0] == wl.app_key_scale[b, (s - 1) // 64 * 64]
        assert rows.any() and keys.any()
