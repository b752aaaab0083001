"""Pins of the oracle's indexer (CPU only)."""
import json
import os

import numpy as np

from oracle import indexer, topk
from workloads import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _paged(keys, rng, fp8=False):
    """keys [T, D] float32 -> a permuted paged pool and block table (1 request)."""
    T, D = keys.shape
    nb = -(-T // 64)
    pad = np.zeros((nb * 64, D), dtype=np.float32)
    pad[:T] = keys
    perm = rng.permutation(nb)
    pool = np.empty((nb, 64, D), dtype=np.float32)
    pool[perm] = pad.reshape(nb, 64, D)
    bt = perm.astype(np.int32)[None, :]
    return pool, bt


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLD, "indexer_tiny.json")))
    q = np.array(g["q"], dtype=np.float32)[None, None]
    w = np.array(g["w"], dtype=np.float32)[None, None]
    k = np.array(g["k"], dtype=np.float32)
    pool, bt = _paged(k, np.random.default_rng(0))
    bias = np.zeros((1, 64), dtype=np.float32)
    bias[0, :3] = g["bias"]
    S = indexer.indexer_scores(q, "f32", w, pool, "f32", None, bt, np.array([3]), bias)
    assert np.array_equal(S[0, 0, :3], np.array(g["scores"]))
    assert np.all(np.isneginf(S[0, 0, 3:]))
    assert list(topk.topk(S, [3], 2)[0, 0]) == g["top2"]


def test_basis_keys_closed_form():
    # keys c_t * e_{d(t)}: q_h . k_t = c_t * q_h[d(t)] exactly, so
    # S[t] = sum_h w_h max(0, c_t q_h[d(t)]) with no contraction at all.
    rng = np.random.default_rng(2)
    T, D, H = 300, 64, 5
    d = rng.integers(0, D, T)
    c = rng.standard_normal(T).astype(np.float32)
    keys = np.zeros((T, D), dtype=np.float32)
    keys[np.arange(T), d] = c
    q = rng.standard_normal((1, 1, H, D)).astype(np.float32)
    w = rng.random((1, 1, H)).astype(np.float32)
    pool, bt = _paged(keys, rng)
    S = indexer.indexer_scores(q, "f32", w, pool, "f32", None, bt, np.array([T]))
    qd = q[0, 0].astype(np.float64)[:, d] * c.astype(np.float64)[None, :]      # [H, T]
    ref = (w[0, 0].astype(np.float64)[:, None] * np.maximum(qd, 0)).sum(0)
    assert np.allclose(S[0, 0, :T], ref, rtol=1e-13, atol=1e-13)


def test_relu_identity_against_linear_form():
    # relu(x) - relu(-x) = x, so S(k) - S(-k) = (sum_h w_h q_h) . k: a linear
    # form in the key; and relu(x) + relu(-x) = |x|.  A dropped ReLU, a wrong
    # sign or a transposed operand breaks one of these.
    rng = np.random.default_rng(3)
    T, D, H = 200, 32, 6
    keys = rng.standard_normal((T, D)).astype(np.float32)
    q = rng.standard_normal((1, 1, H, D)).astype(np.float32)
    w = rng.random((1, 1, H)).astype(np.float32)
    pool, bt = _paged(keys, np.random.default_rng(4))
    S1 = indexer.indexer_scores(q, "f32", w, pool, "f32", None, bt, np.array([T]))[0, 0, :T]
    S2 = indexer.indexer_scores(q, "f32", w, -pool, "f32", None, bt, np.array([T]))[0, 0, :T]
    v = (w[0, 0].astype(np.float64)[:, None] * q[0, 0].astype(np.float64)).sum(0)
    lin = np.array([sum(v[j] * float(keys[t, j]) for j in range(D)) for t in range(T)])
    assert np.allclose(S1 - S2, lin, rtol=1e-12, atol=1e-10)
    qk = np.array([[sum(float(q[0, 0, h, j]) * float(keys[t, j]) for j in range(D))
                    for t in range(T)] for h in range(H)])
    assert np.allclose(S1 + S2, (w[0, 0][:, None] * np.abs(qk)).sum(0), rtol=1e-12, atol=1e-10)


def test_brute_force_loops_multi_request_positions_fp8():
    # Brute force on tiny inputs: every (b, p, t) scored by plain loops from the
    # raw pool bytes, including fp8 codes with per-block scales, P = 3 positions
    # with their causal limits, and a bias.
    rng = np.random.default_rng(5)
    B, P, H, D = 2, 3, 3, 16
    ctx = np.array([130, 67])
    Ts = 192
    keys = rng.standard_normal((5, 64, D)).astype(np.float32)
    codes, scale = gen.quantize_e4m3_blocks(keys)
    bt = np.array([[3, 0, 4], [1, 2, -1]], dtype=np.int32)
    q = gen.bf16_bits(rng.standard_normal((B, P, H, D)))
    w = rng.random((B, P, H)).astype(np.float32)
    bias = rng.standard_normal((B, Ts)).astype(np.float32)
    S = indexer.indexer_scores(q, "bf16", w, codes, "e4m3", scale, bt, ctx, bias, T_stride=Ts)
    from oracle.numerics import e4m3fn_value
    qv = gen.bf16_values(q).astype(np.float64)
    for b in range(B):
        for p in range(P):
            lim = ctx[b] - P + p
            for t in range(Ts):
                if t > lim:
                    assert S[b, p, t] == -np.inf
                    continue
                blk = bt[b, t // 64]
                s = 0.0
                for h in range(H):
                    dot = 0.0
                    for j in range(D):
                        dot += qv[b, p, h, j] * e4m3fn_value(codes[blk, t % 64, j]) * float(scale[blk])
                    s += float(w[b, p, h]) * max(dot, 0.0)
                s += float(bias[b, t])
                assert abs(S[b, p, t] - s) <= 1e-12 * max(1.0, abs(s)), (b, p, t)
    # token-by-token evaluation agrees with the matrix form
    toks = np.array([0, 5, 64, 127])
    at = indexer.indexer_scores_at(q, "bf16", w, codes, "e4m3", scale, bt, 0, 1, toks, bias)
    assert np.allclose(at, S[0, 1, toks], rtol=1e-13)


def test_invariances_block_permutation_scale_and_weights():
    rng = np.random.default_rng(6)
    T, D, H = 500, 16, 4
    keys = rng.standard_normal((T, D)).astype(np.float32)
    q = rng.standard_normal((1, 1, H, D)).astype(np.float32)
    w1 = rng.random((1, 1, H)).astype(np.float32)
    w2 = rng.random((1, 1, H)).astype(np.float32)
    pa, ba = _paged(keys, np.random.default_rng(7))
    pb, bb = _paged(keys, np.random.default_rng(8))
    f = lambda pool, bt, w: indexer.indexer_scores(q, "f32", w, pool, "f32", None, bt, [T])[0, 0, :T]
    assert np.array_equal(f(pa, ba, w1), f(pb, bb, w1))                 # physical placement
    assert np.allclose(f(pa, ba, w1 + w2), f(pa, ba, w1) + f(pa, ba, w2), rtol=1e-6)  # linear in w
    assert np.allclose(f(2 * pa, ba, w1), 2 * f(pa, ba, w1), rtol=1e-13)  # homogeneous in k
