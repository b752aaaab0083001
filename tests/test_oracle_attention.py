"""Pins of the oracle's sparse MLA attention (CPU only)."""
import json
import math
import os

import numpy as np
import torch

from oracle import attention
from workloads import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _setup(rng, T=300, Hq=4, B=1, P=1, fp8=True):
    x = rng.standard_normal((B, -(-T // 64), 64, 576)).astype(np.float32)
    if fp8:
        codes, sc = gen.quantize_e4m3_blocks(x)
        lat = codes.reshape(B, -1, 576)
        lsc = sc.reshape(B, -1)
    else:
        lat, lsc = x.reshape(B, -1, 576), None
    q = gen.bf16_bits(rng.standard_normal((B, P, Hq, 576)))
    return lat, lsc, q


def test_hand_worked_two_rows():
    g = json.load(open(os.path.join(GOLD, "attention_tiny.json")))
    lat = np.zeros((1, 64, 576), np.float32)
    lat[0, 0, 0] = 1.0
    lat[0, 1, 1] = 1.0
    q = np.zeros((1, 1, 1, 576), np.float32)
    q[..., 0] = np.float32(24 * math.log(3))
    out, lse = attention.sparse_mla(q, "f32", lat, None, "f32", np.array([[[0, 1]]]), 1 / 24)
    assert abs(out[0, 0, 0, 0] - g["out_dim0"]) < 1e-7
    assert abs(out[0, 0, 0, 1] - g["out_dim1"]) < 1e-7
    assert np.all(out[0, 0, 0, 2:] == 0)
    assert abs(lse[0, 0, 0] - g["lse"]) < 1e-7


def test_sparse_with_k_ge_context_equals_dense_and_library_sdpa():
    rng = np.random.default_rng(0)
    T = 300
    lat, lsc, q = _setup(rng, T=T, Hq=4, B=1, P=2)
    ctx = np.array([T])
    K = 512
    topk = np.full((1, 2, K), -1, np.int32)
    topk[0, 0, :T - 1] = np.arange(T - 1)     # position 0 sees T - 2 + 1 tokens
    topk[0, 1, :T] = np.arange(T)
    so, sl = attention.sparse_mla(q, "bf16", lat, lsc, "e4m3", topk, 1 / 24)
    do, dl = attention.dense_mla(q, "bf16", lat, lsc, "e4m3", ctx, 1 / 24)
    assert np.max(np.abs(so - do)) < 1e-12 and np.max(np.abs(sl - dl)) < 1e-12
    # library routine: torch scaled_dot_product_attention in float64, MQA by broadcast
    for p, n in ((0, T - 1), (1, T)):
        x = attention.logical_rows(lat[0], lsc[0], "e4m3", np.arange(n))
        qq = torch.from_numpy(gen.bf16_values(q[0, p]).astype(np.float64))[None]      # [1, Hq, 576]
        kk = torch.from_numpy(x)[None, None].expand(1, qq.shape[1], n, 576)
        vv = torch.from_numpy(x[:, :512])[None, None].expand(1, qq.shape[1], n, 512)
        ref = torch.nn.functional.scaled_dot_product_attention(qq[:, :, None], kk, vv, scale=1 / 24)
        assert np.max(np.abs(so[0, p] - ref[0, :, 0].numpy())) < 1e-12


def test_closed_forms():
    rng = np.random.default_rng(1)
    lat, lsc, q = _setup(rng, T=256, Hq=3)
    x = attention.logical_rows(lat[0], lsc[0], "e4m3", np.arange(256))
    # K = 1: the output is the row's value part exactly; lse is the logit
    out, lse = attention.sparse_mla(q, "bf16", lat, lsc, "e4m3", np.array([[[17, -1, -1]]]), 1 / 24)
    assert np.array_equal(out[0, 0], np.broadcast_to(x[17, :512], (3, 512)))
    qv = gen.bf16_values(q[0, 0]).astype(np.float64)
    assert np.allclose(lse[0, 0], (qv @ x[17]) / 24, rtol=1e-13)
    # identical rows: out = that row, lse = z + ln n
    lat2 = lat.copy()
    lsc2 = lsc.copy()
    lat2[0, :128] = lat[0, 5]
    lsc2[0, :2] = lsc[0, 0]
    sel = np.arange(0, 128, 3)[None, None].astype(np.int32)
    out, lse = attention.sparse_mla(q, "bf16", lat2, lsc2, "e4m3", sel, 1 / 24)
    assert np.allclose(out[0, 0], np.broadcast_to(x[5, :512], (3, 512)), rtol=1e-12, atol=1e-12)
    assert np.allclose(lse[0, 0], (qv @ x[5]) / 24 + np.log(sel.size), rtol=1e-12)
    # zero query: equal weights, so out = mean of the rows and lse = ln n
    qz = np.zeros_like(q)
    sel = np.array([[[3, 9, 77, 200]]], np.int32)
    out, lse = attention.sparse_mla(qz, "bf16", lat, lsc, "e4m3", sel, 1 / 24)
    assert np.allclose(out[0, 0], np.broadcast_to(x[[3, 9, 77, 200], :512].mean(0), (3, 512)), atol=1e-13)
    assert np.allclose(lse[0, 0], np.log(4))
    # no valid row: zero output, lse = -inf
    out, lse = attention.sparse_mla(q, "bf16", lat, lsc, "e4m3", np.full((1, 1, 4), -1, np.int32), 1 / 24)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_row_order_does_not_matter_and_max_rel_err():
    rng = np.random.default_rng(2)
    lat, lsc, q = _setup(rng, T=256, Hq=2)
    sel = np.array([[[1, 50, 100, 101, 255]]], np.int32)
    o1, l1 = attention.sparse_mla(q, "bf16", lat, lsc, "e4m3", sel, 1 / 24)
    o2, l2 = attention.sparse_mla(q, "bf16", lat, lsc, "e4m3", sel[:, :, ::-1].copy(), 1 / 24)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-13) and np.allclose(l1, l2, rtol=1e-13)
    a = np.array([[1.0, -2.0, 4.0]])
    assert abs(attention.max_rel_err(a + np.array([[0, 0.04, 0]]), a) - 0.01) < 1e-15


def test_sharded_attention_merges_to_the_global_attention():
    """Token-sharded attention: the log-sum-exp merge of the shard fragments is
    the attention over the whole selection (an identity of the softmax), for
    shard counts that leave empty shards, split the selection unevenly or put
    everything in one shard; each fragment is the attention over the selected
    tokens of its shard alone."""
    rng = np.random.default_rng(7)
    T = 1024
    lat, lsc, q = _setup(rng, T=T, Hq=4, B=2, P=2)
    K = 96
    topk = np.full((2, 2, K), -1, np.int32)
    topk[0, 0] = np.sort(rng.choice(T, K, replace=False))
    topk[0, 1, :40] = np.sort(rng.choice(200, 40, replace=False))     # one region only
    topk[1, 0, :K - 5] = np.sort(rng.choice(T, K - 5, replace=False)) # -1 padded
    topk[1, 1, :1] = [777]                                            # a single row
    ref_o, ref_l = attention.sparse_mla(q, "bf16", lat, lsc, "e4m3", topk, 1 / 24)
    for shard_len in (1024, 512, 256, 64, 16):
        o, l, so, sl = attention.sparse_mla_sharded(q, "bf16", lat, lsc, "e4m3", topk, 1 / 24,
                                                    shard_len)
        assert so.shape[2] == T // shard_len
        assert np.max(np.abs(o - ref_o)) < 1e-12 and np.max(np.abs(l - ref_l)) < 1e-12
        for b in range(2):
            for p in range(2):
                sel = topk[b, p][topk[b, p] >= 0]
                for s in range(T // shard_len):
                    mine = sel[(sel >= s * shard_len) & (sel < (s + 1) * shard_len)]
                    if len(mine) == 0:
                        assert np.all(so[b, p, s] == 0) and np.all(np.isneginf(sl[b, p, s]))
                        continue
                    x = attention.logical_rows(lat[b], lsc[b], "e4m3", mine)
                    qv = gen.bf16_values(q[b, p]).astype(np.float64)
                    z = (qv @ x.T) / 24
                    # closed forms: one row gives that row; the lse of the
                    # fragment is the log of the partition sum over its rows
                    assert np.allclose(sl[b, p, s], np.log(np.exp(z).sum(axis=1)), rtol=1e-12)
                    if len(mine) == 1:
                        assert np.allclose(so[b, p, s], np.broadcast_to(x[0, :512], so[b, p, s].shape),
                                           rtol=1e-12)
                # the fragment weights exp(lse_s - LSE) sum to one
                w = np.exp(sl[b, p] - l[b, p][None, :])
                assert np.allclose(w.sum(axis=0), 1.0, rtol=1e-12)
    # one shard: the fragment is the global attention
    o, l, so, sl = attention.sparse_mla_sharded(q, "bf16", lat, lsc, "e4m3", topk, 1 / 24, T)
    assert np.array_equal(so[:, :, 0], o) and np.array_equal(sl[:, :, 0], l)
