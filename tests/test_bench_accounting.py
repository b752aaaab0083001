"""bench.py's accounting (CPU only): the algorithmic bytes of the 128K step's indexer
and HBM phase, worked out by hand from the configuration, and the matrix-core
roofline of the multi-position indexer against a brute-force count of the visible
(position, token) pairs."""
import os
import sys
from types import SimpleNamespace

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _cfg(B, T, P=1, K=2048, L=1, Hq=16, bias=True):
    return SimpleNamespace(B=B, P=P, K=K, L=L, Hq=Hq, H_idx=64, D_idx=128,
                           ctx_len=np.full(B, T, dtype=np.int64),
                           bias=np.zeros(1) if bias else None)


def test_indexer_bytes_of_the_128k_step():
    wl = _cfg(32, 131072)
    counts = np.zeros((32, 4), dtype=np.int64)
    alg = bench._algorithmic_bytes(wl, counts)
    keys = 32 * 131072 * 128                 # one 128-byte fp8 key per token
    pages = 32 * 131072 // 64                # 64-token pages: one scale and one block id each
    bias = 32 * 131072 * 4
    qw = 32 * 64 * (128 * 2 + 4)             # bf16 queries and fp32 head weights
    assert alg["indexer"] == {"keys": keys, "key_scales": 4 * pages, "block_table": 4 * pages,
                              "bias": bias, "queries_weights": qw}
    assert sum(alg["indexer"].values()) == 554_704_896
    # the score round trip is implementation traffic, never in the method's bytes
    assert alg["implementation"]["scores_written"] == 32 * 131072 * 4
    assert "scores" not in alg["indexer"]


def test_attention_bytes_and_host_link_follow_the_counts():
    wl = _cfg(2, 4096, K=128, L=3)
    counts = np.array([[10, 50, 68, 68], [0, 100, 28, 28]])
    alg = bench._algorithmic_bytes(wl, counts)
    rows = 2 * 128
    assert alg["attention"]["rows"] == 3 * rows * (576 + 4)
    assert alg["attention"]["row_ids"] == 3 * rows * 4
    assert alg["host_link"] == (68 + 28) * 3 * 576
    assert alg["resolve"]["fault_list_out"] == (68 + 28) * 8


def test_multi_position_roofline_counts_visible_pairs():
    T = np.array([7000, 86034, 4099])
    wl = SimpleNamespace(B=3, P=4, H_idx=64, D_idx=128, ctx_len=T)
    # brute force: position p of a request of T tokens sees tokens t <= T - P + p
    pairs = sum(sum(1 for t in range(int(n)) if t <= n - 4 + p) for n in T for p in range(4))
    stage = {"indexer": 0.1, "indexer_standalone": 0.08}
    r = bench._indexer_roofline(wl, False, 1, 1.0, 1.0, None, stage)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["algorithmic_flops"] == 2.0 * 64 * 128 * pairs
    assert abs(r["achieved"] - r["algorithmic_flops"] / 1e-4 / 1e12) < 0.1
    r8 = bench._indexer_roofline(wl, True, 1, 1.0, 1.0, None, stage)
    assert r8["peak"] == 5000.0 and r8["kernel"].startswith("indexer_e4m3_mp_kernel")


def test_one_position_roofline_is_hbm():
    wl = _cfg(4, 8192)
    r = bench._indexer_roofline(wl, False, 10, 4000.0, 5000.0, None,
                                {"indexer": 1.0, "indexer_standalone": 1.0})
    assert r["bound"] == "hbm" and r["frac"] == 0.5 and r["standalone_frac"] == 0.625
