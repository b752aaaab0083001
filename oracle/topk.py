"""Top-K selection (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The indexer keeps the K highest-scoring tokens of each query ("Un contexte
d'un million sur huit H200", section "Ce qui se passe"); K = 2048 is the
number of selected tokens named on "vLLM sert GLM-5.3 en contexte 1M sur
16 H200", section "Comment s'y prendre".

Readings (the pages fix none of these):
* Order: score descending, equal scores broken toward the lower token index.
* Output: the K selected token indices in ascending token order (this makes
  the attention's reduction order canonical, independent of where a row is
  stored).
* A position that sees n <= K tokens selects all of them; the rest of its
  K entries are -1.
"""

from __future__ import annotations

import numpy as np

from .indexer import visible_limit


def topk_row(scores_row: np.ndarray, n_visible: int, K: int) -> np.ndarray:
    """int32 [K]: the selection for one (request, position)."""
    out = np.full(K, -1, dtype=np.int32)
    n = max(int(n_visible), 0)
    if n == 0:
        return out
    if n <= K:
        out[:n] = np.arange(n, dtype=np.int32)
        return out
    s = np.asarray(scores_row[:n], dtype=np.float64)
    t = np.arange(n)
    order = np.lexsort((t, -s))          # primary key: score desc; secondary: token asc
    out[:] = np.sort(order[:K]).astype(np.int32)
    return out


def topk(scores: np.ndarray, ctx_len, K: int) -> np.ndarray:
    """int32 [B, P, K] for scores [B, P, T_stride]."""
    B, P, _ = scores.shape
    out = np.empty((B, P, K), dtype=np.int32)
    for b in range(B):
        for p in range(P):
            out[b, p] = topk_row(scores[b, p], visible_limit(int(ctx_len[b]), P, p) + 1, K)
    return out


def kth_score(scores_row: np.ndarray, n_visible: int, K: int) -> float:
    """The K-th largest visible score (the selection threshold), or -inf if n <= K."""
    n = max(int(n_visible), 0)
    if n <= K:
        return -np.inf
    s = np.asarray(scores_row[:n], dtype=np.float64)
    return float(np.partition(s, n - K)[n - K])


def topk_sharded_row(scores_row: np.ndarray, n_visible: int, K: int, shard_len: int) -> np.ndarray:
    """The selection computed the way a token-sharded cache would: the visible
    tokens are cut into contiguous shards of shard_len tokens, each shard keeps
    its own top-K (the rule of topk_row), and the K best of the union of those
    candidates are kept (same order and tie rule), in ascending token order.

    Page "vLLM sert GLM-5.3 en contexte 1M sur 16 H200", section "Le
    mécanisme" (DCP: the KV cache is split across GPUs by tokens).  Every token of the global
    top-K is in its shard's top-K, so this equals topk_row; the function is the
    definition the sharded GPU path follows, and the tests pin the equality.
    """
    n = max(int(n_visible), 0)
    cand = []
    for s0 in range(0, n, shard_len):
        m = min(shard_len, n - s0)
        sel = topk_row(np.asarray(scores_row)[s0:s0 + m], m, K)
        cand.extend(int(t) + s0 for t in sel if t >= 0)
    cand = np.array(sorted(cand), dtype=np.int64)
    out = np.full(K, -1, dtype=np.int32)
    if len(cand) == 0:
        return out
    sub = topk_row(np.asarray(scores_row)[cand], len(cand), K)
    sub = sub[sub >= 0]
    out[:len(sub)] = cand[sub]
    return out
