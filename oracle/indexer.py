"""Indexer scores (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The page "Un contexte d'un million sur huit H200" (section "Ce qui se passe")
says that an indexer picks the top-K tokens that sparse MLA attends to, and
that the indexer's own cache stays resident and grows with the context while
being much smaller than the latent cache.  The pages give no formula.  The
reading taken here:

    S[b,p,t] = sum_h  w[b,p,h] * max(0, sum_d q[b,p,h,d] * k[b,t,d])  (+ bias[b,t])

for every visible token 0 <= t <= lim[b,p] = T_b - P + p (the P newest tokens
are the P query positions of a multi-token-prediction step; with P = 1 every
cached token is visible).  One key vector per token is shared by all indexer
heads, which is what keeps that cache small.  No 1/sqrt(d) factor is applied:
a positive factor cannot change which tokens are the largest.

Keys live in a paged pool of 64-token blocks: token t of request b is row
t % 64 of physical block idx_bt[b, t // 64].  An FP8 key's value is its code's
value times the fp32 scale of its block.
"""

from __future__ import annotations

import numpy as np

from .numerics import to_f64

BLOCK = 64


def visible_limit(ctx_len: int, P: int, p: int) -> int:
    """Index of the last token position p may see (may be negative)."""
    return int(ctx_len) - P + p


def gather_keys(idx_pool, idx_scale, idx_bt_row, k_dtype: str, t0: int, t1: int) -> np.ndarray:
    """float64 [t1 - t0, D]: the logical keys of tokens t0..t1-1 of one request."""
    t = np.arange(t0, t1)
    blk = np.asarray(idx_bt_row)[t // BLOCK]
    if np.any(blk < 0):
        raise ValueError("indexer block table has no block for a cached token")
    codes = np.asarray(idx_pool)[blk, t % BLOCK]
    k = to_f64(codes, k_dtype)
    if idx_scale is not None:
        k = k * np.asarray(idx_scale, dtype=np.float32).astype(np.float64)[blk][:, None]
    return k


def indexer_scores(q_idx, q_dtype: str, w, idx_pool, k_dtype: str, idx_scale, idx_bt,
                   ctx_len, bias=None, T_stride: int | None = None,
                   chunk: int = 32768) -> np.ndarray:
    """Scores for every request, position and visible token.

    Returns float64 [B, P, T_stride]; entries past a position's visible limit
    are -inf.
    """
    q = to_f64(q_idx, q_dtype)                       # [B, P, H, D]
    w = np.asarray(w, dtype=np.float32).astype(np.float64)   # [B, P, H]
    B, P, H, D = q.shape
    ctx_len = np.asarray(ctx_len).astype(np.int64)
    if T_stride is None:
        T_stride = int(np.asarray(idx_bt).shape[1]) * BLOCK
    S = np.full((B, P, T_stride), -np.inf, dtype=np.float64)
    for b in range(B):
        T = int(ctx_len[b])
        if T <= 0:
            continue
        qb = q[b].reshape(P * H, D)                  # every (position, head) pair
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            k = gather_keys(idx_pool, idx_scale, idx_bt[b], k_dtype, t0, t1)   # [n, D]
            dots = k @ qb.T                           # [n, P*H]: q[b,p,h] . k[t]
            relu = np.maximum(dots, 0.0).reshape(t1 - t0, P, H)
            s = np.einsum("nph,ph->pn", relu, w[b])   # weighted sum over heads
            if bias is not None:
                s = s + np.asarray(bias[b, t0:t1], dtype=np.float32).astype(np.float64)[None, :]
            S[b, :, t0:t1] = s
        for p in range(P):
            lim = visible_limit(T, P, p)
            S[b, p, max(lim + 1, 0):] = -np.inf
    return S


def indexer_scores_at(q_idx, q_dtype: str, w, idx_pool, k_dtype: str, idx_scale, idx_bt,
                      b: int, p: int, tokens, bias=None) -> np.ndarray:
    """Scores of selected tokens of one (request, position): float64 [len(tokens)].

    The same definition as ``indexer_scores``, evaluated token by token, for
    spot checks at sizes where the whole score matrix is too large.
    """
    q = to_f64(q_idx[b, p], q_dtype)                  # [H, D]
    w_bp = np.asarray(w[b, p], dtype=np.float32).astype(np.float64)
    out = np.empty(len(tokens), dtype=np.float64)
    for i, t in enumerate(np.asarray(tokens)):
        k = gather_keys(idx_pool, idx_scale, idx_bt[b], k_dtype, int(t), int(t) + 1)[0]
        s = float(np.dot(w_bp, np.maximum(q @ k, 0.0)))
        if bias is not None:
            s += float(np.float32(bias[b, t]))
        out[i] = s
    return out
