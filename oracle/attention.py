"""Sparse MLA decode attention (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The model attends only to the tokens the indexer selected ("Un contexte d'un
million sur huit H200", section "Ce qui se passe").  The option
``sparse_mla_force_mqa`` on "vLLM sert GLM-5.3 en contexte 1M sur 16 H200"
(section "Comment s'y prendre") keeps short batches on the sparse kernel in
its MQA form; the reading taken is the absorbed-latent MQA form of MLA:

* every head attends over the same latent row x_t of 576 values
  (512 compressed + 64 rotary), which serves as the key;
* the value is the first 512 values of the same row;
* z_j = sm_scale * (q_h . x_{t_j}),  out_h = sum_j softmax(z)_j * x_{t_j}[:512],
  lse_h = ln sum_j exp(z_j) (natural log).

An FP8 row's value is its codes' values times the row's fp32 scale.  Rows are
the LOGICAL rows of the selected tokens: where a row is stored (resident page,
hot slot, host pool) cannot change the result.
"""

from __future__ import annotations

import numpy as np

from .numerics import to_f64
from .indexer import visible_limit

D_LATENT = 576
D_VALUE = 512
BLOCK = 64


def logical_rows(lat_b, lat_scale_b, kv_dtype: str, tokens) -> np.ndarray:
    """float64 [n, 576]: dequantized logical latent rows of one request.

    lat_b [T_stride, 576] (uint8 codes or float32), lat_scale_b [T_stride // 64]
    fp32 per-64-token-block scales, or None for unscaled rows.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    x = to_f64(np.asarray(lat_b)[tokens], kv_dtype)
    if lat_scale_b is not None:
        x = x * np.asarray(lat_scale_b, dtype=np.float32).astype(np.float64)[tokens // BLOCK][:, None]
    return x


def attend(q_bp: np.ndarray, x: np.ndarray, sm_scale: float):
    """Softmax attention of Hq query heads over rows x.

    q_bp float64 [Hq, 576], x float64 [n, 576] -> (out [Hq, 512], lse [Hq]).
    With n = 0 the output is 0 and lse is -inf.
    """
    Hq = q_bp.shape[0]
    if x.shape[0] == 0:
        return np.zeros((Hq, D_VALUE)), np.full(Hq, -np.inf)
    z = float(sm_scale) * (q_bp @ x.T)                 # [Hq, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ x[:, :D_VALUE]) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def sparse_mla(q, q_dtype: str, lat, lat_scale, kv_dtype: str, topk, sm_scale: float,
               pairs=None):
    """Sparse attention over the selected tokens of each (request, position).

    q [B, P, Hq, 576]; lat [B, T_stride, 576] one layer's logical latent;
    lat_scale [B, T_stride // 64] or None; topk [B, P, K] (ascending, -1 pad).
    ``pairs`` optionally restricts the work to a list of (b, p).
    Returns out float64 [B, P, Hq, 512] and lse float64 [B, P, Hq]
    (entries outside ``pairs`` are NaN).
    """
    qf = to_f64(q, q_dtype)
    B, P, Hq, _ = qf.shape
    out = np.full((B, P, Hq, D_VALUE), np.nan)
    lse = np.full((B, P, Hq), np.nan)
    todo = pairs if pairs is not None else [(b, p) for b in range(B) for p in range(P)]
    for b, p in todo:
        sel = np.asarray(topk[b, p])
        sel = sel[sel >= 0]
        x = logical_rows(lat[b], None if lat_scale is None else lat_scale[b], kv_dtype, sel)
        out[b, p], lse[b, p] = attend(qf[b, p], x, sm_scale)
    return out, lse


def sparse_mla_sharded(q, q_dtype: str, lat, lat_scale, kv_dtype: str, topk, sm_scale: float,
                       shard_len: int):
    """The same attention computed the way a cache split across GPUs by tokens
    computes it (page "vLLM sert GLM-5.3 en contexte 1M sur 16 H200", section
    "Le mécanisme": DCP splits the KV cache by tokens across GPUs and gathers
    the fragments at every layer).  The tokens are cut into contiguous shards
    of shard_len tokens; each shard attends over the selected tokens it holds
    and hands over its normalised output and log-sum-exp; the fragments are
    merged in shard order by their log-sum-exp weights:

      LSE = ln sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) * out_s.

    A shard holding no selected token contributes out_s = 0, lse_s = -inf
    (weight 0).  Returns (out [B,P,Hq,512], lse [B,P,Hq], shard_out
    [B,P,S,Hq,512], shard_lse [B,P,S,Hq]) in float64, S = ceil(T_stride /
    shard_len) with T_stride = lat.shape[1].
    """
    qf = to_f64(q, q_dtype)
    B, P, Hq, _ = qf.shape
    S = -(-lat.shape[1] // shard_len)
    shard_out = np.zeros((B, P, S, Hq, D_VALUE))
    shard_lse = np.full((B, P, S, Hq), -np.inf)
    out = np.zeros((B, P, Hq, D_VALUE))
    lse = np.full((B, P, Hq), -np.inf)
    for b in range(B):
        for p in range(P):
            sel = np.asarray(topk[b, p])
            sel = sel[sel >= 0]
            for s in range(S):
                mine = sel[(sel >= s * shard_len) & (sel < (s + 1) * shard_len)]
                if len(mine) == 0:
                    continue
                x = logical_rows(lat[b], None if lat_scale is None else lat_scale[b], kv_dtype,
                                 mine)
                shard_out[b, p, s], shard_lse[b, p, s] = attend(qf[b, p], x, sm_scale)
            ls = shard_lse[b, p]                                      # [S, Hq]
            M = ls.max(axis=0)                                        # [Hq]
            ok = np.isfinite(M)
            w = np.where(ok[None, :], np.exp(ls - np.where(ok, M, 0.0)[None, :]), 0.0)
            tot = w.sum(axis=0)
            out[b, p] = np.where(ok[:, None],
                                 (w[:, :, None] * shard_out[b, p]).sum(axis=0)
                                 / np.where(ok, tot, 1.0)[:, None], 0.0)
            lse[b, p] = np.where(ok, M + np.log(np.where(ok, tot, 1.0)), -np.inf)
    return out, lse, shard_out, shard_lse


def dense_mla(q, q_dtype: str, lat, lat_scale, kv_dtype: str, ctx_len, sm_scale: float):
    """Dense attention over every visible token (the K >= context reference)."""
    qf = to_f64(q, q_dtype)
    B, P, Hq, _ = qf.shape
    out = np.zeros((B, P, Hq, D_VALUE))
    lse = np.zeros((B, P, Hq))
    for b in range(B):
        for p in range(P):
            n = max(visible_limit(int(ctx_len[b]), P, p) + 1, 0)
            x = logical_rows(lat[b], None if lat_scale is None else lat_scale[b], kv_dtype,
                             np.arange(n))
            out[b, p], lse[b, p] = attend(qf[b, p], x, sm_scale)
    return out, lse


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over output vectors of ||got - ref||_inf / ||ref||_inf (last axis = vector)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if num.size else 0.0
