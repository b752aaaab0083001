"""Stage-isolated comparison of one GPU decode step against the oracle.

Each GPU stage is checked against the oracle stage fed with the inputs that
GPU stage consumed: GPU scores vs oracle scores (floating point); GPU top-K vs
the oracle's top-K of the GPU scores (exact) and of the oracle scores (swaps
only among near-ties); GPU resolve vs the oracle resolve of the GPU top-K
(bit-exact tables, rows, faults, counts and copied bytes); GPU attention vs the
oracle attention over the GPU top-K (max relative error per output vector).
"""
from __future__ import annotations

import numpy as np

from oracle import attention as o_attn, indexer as o_idx, quant as o_quant, resolve as o_res, \
    topk as o_topk

SCORE_RTOL = 2e-5       # |gpu - oracle| / max|S| of the row (fp32 accumulation)
TOPK_TIE_REL = 1e-3     # swaps allowed only within 1e-3 relative of the K-th score


def oracle_state(wl):
    return o_res.ResidencyState(wl.bt.copy(), wl.hot_blocks.copy(), wl.tok2slot.copy(),
                                wl.slot2tok.copy(), wl.stamp.copy(), wl.host_bt.copy(), int(wl.step))


def indexer_queries(wl, q_idx, indexer_q=None):
    """(queries, their type tag, head weights) as the indexer consumes them:
    the workload's own, or with indexer_q == "e4m3" the oracle's per-head E4M3
    quantization of them (codes and scaled weights)."""
    if indexer_q in (None, wl.q_dtype):
        return q_idx, wl.q_dtype, wl.w
    assert indexer_q == "e4m3"
    codes, w_scaled, _ = o_quant.quantize_queries(q_idx, wl.w)
    return codes, "e4m3", w_scaled


def check_quantized(q_idx, w, q8, w_scaled):
    """GPU query quantization against the oracle's: codes bit-exact (a zero
    may carry either sign) and scaled weights bit-exact."""
    codes, ws, _ = o_quant.quantize_queries(q_idx, w)
    strip = lambda c: np.where(c == 0x80, np.uint8(0), c)
    bad = np.argwhere(strip(codes) != strip(q8))
    assert len(bad) == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"
    bits = lambda x: np.where(x == 0, np.uint32(0), np.ascontiguousarray(x, np.float32).view(np.uint32))
    assert np.array_equal(bits(ws), bits(w_scaled)), "w_scaled"


def check_scores(wl, q_idx, scores, rows=None, sample=None, rng=None, q_dtype=None, w=None):
    """Compare GPU scores with the oracle: every visible token of the listed
    (b, p) rows, or a random sample of tokens per row when ``sample`` is set.
    q_dtype / w override the workload's query type and head weights."""
    B, P = wl.B, wl.P
    q_dtype = q_dtype or wl.q_dtype
    w = wl.w if w is None else w
    rows = rows if rows is not None else [(b, p) for b in range(B) for p in range(P)]
    worst = 0.0
    if sample is None:
        S = o_idx.indexer_scores(q_idx, q_dtype, w, wl.idx_pool, wl.k_dtype, wl.idx_scale,
                                 wl.idx_bt, wl.ctx_len, wl.bias, T_stride=wl.T_stride)
    for b, p in rows:
        n = max(o_idx.visible_limit(int(wl.ctx_len[b]), P, p) + 1, 0)
        if n == 0:
            continue
        if sample is None:
            ref = S[b, p, :n]
            got = scores[b, p, :n].astype(np.float64)
        else:
            toks = np.unique(np.concatenate([rng.integers(0, n, sample), [0, n - 1]]))
            ref = o_idx.indexer_scores_at(q_idx, q_dtype, w, wl.idx_pool, wl.k_dtype,
                                          wl.idx_scale, wl.idx_bt, b, p, toks, wl.bias)
            got = scores[b, p, toks].astype(np.float64)
        scale = max(np.max(np.abs(ref)), 1e-30)
        err = float(np.max(np.abs(got - ref)) / scale)
        worst = max(worst, err)
        assert err <= SCORE_RTOL, (b, p, err)
    return worst, (S if sample is None else None)


def check_topk_exact(wl, scores, topk):
    """GPU top-K equals the oracle top-K of the very same (GPU) scores."""
    ref = o_topk.topk(scores.astype(np.float64), wl.ctx_len, wl.K)
    bad = np.argwhere(np.any(ref != topk, axis=2))
    assert len(bad) == 0, f"top-K differs for (b,p) {bad[:5].tolist()}"


def check_topk_vs_oracle_scores(wl, S_oracle, topk):
    """Against the oracle's own scores: equal sizes, and every token in the
    symmetric difference scores within 1e-3 relative of the K-th score."""
    n_swaps = 0
    for b in range(wl.B):
        for p in range(wl.P):
            n = max(o_idx.visible_limit(int(wl.ctx_len[b]), wl.P, p) + 1, 0)
            G = topk[b, p][topk[b, p] >= 0]
            O = o_topk.topk_row(S_oracle[b, p], n, wl.K)
            O = O[O >= 0]
            assert len(G) == len(O) == min(n, wl.K)
            diff = np.setxor1d(G, O)
            if len(diff) == 0:
                continue
            sk = o_topk.kth_score(S_oracle[b, p], n, wl.K)
            assert np.all(np.abs(S_oracle[b, p, diff] - sk) <= TOPK_TIE_REL * abs(sk)), (b, p)
            n_swaps += len(diff)
    return n_swaps


def check_topk_vs_oracle_scores_rows(wl, q_idx, topk, requests, q_dtype=None, w=None):
    """check_topk_vs_oracle_scores for the listed requests only, with the
    oracle's scores computed for those requests alone (full-size workloads)."""
    n_swaps = 0
    q_dtype = q_dtype or wl.q_dtype
    w = wl.w if w is None else w
    for b in requests:
        sl = [b]
        S = o_idx.indexer_scores(q_idx[sl], q_dtype, w[sl], wl.idx_pool, wl.k_dtype,
                                 wl.idx_scale, wl.idx_bt[sl], wl.ctx_len[sl],
                                 None if wl.bias is None else wl.bias[sl], T_stride=wl.T_stride)
        for p in range(wl.P):
            n = max(o_idx.visible_limit(int(wl.ctx_len[b]), wl.P, p) + 1, 0)
            G = topk[b, p][topk[b, p] >= 0]
            O = o_topk.topk_row(S[0, p], n, wl.K)
            O = O[O >= 0]
            assert len(G) == len(O) == min(n, wl.K)
            diff = np.setxor1d(G, O)
            if len(diff):
                sk = o_topk.kth_score(S[0, p], n, wl.K)
                assert np.all(np.abs(S[0, p, diff] - sk) <= TOPK_TIE_REL * abs(sk)), (b, p)
                n_swaps += len(diff)
    return n_swaps


def check_resolve(wl, ostate, topk, got: dict):
    """Bit-exact: rows, counts, fault lists, tables, step and error bits."""
    new, rr = o_res.resolve(topk, ostate)
    assert np.array_equal(got["row_ids"], rr.row_ids), "row ids"
    assert np.array_equal(got["counts"], rr.counts), (got["counts"][:4], rr.counts[:4])
    for b in range(wl.B):
        n = rr.counts[b, 2]
        assert np.array_equal(got["faults"][b, :n], rr.faults[b]), f"faults of request {b}"
    assert got["step"] == new.step and got["err"] == rr.err
    if wl.C:
        for name in ("tok2slot", "slot2tok", "stamp"):
            assert np.array_equal(got[name], getattr(new, name)), name
    return new, rr


def check_copies(wl, rr, pool, row_scale, max_per_request=None):
    """Every faulted row's bytes (and scale) in every layer equal the host row."""
    for b in range(wl.B):
        cl = rr.copies[b]
        if max_per_request is not None:
            cl = cl[:max_per_request]
        for hr, pr in cl:
            bb, t = divmod(int(hr), wl.T_stride)
            assert bb == b
            for l in range(wl.L):
                assert np.array_equal(pool[l, pr], wl.lat[l, b, t]), (b, t, l)
                if row_scale is not None:
                    assert row_scale[l, pr] == wl.lat_scale[l, b, t // 64]


def lse_bound(tol, ref_lse):
    """Allowed |lse_gpu - lse_ref|.  e^d - 1 is the relative error of the
    softmax normaliser.  The logits are exact products of bf16 queries and
    bf16-exact rows summed in fp32 on the GPU, so lse does not see the bf16
    rounding of the probabilities that sets the 2e-2 output budget of the fp8
    path: the bound is min(tol, 1e-3) relative to max(1, |lse|), i.e. 1e-5
    relative in fp32 and 1e-3 relative on the fp8 path."""
    return min(tol, 1e-3) * np.maximum(1.0, np.abs(ref_lse))


def check_attention(wl, q_layers, topk, out, lse, tol, pairs=None):
    """Max relative error per output vector against the oracle over the same
    selection, and the log-sum-exp within lse_bound."""
    worst = 0.0
    for l in range(wl.L):
        ref_o, ref_l = o_attn.sparse_mla(q_layers[l], wl.q_dtype, wl.lat[l],
                                         None if wl.lat_scale is None else wl.lat_scale[l],
                                         wl.kv_dtype, topk, wl.sm_scale, pairs=pairs)
        todo = pairs if pairs is not None else [(b, p) for b in range(wl.B) for p in range(wl.P)]
        for b, p in todo:
            e = o_attn.max_rel_err(out[l, b, p], ref_o[b, p])
            worst = max(worst, e)
            assert e <= tol, (l, b, p, e)
            fin = np.isfinite(ref_l[b, p])
            assert np.array_equal(fin, np.isfinite(lse[l, b, p]))
            if fin.any():
                d = np.abs(lse[l, b, p][fin].astype(np.float64) - ref_l[b, p][fin])
                assert np.all(d <= lse_bound(tol, ref_l[b, p][fin])), (l, b, p, float(d.max()))
    return worst


def gpu_outputs(ds) -> dict:
    import torch
    torch.cuda.synchronize()
    g = {"scores": ds.scores.cpu().numpy(), "topk": ds.topk.cpu().numpy(),
         "row_ids": ds.row_ids.cpu().numpy(), "counts": ds.counts.cpu().numpy(),
         "faults": ds.faults.cpu().numpy(), "out": ds.out.cpu().numpy(),
         "lse": ds.lse.cpu().numpy()}
    g.update(ds.state_numpy())
    return g


def full_check(ds, wl, ostate, s=1, attn_tol=2e-2, check_oracle_topk=True, pairs=None,
               score_sample=None, rng=None, copies=True, copy_limit=None):
    """Check every stage of GPU step s (already run on the device step `ds`).
    When ds quantizes the indexer's queries, the quantization is checked first
    and the scores are compared with the oracle's indexer on its own codes."""
    q_idx, q = wl.step_inputs(s)
    g = gpu_outputs(ds)
    indexer_q = getattr(ds, "indexer_q", None)
    if indexer_q == "e4m3":
        check_quantized(q_idx, wl.w, ds.q8.cpu().numpy(), ds.w_scaled.cpu().numpy())
    qi, qdt, w = indexer_queries(wl, q_idx, indexer_q)
    worst_s, S = check_scores(wl, qi, g["scores"], sample=score_sample,
                              rng=rng or np.random.default_rng(0), q_dtype=qdt, w=w)
    check_topk_exact(wl, g["scores"], g["topk"])
    swaps = 0
    if check_oracle_topk and S is not None:
        swaps = check_topk_vs_oracle_scores(wl, S, g["topk"])
    new, rr = check_resolve(wl, ostate, g["topk"], g)
    if copies and wl.C:
        pool = ds.pool.cpu().numpy()
        rsc = None if ds.row_scale is None else ds.row_scale.cpu().numpy()
        check_copies(wl, rr, pool, rsc, copy_limit)
    worst_a = check_attention(wl, q, g["topk"], g["out"], g["lse"], attn_tol, pairs)
    return new, rr, {"score_err": worst_s, "attn_err": worst_a, "topk_swaps": swaps,
                     "counts": g["counts"]}


# ------------------------------------------------------------------ decode loop with append

def cache_mirror(wl):
    """The oracle's own copy of the tables a KV append changes (oracle/cache_ops
    state): block tables, indexer cache, free lists, and a zero latent pool of the
    workload's size (only the appended rows are ever compared)."""
    from oracle import cache_ops as o_co
    L, n_rows = wl.L, wl.n_pool_blocks * 64
    dt = np.float32 if wl.kv_dtype == "f32" else np.uint8
    return o_co.CacheState(
        ctx_len=wl.ctx_len.copy(), bt=wl.bt.copy(), idx_bt=wl.idx_bt.copy(),
        host_bt=wl.host_bt.copy(), pool=np.zeros((L, n_rows, 576), dt),
        row_scale=None if wl.lat_scale is None else np.zeros((L, n_rows), np.float32),
        idx_pool=wl.idx_pool.copy(), idx_scale=None if wl.idx_scale is None else wl.idx_scale.copy(),
        host_rows=np.zeros((L, 1, 576), dt), host_scale=None,
        free=[int(x) for x in wl.free_blocks], idx_free=[int(x) for x in wl.idx_free_blocks],
        free_capacity=len(wl.free_blocks))


def append_and_check(ds, wl, ostate, cs, s):
    """The KV append after step s, on the device (ds.append) and in the oracle (on
    the mirror cs); the device's tables, free lists, indexer cache and appended
    latent rows must equal the oracle's.  Then the logical workload and the
    oracle residency state follow the append, for the next step's checks."""
    import torch
    from oracle import cache_ops as o_co
    n_new, rows, rsc, keys, ksc = wl.append_inputs(s)
    t_new = cs.ctx_len.astype(np.int64).copy()
    assert o_co.append_tokens(cs, n_new, rows, rsc, keys, ksc) == 0
    ds.append(s)
    torch.cuda.synchronize()

    def eq(d, h, what):
        np.testing.assert_array_equal(d.cpu().numpy(), h, err_msg=f"after step {s}: {what}")
    eq(ds.ctx_len, cs.ctx_len, "ctx_len")
    eq(ds.bt, cs.bt, "bt")
    eq(ds.idx_bt, cs.idx_bt, "idx_bt")
    for b in range(wl.B):                  # the indexer blocks of the pages appended to
        for t in range(int(t_new[b]), int(cs.ctx_len[b])):
            blk = int(cs.idx_bt[b, t // 64])
            eq(ds.idx_pool[blk], cs.idx_pool[blk], f"indexer block {blk}")
    if cs.idx_scale is not None:
        eq(ds.idx_scale.view(torch.int32), cs.idx_scale.view(np.int32), "indexer scales")
    assert int(ds.free_n.item()) == len(cs.free), "latent free list"
    assert int(ds.idx_free_n.item()) == len(cs.idx_free), "indexer free list"
    assert ds.free[:len(cs.free)].cpu().numpy().tolist() == cs.free
    assert ds.idx_free[:len(cs.idx_free)].cpu().numpy().tolist() == cs.idx_free
    assert int(ds.err.item()) == 0
    for b in range(wl.B):
        for i, t in enumerate(range(int(t_new[b]), int(cs.ctx_len[b]))):
            row = int(cs.bt[b, t // 64]) * 64 + t % 64
            eq(ds.pool[:, row], cs.pool[:, row], f"latent row of token {t}, request {b}")
            if cs.row_scale is not None:
                eq(ds.row_scale[:, row].view(torch.int32), cs.row_scale[:, row].view(np.int32),
                   f"row scale of token {t}, request {b}")
            assert np.array_equal(cs.pool[:, row], rows[b, i])
    wl.ctx_len[:] = cs.ctx_len
    wl.bt[:] = cs.bt
    wl.idx_bt[:] = cs.idx_bt
    ostate.bt[:] = cs.bt
    for b in range(wl.B):
        for t in range(int(t_new[b]), int(cs.ctx_len[b])):
            blk = int(cs.idx_bt[b, t // 64])
            wl.idx_pool[blk] = cs.idx_pool[blk]
            if cs.idx_scale is not None:
                wl.idx_scale[blk] = cs.idx_scale[blk]
    return ostate
