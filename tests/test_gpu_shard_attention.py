"""GPU parity of the token-sharded attention and of head groups, through the C ABI.

hs_sparse_mla_decode_sharded against the oracle's sharded attention (which the
CPU tests pin equal to the global attention): every shard's fragment (output
and log-sum-exp), and the merged output and log-sum-exp, for S from 1 to 64,
shards holding from zero to 8192 selected rows (one to 32 chunks of 256 rows),
empty and short requests, K from 1 to 8192, 16 to 128 heads, fp32 and E4M3
rows; then end to end behind hs_topk_sharded.  hs_sparse_mla_decode and
hs_sparse_mla_decode_layers with 32, 64 and 128 heads against the oracle's
attention over the same rows.
"""
import sys

import numpy as np
import pytest

from oracle import attention as o_attn, numerics as o_num, topk as o_topk
from workloads import gen
import gpu_check as gc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SM = 1.0 / 24.0


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_indexer_logits_amd import _lib
    _lib.load()


def _latent(rng, kv, B, Ts):
    """Logical latent [B, Ts, 576] and its per-64-token scales (E4M3)."""
    if kv == "e4m3":
        lat = rng.integers(0, 256, (B, Ts, 576), dtype=np.uint8)
        lat[(lat & 0x7F) == 0x7F] = 0                       # no NaN codes
        scale = (rng.random((B, Ts // 64)) * 0.02 + 1e-3).astype(np.float32)
        return lat, scale
    return rng.standard_normal((B, Ts, 576)).astype(np.float32), None


def _queries(rng, kv, shape):
    if kv == "e4m3":
        return gen.bf16_bits(rng.standard_normal(shape)), "bf16"
    return rng.standard_normal(shape).astype(np.float32), "f32"


def _selection(rng, ctx, P, K):
    """Ascending distinct visible tokens per (b, p), -1 after them; the first
    position of request 0 takes its first min(K, ctx) tokens (its first shards
    dense, the rest empty), every other position a uniform sample."""
    B = len(ctx)
    topk = np.full((B, P, K), -1, dtype=np.int32)
    for b, n in enumerate(ctx):
        for p in range(P):
            m = min(K, int(n))
            dense = b == 0 and p == 0
            sel = np.arange(m) if dense else np.sort(rng.choice(int(n), m, replace=False))
            topk[b, p, :m] = sel
    return topk


def _device(lat, scale, q, topk):
    B, Ts = lat.shape[:2]
    pool = torch.from_numpy(lat.reshape(B * Ts, 576)).cuda()
    rs = None if scale is None else torch.from_numpy(np.repeat(scale, 64, axis=1).reshape(-1)).cuda()
    rid = np.where(topk >= 0, np.arange(B, dtype=np.int64)[:, None, None] * Ts + topk, -1)
    qd = torch.from_numpy(q.view(np.int16) if q.dtype == np.uint16 else q).cuda()
    return pool, rs, torch.from_numpy(rid.astype(np.int32)).cuda(), qd


def _run_sharded(lat, scale, q, qt, kv, topk, ctx, S, topk_dev=None):
    from decode_indexer_logits_amd import _lib
    B, P, Hq, _ = q.shape
    Ts, K = lat.shape[1], topk.shape[2]
    d_ctx = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).cuda()
    batch = _lib.make_batch(B, P, Ts, d_ctx)
    pool, rs, rid, qd = _device(lat, scale, q, topk)
    tk = torch.from_numpy(topk).cuda() if topk_dev is None else topk_dev
    shard_out = torch.full((B, P, S, Hq, 512), float("nan"), device="cuda")
    shard_lse = torch.full((B, P, S, Hq), float("nan"), device="cuda")
    out = torch.full((B, P, Hq, 512), float("nan"), device="cuda")
    lse = torch.full((B, P, Hq), float("nan"), device="cuda")
    need = _lib.mla_sharded_workspace_bytes(B, P, K, S, Hq)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")   # contents do not matter
    _say(f"sharded attention B={B} P={P} Ts={Ts} K={K} S={S} Hq={Hq} kv={kv}")
    _lib.sparse_mla_decode_sharded(batch, K, S, Hq, qt, qd, kv, pool, rs, tk, rid, SM, shard_out,
                                   shard_lse, out, lse, ws)
    torch.cuda.synchronize()
    return (shard_out.cpu().numpy(), shard_lse.cpu().numpy(), out.cpu().numpy(),
            lse.cpu().numpy())


def _check_sharded(got, lat, scale, q, qt, kv, topk, S):
    g_so, g_sl, g_o, g_l = got
    tol = 2e-2 if kv == "e4m3" else 1e-5
    r_o, r_l, r_so, r_sl = o_attn.sparse_mla_sharded(q, qt, lat, scale, kv, topk, SM,
                                                     lat.shape[1] // S)
    B, P = topk.shape[:2]
    worst = 0.0
    for b in range(B):
        for p in range(P):
            for s in range(S):
                fin = np.isfinite(r_sl[b, p, s])
                assert np.array_equal(fin, np.isfinite(g_sl[b, p, s])), (b, p, s)
                if not fin.any():                       # a shard with no selected row
                    assert np.all(g_so[b, p, s] == 0.0) and np.all(g_sl[b, p, s] == -np.inf)
                    continue
                e = o_attn.max_rel_err(g_so[b, p, s], r_so[b, p, s])
                worst = max(worst, e)
                assert e <= tol, (b, p, s, e)
                d = np.abs(g_sl[b, p, s].astype(np.float64) - r_sl[b, p, s])
                assert np.all(d <= gc.lse_bound(tol, r_sl[b, p, s])), (b, p, s, float(d.max()))
            fin = np.isfinite(r_l[b, p])
            assert np.array_equal(fin, np.isfinite(g_l[b, p])), (b, p)
            if not fin.any():
                assert np.all(g_o[b, p] == 0.0)
                continue
            e = o_attn.max_rel_err(g_o[b, p], r_o[b, p])
            worst = max(worst, e)
            assert e <= tol, (b, p, e)
            d = np.abs(g_l[b, p].astype(np.float64) - r_l[b, p])
            assert np.all(d <= gc.lse_bound(tol, r_l[b, p])), (b, p, float(d.max()))
    return worst


@pytest.mark.parametrize("kv,S,Ts,K,Hq,P", [
    ("f32", 1, 4096, 512, 16, 1),
    ("e4m3", 2, 4096, 2048, 16, 1),          # four chunks per shard
    ("e4m3", 8, 4096, 2048, 16, 2),
    ("f32", 3, 3072, 700, 32, 2),            # two head groups, S not a power of two
    ("e4m3", 64, 8192, 2048, 16, 1),         # 128-token shards
    ("e4m3", 6, 6144, 1, 16, 1),             # one row
    ("e4m3", 1, 16384, 8192, 16, 1),         # 32 chunks in one shard
    ("e4m3", 16, 16384, 8192, 64, 1),
    ("e4m3", 4, 4096, 1024, 128, 1),
])
def test_sharded_attention_matches_oracle(kv, S, Ts, K, Hq, P):
    rng = np.random.default_rng(1000 + 7 * S + K + Hq + P)
    # full, empty, one token, within the first shard, just past a shard edge
    ctx = np.clip(np.array([Ts, 0, 1, Ts // S - 3, Ts // S + 5, Ts - 17]), 0, Ts)
    B = len(ctx)
    lat, scale = _latent(rng, kv, B, Ts)
    q, qt = _queries(rng, kv, (B, P, Hq, 576))
    topk = _selection(rng, ctx, P, K)
    got = _run_sharded(lat, scale, q, qt, kv, topk, ctx, S)
    worst = _check_sharded(got, lat, scale, q, qt, kv, topk, S)
    _say("worst relative error", worst)


def test_sharded_topk_then_sharded_attention():
    """Scores -> hs_topk_sharded -> hs_sparse_mla_decode_sharded, the selection
    checked bit for bit against the oracle's sharded top-K and the attention
    against the oracle's sharded attention over that selection."""
    from decode_indexer_logits_amd import _lib
    rng = np.random.default_rng(4242)
    B, Ts, K, S, Hq = 4, 65536, 2048, 8, 64
    ctx = np.array([Ts, Ts - 1000, 3 * (Ts // S) + 11, 1500])
    scores = (np.round(rng.standard_normal((B, Ts)) * 16) / 16).astype(np.float32)
    d_ctx = torch.from_numpy(ctx.astype(np.int32)).cuda()
    batch = _lib.make_batch(B, 1, Ts, d_ctx)
    d_scores = torch.from_numpy(scores.reshape(B, 1, Ts)).cuda()
    tk = torch.empty((B, 1, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(_lib.topk_sharded_workspace_bytes(B, Ts, K, S), dtype=torch.uint8,
                     device="cuda")
    _say("sharded top-K then sharded attention, B=4 Ts=65536 K=2048 S=8 Hq=64")
    _lib.topk_sharded(batch, K, S, d_scores, tk, ws)
    torch.cuda.synchronize()
    topk = tk.cpu().numpy()
    for b in range(B):
        want = o_topk.topk_sharded_row(scores[b].astype(np.float64), int(ctx[b]), K, Ts // S)
        assert np.array_equal(topk[b, 0], want), b
    lat, scale = _latent(rng, "e4m3", B, Ts)
    q, qt = _queries(rng, "e4m3", (B, 1, Hq, 576))
    got = _run_sharded(lat, scale, q, qt, "e4m3", topk, ctx, S, topk_dev=tk)
    _check_sharded(got, lat, scale, q, qt, "e4m3", topk, S)


@pytest.mark.parametrize("Hq", [32, 64, 128])
@pytest.mark.parametrize("kv", ["e4m3", "f32"])
def test_head_groups_single_and_layers_calls(kv, Hq):
    """Hq = 16 G heads: every head of every (request, position) of a single
    call and of a two-layer call against the oracle over the same rows."""
    from decode_indexer_logits_amd import _lib
    rng = np.random.default_rng(500 + Hq + (kv == "f32"))
    B, P, K, L, n_rows = 3, 2, 1000, 2, 4096
    ctx = torch.tensor([K] * B, dtype=torch.int32, device="cuda")
    batch = _lib.make_batch(B, P, 1024, ctx)
    rid = np.stack([rng.choice(n_rows, K, replace=False) for _ in range(B * P)]).astype(np.int32)
    rid[1, 600:] = -1                                   # a short selection
    rid[4, :] = -1                                      # none at all
    rid = rid.reshape(B, P, K)
    row_ids = torch.from_numpy(rid).cuda()
    if kv == "e4m3":
        qn = gen.bf16_bits(rng.standard_normal((L, B, P, Hq, 576)))
        q = torch.from_numpy(qn.view(np.int16)).cuda()
        pn = rng.integers(0, 256, (L, n_rows, 576), dtype=np.uint8)
        pn[(pn & 0x7F) == 0x7F] = 0
        rsn = (rng.random((L, n_rows)) * 0.02).astype(np.float32)
        qt, tol = "bf16", 2e-2
    else:
        qn = rng.standard_normal((L, B, P, Hq, 576)).astype(np.float32)
        q = torch.from_numpy(qn).cuda()
        pn = rng.standard_normal((L, n_rows, 576)).astype(np.float32)
        rsn = None
        qt, tol = "f32", 1e-5
    pool = torch.from_numpy(pn).cuda()
    rs = None if rsn is None else torch.from_numpy(rsn).cuda()
    ws = torch.empty(max(_lib.mla_layers_workspace_bytes(B, P, K, Hq, L),
                         _lib.workspace_bytes(_lib.HS_OP_MLA, B, P, 1024, K, Hq), 16),
                     dtype=torch.uint8, device="cuda")
    _say(f"head groups Hq={Hq} kv={kv}")
    one = torch.full((B, P, Hq, 512), float("nan"), device="cuda")
    one_lse = torch.full((B, P, Hq), float("nan"), device="cuda")
    _lib.sparse_mla_decode(batch, K, Hq, qt, q[0], kv, pool[0], None if rs is None else rs[0],
                           row_ids, SM, one, one_lse, ws)
    outL = torch.full((L, B, P, Hq, 512), float("nan"), device="cuda")
    lseL = torch.full((L, B, P, Hq), float("nan"), device="cuda")
    _lib.sparse_mla_decode_layers(batch, K, Hq, L, qt, q, kv, pool, n_rows, rs, row_ids, SM,
                                  outL, lseL, ws)
    torch.cuda.synchronize()
    results = [(0, one.cpu().numpy(), one_lse.cpu().numpy())]
    results += [(l, outL[l].cpu().numpy(), lseL[l].cpu().numpy()) for l in range(L)]
    for l, o, ls in results:
        for b in range(B):
            for p in range(P):
                sel = rid[b, p][rid[b, p] >= 0]
                x = o_num.to_f64(pn[l][sel], kv)
                if rsn is not None:
                    x = x * rsn[l][sel].astype(np.float64)[:, None]
                ro, rl = o_attn.attend(o_num.to_f64(qn[l, b, p], qt), x, SM)
                if sel.size == 0:
                    assert np.all(o[b, p] == 0.0) and np.all(ls[b, p] == -np.inf)
                    continue
                assert o_attn.max_rel_err(o[b, p], ro) <= tol, (l, b, p)
                assert np.all(np.abs(ls[b, p] - rl) <= gc.lse_bound(tol, rl)), (l, b, p)


def test_head_groups_long_slices_shared_tile_kernel():
    """Many request-positions and 32 heads: slices of 1024 rows, which go to the
    shared-tile attention kernel; every head of every position against the
    oracle over the same rows."""
    from decode_indexer_logits_amd import _lib
    rng = np.random.default_rng(77)
    B, P, K, Hq, n_rows = 32, 4, 2048, 32, 16384
    ctx = torch.tensor([4096] * B, dtype=torch.int32, device="cuda")
    batch = _lib.make_batch(B, P, 4096, ctx)
    rid = np.stack([rng.choice(n_rows, K, replace=False) for _ in range(B * P)]).astype(np.int32)
    rid[5, 1500:] = -1
    rid = rid.reshape(B, P, K)
    qn = gen.bf16_bits(rng.standard_normal((B, P, Hq, 576)))
    pn = rng.integers(0, 256, (n_rows, 576), dtype=np.uint8)
    pn[(pn & 0x7F) == 0x7F] = 0
    rsn = (rng.random(n_rows) * 0.02).astype(np.float32)
    ws = torch.empty(max(_lib.workspace_bytes(_lib.HS_OP_MLA, B, P, 4096, K, Hq), 16),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((B, P, Hq, 512), float("nan"), device="cuda")
    lse = torch.full((B, P, Hq), float("nan"), device="cuda")
    _say("head groups, long slices: B=32 P=4 K=2048 Hq=32")
    _lib.sparse_mla_decode(batch, K, Hq, "bf16", torch.from_numpy(qn.view(np.int16)).cuda(), "e4m3",
                           torch.from_numpy(pn).cuda(), torch.from_numpy(rsn).cuda(),
                           torch.from_numpy(rid).cuda(), SM, out, lse, ws)
    torch.cuda.synchronize()
    o, ls = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for p in range(P):
            sel = rid[b, p][rid[b, p] >= 0]
            x = o_num.to_f64(pn[sel], "e4m3") * rsn[sel].astype(np.float64)[:, None]
            ro, rl = o_attn.attend(o_num.to_f64(qn[b, p], "bf16"), x, SM)
            assert o_attn.max_rel_err(o[b, p], ro) <= 2e-2, (b, p)
            assert np.all(np.abs(ls[b, p] - rl) <= gc.lse_bound(2e-2, rl)), (b, p)
