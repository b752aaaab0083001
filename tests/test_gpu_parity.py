"""GPU parity of the HIP decode step against the oracle, through the C ABI.

Sizes here finish in seconds on the oracle and still span many tiles, ragged
contexts and the degenerate cases; the full-size workloads are in
test_gpu_fullsize.py.
"""
import dataclasses
import sys

import numpy as np
import pytest

from workloads import gen
from workloads.calibrate_mixed import calibrate
import gpu_check as gc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_indexer_logits_amd import _lib
    _lib.load()


def _run(wl, s=1, **kw):
    from decode_indexer_logits_amd.device import DeviceStep
    ds = DeviceStep(wl)
    if s != 1:
        ds.set_queries(s)
    ds.run()
    return ds


@pytest.mark.parametrize("K", [256, 4096, 8192])
def test_tiny_fp32(K):
    _say(f"tiny_fp32 K={K}")
    wl = gen.tiny_fp32(K=K)
    ds = _run(wl)
    _, _, info = gc.full_check(ds, wl, gc.oracle_state(wl), attn_tol=1e-5)
    _say(info)
    if K >= 4096:
        # K >= context: sparse attention over all rows = dense attention
        from oracle import attention as oa
        g = gc.gpu_outputs(ds)
        do, dl = oa.dense_mla(wl.q[0], "f32", wl.lat[0], None, "f32", wl.ctx_len, wl.sm_scale)
        assert oa.max_rel_err(g["out"][0], do) <= 1e-5
        assert np.max(np.abs(g["lse"][0] - dl)) <= 1e-5


def test_tiny_fp32_ragged_and_short():
    # a context that is not a multiple of 64 and shorter than K
    for T, K in ((4000, 256), (100, 256), (1, 8)):
        _say(f"tiny_fp32 T={T} K={K}")
        wl = gen.tiny_fp32(K=K, T=T)
        ds = _run(wl)
        gc.full_check(ds, wl, gc.oracle_state(wl), attn_tol=1e-5)


def test_resident_fp8():
    _say("resident_fp8 full size")
    wl = gen.resident_fp8()
    ds = _run(wl)
    _, _, info = gc.full_check(ds, wl, gc.oracle_state(wl), attn_tol=2e-2)
    _say(info)


def test_resident_fp8_ragged_batch():
    _say("resident_fp8 ragged small")
    wl = gen.resident_fp8(B=5, T_lo=1, T_hi=3000, K=512)
    ds = _run(wl)
    _, _, info = gc.full_check(ds, wl, gc.oracle_state(wl), attn_tol=2e-2)
    _say(info, wl.ctx_len)


def test_empty_single_and_page_edge_requests():
    """A request with no tokens (every output -1, attention output 0 and lse
    -inf), one token, and contexts at and around page edges, shorter and
    longer than K, through the whole step."""
    _say("edge contexts [0, 1, 63, 64, 65, 130, 2000]")
    wl = gen.resident_fp8(K=128, ctx_len=[0, 1, 63, 64, 65, 130, 2000])
    ds = _run(wl)
    _, _, info = gc.full_check(ds, wl, gc.oracle_state(wl), attn_tol=2e-2)
    g = gc.gpu_outputs(ds)
    assert np.all(g["topk"][0] == -1) and np.all(g["out"][:, 0] == 0)
    assert np.all(np.isneginf(g["lse"][:, 0]))
    assert np.array_equal(g["topk"][1, 0, :2], [0, -1])
    _say(info)


def _mixed_small(B=4, T=16384, K=512, tail=1024, seed=1003):
    beta, hot, frac = calibrate(seed=seed, B=B, T=T, K=K, tail=tail)
    return gen.mixed_128k(seed=seed, B=B, T=T, K=K, tail=tail, beta=beta, hot_tokens=hot)


def test_mixed_small_faults_hits_evictions():
    _say("mixed small")
    wl = _mixed_small()
    ds = _run(wl)
    new, rr, info = gc.full_check(ds, wl, gc.oracle_state(wl), attn_tol=2e-2)
    _say(info)
    c = info["counts"]
    assert np.all(c[:, 1] >= wl.K // 2 - 16)      # about half of the top-K hit
    assert np.all(c[:, 2] > 0) and np.all(c[:, 3] == c[:, 2])   # full buffers: every fault evicts


def test_maximum_sizes_k8192_hot16384():
    """The largest supported selection and hot buffer: K = 8192 (P*K = 8192
    entries per request in resolve) with C = 2K = 16384 hot rows (16 slots per
    resolve thread), rows of 40960 tokens."""
    _say("mixed K=8192 C=16384")
    wl = _mixed_small(B=2, T=40960, K=8192, tail=1024)
    assert wl.C == 16384 and wl.K == 8192
    ds = _run(wl)
    new, rr, info = gc.full_check(ds, wl, gc.oracle_state(wl), attn_tol=2e-2)
    _say(info)
    assert np.all(info["counts"][:, 2] > 0)


def test_single_row_selection_k1():
    """K = 1: the best token alone; attention over one row returns that row."""
    _say("tiny_fp32 K=1")
    wl = gen.tiny_fp32(K=1)
    ds = _run(wl)
    gc.full_check(ds, wl, gc.oracle_state(wl), attn_tol=1e-5)


def test_mtp3_small_multi_step():
    _say("mtp3 small, 3 steps")
    wl = gen.mtp3_agentic(B=3, K=128, steps=3, first_turn=6000, per_turn=300, turns=5, out_max=50)
    from decode_indexer_logits_amd.device import DeviceStep
    ds = DeviceStep(wl)
    ost = gc.oracle_state(wl)
    for s in range(1, wl.steps + 1):
        ds.set_queries(s)
        ds.run()
        ost, rr, info = gc.full_check(ds, wl, ost, s=s, attn_tol=2e-2)
        _say(s, info["counts"].tolist())


@pytest.mark.parametrize("P", [2, 3])
def test_speculative_positions_two_and_three(P):
    """P = 2 and 3 query positions (the shared-key indexer splits a page's
    groups between two waves per position at P = 2 and leaves one converting
    wave idle at P = 3); two steps, every stage against the oracle."""
    _say(f"mtp P={P} small, 2 steps")
    wl = gen.mtp3_agentic(B=3, K=128, steps=2, first_turn=9000, per_turn=300, turns=5,
                          out_max=50, P=P)
    from decode_indexer_logits_amd.device import DeviceStep
    ds = DeviceStep(wl)
    ost = gc.oracle_state(wl)
    for s in range(1, wl.steps + 1):
        ds.set_queries(s)
        ds.run()
        ost, rr, info = gc.full_check(ds, wl, ost, s=s, attn_tol=2e-2)
        _say(s, info["counts"].tolist())


@pytest.mark.parametrize("layout", ["interleaved", "layer_major"])
def test_norescache_small_hit_rate_warms_up(layout):
    """Four steps from an empty hot buffer with two layers, the host pool laid
    out with the layers of a token together or one plane per layer."""
    _say(f"no-residency small, 4 steps, host pool {layout}")
    wl = gen.norescache_1m(B=2, T=32768, K=256, L=2, steps=4)
    from decode_indexer_logits_amd.device import DeviceStep
    ds = DeviceStep(wl, host_layout=layout)
    ost = gc.oracle_state(wl)
    rates = []
    for s in range(1, wl.steps + 1):
        ds.set_queries(s)
        ds.run()
        ost, rr, info = gc.full_check(ds, wl, ost, s=s, attn_tol=2e-2)
        c = info["counts"]
        if s == 1:
            assert np.all(c[:, 1] == 0) and np.all(c[:, 2] == wl.K) and np.all(c[:, 3] == 0)
        rates.append(float(c[:, 1].sum() / max(c[:, 1].sum() + c[:, 2].sum(), 1)))
    _say("hit rates", rates)
    assert rates[0] == 0.0 and rates[-1] > 0.5


@pytest.mark.parametrize("layout,groups", [("interleaved", 0), ("layer_major", 0),
                                           ("interleaved", 2)])
def test_layer_pipelined_step_against_oracle(layout, groups):
    """The layers of one selection overlapped (fault copies one layer at a time
    on a second stream, each layer's attention behind its layer's copy): three
    steps from an empty hot buffer with four layers, every stage of every step
    against the oracle (tables, faulted rows of every layer, every layer's
    attention); tables, pool and step equal to the single-stream step's; then
    a captured graph of the first step replayed three times."""
    _say(f"layer-pipelined step, 4 layers, host pool {layout}, groups {groups}")
    wl = gen.norescache_1m(B=2, T=32768, K=256, L=4, steps=3)
    from decode_indexer_logits_amd.device import DeviceStep
    ds = DeviceStep(wl, host_layout=layout)
    ref = DeviceStep(wl, host_layout=layout)
    snap = ds.snapshot()
    ost = gc.oracle_state(wl)
    first = None
    for s in range(1, wl.steps + 1):
        ds.set_queries(s)
        ds.run_layer_pipelined(groups=groups)
        ref.set_queries(s)
        ref.run()
        ost, rr, info = gc.full_check(ds, wl, ost, s=s, attn_tol=2e-2)
        g, r = gc.gpu_outputs(ds), gc.gpu_outputs(ref)
        for k in ("topk", "row_ids", "counts", "tok2slot", "slot2tok", "stamp"):
            assert np.array_equal(g[k], r[k]), (s, k)
        assert g["step"] == r["step"] == wl.step + s and g["err"] == 0
        assert torch.equal(ds.pool, ref.pool) and torch.equal(ds.row_scale, ref.row_scale)
        if s == 1:
            first = g
        _say(s, info["counts"].tolist())
    ds.restore(snap)
    ds.set_queries(1)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            ds.run_layer_pipelined(groups=groups)
    torch.cuda.synchronize()
    for rep in range(3):
        ds.restore(snap)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = gc.gpu_outputs(ds)
        for k in ("topk", "row_ids", "counts", "out", "lse", "tok2slot", "slot2tok", "stamp"):
            assert np.array_equal(got[k], first[k]), ("graph", rep, k)
        assert got["step"] == first["step"]


def _relayout(wl, mode, seed=5):
    """The same logical data with every page resident ("full") or none ("none")."""
    B, nb = wl.B, wl.T_stride // 64
    rng = np.random.default_rng(seed)
    nblk = [-(-int(t) // 64) for t in wl.ctx_len]
    hot_b = wl.C // 64
    if mode == "full":
        n_res = sum(nblk)
    else:
        n_res = 0
    perm = rng.permutation(n_res + B * hot_b).astype(np.int32)
    bt = np.full((B, nb), -1, np.int32)
    off = 0
    if mode == "full":
        for b in range(B):
            bt[b, :nblk[b]] = perm[off:off + nblk[b]]
            off += nblk[b]
    hot = perm[off:].reshape(B, hot_b)
    return dataclasses.replace(wl, n_pool_blocks=n_res + B * hot_b, bt=bt, hot_blocks=hot,
                               tok2slot=np.full_like(wl.tok2slot, -1),
                               slot2tok=np.full_like(wl.slot2tok, -1),
                               stamp=np.zeros_like(wl.stamp), step=0)


def test_residency_invariance_bit_identical():
    _say("residency invariance")
    wl = _mixed_small(B=3, T=8192, K=256, tail=512)
    outs = {}
    for mode in ("mixed", "full", "none"):
        w = wl if mode == "mixed" else _relayout(wl, mode)
        ds = _run(w)
        g = gc.gpu_outputs(ds)
        gc.check_resolve(w, gc.oracle_state(w), g["topk"], g)
        outs[mode] = (g["topk"], g["out"], g["lse"], g["counts"])
        _say(mode, g["counts"].tolist())
    for mode in ("full", "none"):
        assert np.array_equal(outs[mode][0], outs["mixed"][0])
        assert np.array_equal(outs[mode][1], outs["mixed"][1]), mode
        assert np.array_equal(outs[mode][2], outs["mixed"][2]), mode
    assert np.all(outs["full"][3][:, 0] == wl.K) and np.all(outs["none"][3][:, 0] == 0)


def test_graph_capture_replays_match_eager():
    _say("graph capture")
    wl = _mixed_small(B=2, T=8192, K=256, tail=512)
    from decode_indexer_logits_amd.device import DeviceStep
    ds = DeviceStep(wl)
    snap = ds.snapshot()
    ds.run()
    ref = gc.gpu_outputs(ds)
    ds.restore(snap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ds.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        ds.restore(snap)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = gc.gpu_outputs(ds)
        for k in ("topk", "row_ids", "counts", "out", "lse", "tok2slot", "slot2tok", "stamp"):
            assert np.array_equal(got[k], ref[k]), (rep, k)
        assert got["step"] == ref["step"]
        _ = torch.ones(1024, device="cuda").sum().item()   # unrelated eager work between replays


def test_pipelined_step_matches_single_stream():
    _say("pipelined vs single stream")
    wl = _mixed_small(B=5, T=8192, K=256, tail=512)
    from decode_indexer_logits_amd.device import DeviceStep
    ds = DeviceStep(wl)
    snap = ds.snapshot()
    ds.run()
    ref = gc.gpu_outputs(ds)
    ref_pool = ds.pool.cpu().numpy()
    gc.check_resolve(wl, gc.oracle_state(wl), ref["topk"], ref)
    keys = ("scores", "topk", "row_ids", "counts", "out", "lse", "tok2slot", "slot2tok", "stamp")
    q = wl.step_inputs(1)[1]
    gc.check_attention(wl, q, ref["topk"], ref["out"], ref["lse"], 2e-2)
    for nchunks in (2, 3, 5):
        ds.restore(snap)
        ds.run_pipelined(nchunks)
        got = gc.gpu_outputs(ds)
        gc.check_resolve(wl, gc.oracle_state(wl), got["topk"], got)
        gc.check_attention(wl, q, got["topk"], got["out"], got["lse"], 2e-2)
        for k in keys:
            if k == "scores":
                for b in range(wl.B):
                    n = int(wl.ctx_len[b])
                    assert np.array_equal(got[k][b, :, :n], ref[k][b, :, :n])
            else:
                assert np.array_equal(got[k], ref[k]), (nchunks, k)
        assert got["step"] == ref["step"]
        assert np.array_equal(ds.pool.cpu().numpy(), ref_pool), nchunks
    # captured as one graph, replayed
    ds.restore(snap)
    ds.run_pipelined(3)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    ds.restore(snap)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ds.run_pipelined(3)
    torch.cuda.synchronize()
    for rep in range(3):
        ds.restore(snap)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = gc.gpu_outputs(ds)
        gc.check_attention(wl, q, got["topk"], got["out"], got["lse"], 2e-2)
        for k in keys[1:]:
            assert np.array_equal(got[k], ref[k]), ("graph", rep, k)


@pytest.mark.parametrize("stamps", ["distinct", "range100", "two"])
def test_resolve_victim_orders(stamps):
    # victims spread over many distinct stamps (the general radix-select path),
    # a moderate range, and only two stamps (the per-stamp fast path)
    _say(f"victim order: {stamps}")
    wl = _mixed_small(B=3, T=8192, K=256, tail=512)
    rng = np.random.default_rng(11)
    st = np.empty_like(wl.stamp)
    for b in range(wl.B):
        if stamps == "distinct":
            st[b] = rng.permutation(wl.C) + 1
        elif stamps == "range100":
            st[b] = rng.integers(1, 101, wl.C)
        else:
            st[b] = rng.integers(1, 3, wl.C)
    w2 = dataclasses.replace(wl, stamp=st.astype(np.int32), step=int(st.max()))
    ds = _run(w2)
    _, rr, info = gc.full_check(ds, w2, gc.oracle_state(w2), attn_tol=2e-2)
    _say(info["counts"].tolist())
    assert np.all(info["counts"][:, 3] > 0)


def test_pipelined_chunks_of_eight_against_oracle():
    # 32 requests in 4 chunks of 8, eager and as a graph: each replay checked
    # bit-exactly against the oracle's resolve of the same selection
    _say("pipelined B=32 in 4 chunks")
    wl = _mixed_small(B=32, T=16384, K=512, tail=1024)
    from decode_indexer_logits_amd.device import DeviceStep
    ds = DeviceStep(wl)
    snap = ds.snapshot()
    ds.run_pipelined(4)
    g1 = gc.gpu_outputs(ds)
    gc.check_resolve(wl, gc.oracle_state(wl), g1["topk"], g1)
    q = wl.step_inputs(1)[1]
    gc.check_attention(wl, q, g1["topk"], g1["out"], g1["lse"], 2e-2)
    assert np.all(g1["counts"][:, 3] == g1["counts"][:, 2])   # full buffers: every fault evicts
    ds.restore(snap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            ds.run_pipelined(4)
    torch.cuda.synchronize()
    for rep in range(3):
        ds.restore(snap)
        g.replay()
        got = gc.gpu_outputs(ds)
        gc.check_resolve(wl, gc.oracle_state(wl), got["topk"], got)
        for k in ("topk", "row_ids", "counts", "out", "lse"):
            assert np.array_equal(got[k], g1[k]), (rep, k)


@pytest.mark.parametrize("name", ["resident_fp8", "mtp3", "tiny"])
def test_fused_indexer_topk_matches_separate_calls(name):
    _say(f"fused indexer+top-K vs separate: {name}")
    if name == "resident_fp8":
        wl = gen.resident_fp8(B=4)
    elif name == "mtp3":
        wl = gen.mtp3_agentic(B=3, K=128, steps=1, first_turn=6000, per_turn=300, turns=5, out_max=50)
    else:
        wl = gen.tiny_fp32(K=256)
    from decode_indexer_logits_amd.device import DeviceStep
    ds = DeviceStep(wl)
    ds.run_indexer()
    ds.run_topk()
    torch.cuda.synchronize()
    s1, t1 = ds.scores.clone(), ds.topk.clone()
    ds.scores.fill_(float("nan"))
    ds.topk.fill_(-7)
    ds.run_indexer_topk()
    torch.cuda.synchronize()
    for b in range(wl.B):
        for p in range(wl.P):
            n = max(int(wl.ctx_len[b]) - wl.P + p + 1, 0)
            assert torch.equal(ds.scores[b, p, :n], s1[b, p, :n])
    assert torch.equal(ds.topk, t1)
    gc.check_topk_exact(wl, ds.scores.cpu().numpy(), ds.topk.cpu().numpy())


def test_fused_indexer_topk_workspace_reuse_and_halves():
    """The selection returns every workspace word it wrote to zero, so fused
    calls in a row on one workspace (zeroed once) stay exact whether B*P grows
    or shrinks (the histogram area of a larger batch covers the selections and
    candidates of a smaller one); the two halves (hs_indexer_topk_scores, then
    hs_indexer_topk_select) give the fused call's scores and top-K bit for
    bit; after hs_topk on a dirtied workspace the fused call is exact again."""
    from decode_indexer_logits_amd import _lib
    from oracle import topk as o_topk
    Ts, K = 16384, 512
    ws = torch.zeros(_lib.workspace_bytes(_lib.HS_OP_TOPK, 24, 1, Ts, K), dtype=torch.uint8,
                     device="cuda")

    def inputs(seed, B):
        rng = np.random.default_rng(seed)
        ctx = rng.integers(1, Ts + 1, B).astype(np.int32)
        ctx[0] = Ts
        x = gen.indexer_inputs(seed, ctx, Ts)
        dev = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).cuda()
               for k, v in x.items() if isinstance(v, np.ndarray)}
        batch = _lib.make_batch(B, 1, Ts, dev["ctx_len"])
        args = (x["H"], x["D"], "bf16", dev["q_idx"], dev["w"], "e4m3", dev["idx_pool"],
                dev["idx_scale"], dev["idx_bt"], dev["bias"])
        # dev is returned too: the batch holds the address of dev["ctx_len"]
        return ctx, batch, args, dev

    def fused(batch, args, B, w):
        s = torch.empty((B, 1, Ts), device="cuda")
        t = torch.full((B, 1, K), -7, dtype=torch.int32, device="cuda")
        _lib.indexer_topk(batch, *args, s, K, t, w)
        torch.cuda.synchronize()
        return s.cpu().numpy(), t.cpu().numpy()

    for seed, B in ((40, 7), (41, 24), (42, 24), (43, 7)):
        _say(f"fused indexer + top-K on a reused workspace: B={B}")
        ctx, batch, args, dev = inputs(seed, B)
        sc, tk = fused(batch, args, B, ws)
        assert np.array_equal(tk, o_topk.topk(sc.astype(np.float64), ctx, K)), (seed, B)
        # the halves on the same (reused) workspace
        s2 = torch.empty((B, 1, Ts), device="cuda")
        t2 = torch.full((B, 1, K), -7, dtype=torch.int32, device="cuda")
        _lib.indexer_topk_scores(batch, *args, s2, K, ws)
        _lib.indexer_topk_select(batch, "bf16", K, s2, t2, ws)
        torch.cuda.synchronize()
        for b in range(B):
            n = int(ctx[b])
            assert np.array_equal(s2.cpu().numpy()[b, 0, :n].view(np.uint32),
                                  sc[b, 0, :n].view(np.uint32)), b
        assert np.array_equal(t2.cpu().numpy(), tk)
    # a dirtied workspace: hs_topk clears what it needs and leaves it zero again
    ws.fill_(0xA5)
    ctx, batch, args, dev = inputs(44, 24)
    s = torch.empty((24, 1, Ts), device="cuda")
    t = torch.empty((24, 1, K), dtype=torch.int32, device="cuda")
    _lib.indexer_scores(batch, *args, s)
    _lib.topk(batch, K, s, t, ws)
    torch.cuda.synchronize()
    sc = s.cpu().numpy()
    assert np.array_equal(t.cpu().numpy(), o_topk.topk(sc.astype(np.float64), ctx, K))
    sc2, tk2 = fused(batch, args, 24, ws)
    assert np.array_equal(tk2, o_topk.topk(sc2.astype(np.float64), ctx, K))


def _planted_scores(case, rng, B, P, T_stride):
    shape = (B, P, T_stride)
    if case == "quarter_steps":          # few distinct values: heavy ties at the threshold
        return (np.round(rng.standard_normal(shape) * 4) / 4).astype(np.float32)
    if case == "signed_zeros":           # most scores are +0 or -0, which are equal
        s = np.where(rng.random(shape) < 0.5, np.float32(0.0), np.float32(-0.0))
        pos = rng.random(shape) < 0.01
        s[pos] = rng.random(int(pos.sum())).astype(np.float32)
        neg = rng.random(shape) < 0.2
        s[neg] = -rng.random(int(neg.sum())).astype(np.float32)
        return s.astype(np.float32)
    if case == "all_equal":              # every visible token ties
        return np.ones(shape, dtype=np.float32)
    if case == "distinct":
        return rng.standard_normal(shape).astype(np.float32)
    raise ValueError(case)


@pytest.mark.parametrize("case", ["quarter_steps", "signed_zeros", "all_equal", "distinct"])
@pytest.mark.parametrize("T_stride", [65536, (1 << 18) + 64])
def test_topk_planted_ties_against_oracle(case, T_stride):
    """hs_topk alone on planted score rows, bit-exact against the oracle's
    (score desc, token asc) selection, for rows of 64K and 2^18 + 64 tokens
    (four 64K-token bitmap segments); the all-equal and signed-zero cases have
    more candidates than the finalize pass stages in LDS."""
    _say(f"topk planted {case} T_stride={T_stride}")
    from decode_indexer_logits_amd import _lib
    from oracle import topk as o_topk
    seed = ["quarter_steps", "signed_zeros", "all_equal", "distinct"].index(case)
    rng = np.random.default_rng(100 + 2 * seed + (T_stride > 65536))
    B, P, K = 3, 2, 2048
    ctx = np.array([T_stride, T_stride // 2 + 37, 2500], dtype=np.int32)
    S = _planted_scores(case, rng, B, P, T_stride)
    d_ctx = torch.from_numpy(ctx).cuda()
    d_s = torch.from_numpy(S).cuda()
    out = torch.empty((B, P, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(_lib.workspace_bytes(_lib.HS_OP_TOPK, B, P, T_stride, K), dtype=torch.uint8,
                     device="cuda")
    batch = _lib.make_batch(B, P, T_stride, d_ctx)
    _lib.topk(batch, K, d_s, out, ws)
    got = out.cpu().numpy()
    ref = o_topk.topk(S.astype(np.float64), ctx, K)
    bad = np.argwhere(np.any(ref != got, axis=2))
    assert len(bad) == 0, f"rows {bad[:4].tolist()}"


@pytest.mark.parametrize("case", ["quarter_steps", "signed_zeros", "all_equal", "distinct"])
@pytest.mark.parametrize("T_stride", [65536, 1 << 18])
def test_topk_many_rows_planted_ties_against_oracle(case, T_stride):
    """hs_topk on 32 rows of 64K and 2^18 tokens, planted ties included,
    bit-exact against the oracle (the all-equal and signed-zero rows hold more
    threshold-bin keys than the finalize pass stages in LDS); contexts short of
    K, at K + 1, mid-row and full; a workspace zero on entry comes back zero."""
    _say(f"topk 32 rows, {case} T_stride={T_stride}")
    from decode_indexer_logits_amd import _lib
    from oracle import topk as o_topk
    seed = ["quarter_steps", "signed_zeros", "all_equal", "distinct"].index(case)
    rng = np.random.default_rng(300 + 2 * seed + (T_stride > 65536))
    B, P, K = 16, 2, 2048
    ctx = rng.integers(K + 2, T_stride + 1, size=B).astype(np.int32)
    ctx[:4] = [T_stride, K - 5, K + 2, 2500]        # full, short of K, K + 1 visible at p=1
    S = _planted_scores(case, rng, B, P, T_stride)
    d_ctx = torch.from_numpy(ctx).cuda()
    d_s = torch.from_numpy(S).cuda()
    out = torch.empty((B, P, K), dtype=torch.int32, device="cuda")
    ws = torch.zeros(_lib.workspace_bytes(_lib.HS_OP_TOPK, B, P, T_stride, K), dtype=torch.uint8,
                     device="cuda")
    batch = _lib.make_batch(B, P, T_stride, d_ctx)
    _lib.topk(batch, K, d_s, out, ws)
    got = out.cpu().numpy()
    ref = o_topk.topk(S.astype(np.float64), ctx, K)
    bad = np.argwhere(np.any(ref != got, axis=2))
    assert len(bad) == 0, f"rows {bad[:4].tolist()}"
    # a workspace zero on entry comes back zero (the next call needs no clearing)
    assert int(ws.count_nonzero().item()) == 0


@pytest.mark.parametrize("q_t", ["bf16", "e4m3"])
@pytest.mark.parametrize("B", [256, 64, 12])
def test_indexer_many_requests_long_tiles(B, q_t):
    """Requests over a 16K-token stride, as many as select each tile size of the
    one-position indexer: 256 requests take 128-page tiles, 64 take 64-page
    tiles, 12 take 8-page tiles (and 1024-token top-K filter chunks).  Ragged
    contexts (empty, one token, on and off the 512/4096/8192 boundaries); fused
    and separate indexer calls give the same scores bit for bit; every visible
    score against the oracle; top-K exact on the GPU scores and within the
    near-tie rule on the oracle's.  Both query types: bf16, and E4M3 codes
    quantized on the GPU (the one-position E4M3 kernel takes the same tiles)."""
    from decode_indexer_logits_amd import _lib
    from oracle import indexer as o_idx, quant as o_quant, topk as o_topk
    rng = np.random.default_rng(21 + B)
    Ts, K = 16384, 512
    ctx = rng.integers(1, 12001, B).astype(np.int32)
    ctx[:8] = [0, 1, 64, 4096, 8191, 8192, 8193, 16384]
    if B > 11:
        ctx[8:12] = [511, 512, 513, 4097]
    _say(f"indexer many requests B={B} T_stride={Ts} q={q_t}")
    x = gen.indexer_inputs(2100, ctx, Ts)
    dev = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).cuda()
           for k, v in x.items() if isinstance(v, np.ndarray)}
    batch = _lib.make_batch(B, 1, Ts, dev["ctx_len"])
    s1 = torch.empty((B, 1, Ts), dtype=torch.float32, device="cuda")
    s2 = torch.empty_like(s1)
    topk = torch.empty((B, 1, K), dtype=torch.int32, device="cuda")
    ws = torch.zeros(_lib.workspace_bytes(_lib.HS_OP_TOPK, B, 1, Ts, K), dtype=torch.uint8,
                     device="cuda")
    q_dev, w_dev, q_ref, w_ref = dev["q_idx"], dev["w"], x["q_idx"], x["w"]
    if q_t == "e4m3":
        H, D = x["H"], x["D"]
        q_dev = torch.empty((B, 1, H, D), dtype=torch.uint8, device="cuda")
        w_dev = torch.empty((B, 1, H), dtype=torch.float32, device="cuda")
        _lib.quantize_queries(batch, H, D, dev["q_idx"], dev["w"], q_dev, w_dev)
        q_ref, w_ref, _ = o_quant.quantize_queries(x["q_idx"], x["w"])
    args = (x["H"], x["D"], q_t, q_dev, w_dev, "e4m3", dev["idx_pool"],
            dev["idx_scale"], dev["idx_bt"], dev["bias"])
    _lib.indexer_scores(batch, *args, s1)
    _lib.indexer_topk(batch, *args, s2, K, topk, ws)
    torch.cuda.synchronize()
    g1, g2, gt = s1.cpu().numpy(), s2.cpu().numpy(), topk.cpu().numpy()
    S = o_idx.indexer_scores(q_ref, q_t, w_ref, x["idx_pool"], "e4m3", x["idx_scale"],
                             x["idx_bt"], ctx, x["bias"], T_stride=Ts)
    worst, swaps = 0.0, 0
    for b in range(B):
        n = int(ctx[b])
        assert np.array_equal(g1[b, 0, :n].view(np.uint32), g2[b, 0, :n].view(np.uint32)), b
        if n == 0:
            continue
        ref = S[b, 0, :n]
        err = float(np.max(np.abs(g2[b, 0, :n] - ref)) / max(np.max(np.abs(ref)), 1e-30))
        worst = max(worst, err)
        assert err <= gc.SCORE_RTOL, (b, err)
        G = gt[b, 0][gt[b, 0] >= 0]
        O = o_topk.topk_row(S[b, 0], n, K)
        O = O[O >= 0]
        assert len(G) == len(O) == min(n, K)
        diff = np.setxor1d(G, O)
        if len(diff):
            sk = o_topk.kth_score(S[b, 0], n, K)
            assert np.all(np.abs(S[b, 0, diff] - sk) <= gc.TOPK_TIE_REL * abs(sk)), b
            swaps += len(diff)
    ref_t = o_topk.topk(g2.astype(np.float64), ctx, K)
    bad = np.argwhere(np.any(ref_t != gt, axis=2))
    assert len(bad) == 0, f"top-K rows {bad[:4].tolist()}"
    _say(f"worst score error {worst:.2e}, near-tie swaps {swaps}")


@pytest.mark.parametrize("q_t", ["bf16", "e4m3"])
@pytest.mark.parametrize("B,Ts", [(256, 32768), (64, 16384)])
def test_multi_position_indexer_long_tiles_against_oracle(q_t, B, Ts):
    """Four positions on many requests: the multi-position kernels (bf16 and
    E4M3 queries) size their tiles to one round of resident workgroups.  256
    requests of up to 32768 tokens take 128-page tiles, so pages 64..127 of a
    tile take the second block-id register and the scales of every page come
    from LDS; 64 requests of up to 16384 tokens take tiles of 16 to 22 pages.
    Ragged contexts (a page or less, on and off the tile boundaries).  Fused
    and separate indexer calls give the same scores bit for bit; every visible
    score of eight requests against the oracle; the top-K of every row exact
    on the GPU scores."""
    from decode_indexer_logits_amd import _lib
    from oracle import indexer as o_idx, quant as o_quant, topk as o_topk
    rng = np.random.default_rng(31 + B)
    P, K = 4, 512
    ctx = rng.integers(Ts // 2, Ts + 1, B).astype(np.int32)
    ctx[:8] = [Ts, 4, 64, 65, Ts // 4, Ts // 4 + 3, Ts // 2 + 1024, Ts - 8191]
    _say(f"multi-position indexer long tiles: B={B} P={P} T_stride={Ts} q={q_t}")
    x = gen.indexer_inputs(2200, ctx, Ts, P=P)
    dev = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).cuda()
           for k, v in x.items() if isinstance(v, np.ndarray)}
    batch = _lib.make_batch(B, P, Ts, dev["ctx_len"])
    H, D = x["H"], x["D"]
    q_ref, w_ref = x["q_idx"], x["w"]
    if q_t == "e4m3":
        q8 = torch.empty((B, P, H, D), dtype=torch.uint8, device="cuda")
        w8 = torch.empty((B, P, H), dtype=torch.float32, device="cuda")
        _lib.quantize_queries(batch, H, D, dev["q_idx"], dev["w"], q8, w8)
        q_dev, w_dev = q8, w8
        q_ref, w_ref, _ = o_quant.quantize_queries(x["q_idx"], x["w"])
        torch.cuda.synchronize()
        gc.check_quantized(x["q_idx"], x["w"], q8.cpu().numpy(), w8.cpu().numpy())
    else:
        q_dev, w_dev = dev["q_idx"], dev["w"]
    s1 = torch.empty((B, P, Ts), dtype=torch.float32, device="cuda")
    s2 = torch.empty_like(s1)
    topk = torch.empty((B, P, K), dtype=torch.int32, device="cuda")
    ws = torch.zeros(_lib.workspace_bytes(_lib.HS_OP_TOPK, B, P, Ts, K), dtype=torch.uint8,
                     device="cuda")
    args = (H, D, q_t, q_dev, w_dev, "e4m3", dev["idx_pool"], dev["idx_scale"], dev["idx_bt"],
            dev["bias"])
    _lib.indexer_scores(batch, *args, s1)
    _lib.indexer_topk(batch, *args, s2, K, topk, ws)
    torch.cuda.synchronize()
    g1, g2, gt = s1.cpu().numpy(), s2.cpu().numpy(), topk.cpu().numpy()
    for b in range(B):
        for p in range(P):
            n = max(int(ctx[b]) - P + p + 1, 0)
            assert np.array_equal(g1[b, p, :n].view(np.uint32), g2[b, p, :n].view(np.uint32)), (b, p)
    rows = [0, 1, 2, 3, 5, 7, B // 2, B - 1]
    S = o_idx.indexer_scores(q_ref[rows], q_t, w_ref[rows], x["idx_pool"], "e4m3",
                             x["idx_scale"], x["idx_bt"][rows], ctx[rows], x["bias"][rows],
                             T_stride=Ts)
    worst = 0.0
    for i, b in enumerate(rows):
        for p in range(P):
            n = max(int(ctx[b]) - P + p + 1, 0)
            if n == 0:
                continue
            ref = S[i, p, :n]
            err = float(np.max(np.abs(g2[b, p, :n] - ref)) / max(np.max(np.abs(ref)), 1e-30))
            worst = max(worst, err)
            assert err <= gc.SCORE_RTOL, (b, p, err)
    ref_t = o_topk.topk(g2.astype(np.float64), ctx, K)
    bad = np.argwhere(np.any(ref_t != gt, axis=2))
    assert len(bad) == 0, f"top-K rows {bad[:4].tolist()}"
    _say(f"worst score error {worst:.2e}")


def _select_resolve_workload(name):
    if name == "mixed_small":
        beta, hot, _ = calibrate(seed=1003, B=4, T=16384, K=512, tail=1024)
        return gen.mixed_128k(seed=1003, B=4, T=16384, K=512, tail=1024, beta=beta,
                              hot_tokens=hot)
    if name == "one_position_c8192":
        return gen.mtp3_agentic(B=3, K=1024, steps=2, first_turn=40000, per_turn=300, turns=5,
                                out_max=50, P=1, C=8192)
    if name == "resident_k4096":
        return gen.resident_fp8(B=4, K=4096)
    if name == "two_positions":
        return gen.mtp3_agentic(B=3, K=128, steps=2, first_turn=9000, per_turn=300, turns=5,
                                out_max=50, P=2)
    if name == "tiny_fp32":
        return gen.tiny_fp32(K=256)
    raise KeyError(name)


@pytest.mark.parametrize("name", ["mixed_small", "one_position_c8192", "resident_k4096",
                                  "two_positions", "tiny_fp32"])
def test_select_resolve_matches_separate_calls(name):
    """hs_indexer_topk_select_resolve gives what hs_indexer_topk_select followed
    by hs_resolve_tables give, bit for bit: the top-K, row ids, fault lists,
    counts, hot tables, device error word, and the selection workspace back to
    zero.  One query position takes the fused kernel (all three of its
    instances: up to 4096 hot rows with K <= 2048, up to 16384 hot rows, and
    K > 2048); several positions and fp32 queries take the two launches.  Every
    step of the workload, each from the state the previous one left."""
    from decode_indexer_logits_amd.device import DeviceStep
    wl = _select_resolve_workload(name)
    _say(f"select + resolve {name}: B={wl.B} P={wl.P} K={wl.K} C={wl.C} q={wl.q_dtype}")
    ds = DeviceStep(wl)

    def outputs():
        torch.cuda.synchronize()
        o = {"topk": ds.topk.clone(), "row_ids": ds.row_ids.clone(), "counts": ds.counts.clone(),
             "err": ds.err.clone(), "ws_zero": bool((ds.ws_topk == 0).all())}
        c = ds.counts.cpu().numpy()
        f = ds.faults.cpu().numpy()
        o["faults"] = [f[b, :int(c[b, 2])].copy() for b in range(wl.B)]
        for k in ("tok2slot", "slot2tok", "stamp"):
            t = getattr(ds, k, None)
            o[k] = None if t is None else t.clone()
        return o

    for s in range(1, wl.steps + 1):
        if s > 1:
            ds.set_queries(s)
        snap = ds.snapshot()
        ds.run_indexer_topk_scores()
        ds.run_indexer_topk_select()
        ds.run_resolve_tables()
        a = outputs()
        ds.restore(snap)
        ds.run_indexer_topk_scores()
        ds.run_indexer_topk_select_resolve()
        b = outputs()
        assert a["ws_zero"] and b["ws_zero"]
        for k in ("topk", "row_ids", "counts", "err", "tok2slot", "slot2tok", "stamp"):
            if a[k] is None:
                assert b[k] is None
            else:
                assert torch.equal(a[k], b[k]), (s, k)
        for x, y in zip(a["faults"], b["faults"]):
            assert np.array_equal(x, y), s
        ds.run_copy_faults()
        torch.cuda.synchronize()
        _say(f"step {s}: counts {b['counts'].sum(dim=0).tolist()}")


def test_resolve_merge_path_long_stride():
    """Several positions on a token stride past 262144 take the resolve kernel's
    list merge (binary searches and a dedup scan) instead of its token bitmap;
    two steps with two positions, checked stage by stage against the oracle."""
    from decode_indexer_logits_amd.device import DeviceStep
    wl = gen.mtp3_agentic(B=2, K=64, steps=2, first_turn=262200, per_turn=100, turns=2,
                          out_max=20, P=2)
    assert wl.T_stride > 262144 and wl.P == 2
    _say(f"resolve merge path: T_stride={wl.T_stride}, P=2")
    ds = DeviceStep(wl)
    ost = gc.oracle_state(wl)
    for s in range(1, wl.steps + 1):
        ds.set_queries(s)
        ds.run()
        ost, rr, info = gc.full_check(ds, wl, ost, s=s, attn_tol=2e-2)
        _say(s, info["counts"].tolist())


@pytest.mark.parametrize("kv", ["e4m3", "f32"])
def test_attention_layers_call_matches_per_layer_calls(kv):
    """hs_sparse_mla_decode_layers over L layers against the oracle's attention
    over the same rows, and against L calls of hs_sparse_mla_decode: identical
    for L = 1, equal to fp32 summation order for L = 3 (fewer slices per
    layer); both paths (bf16 x E4M3 and fp32)."""
    from decode_indexer_logits_amd import _lib
    rng = np.random.default_rng(71)
    B, P, K, Hq, L, n_rows = 3, 1, 1000, 16, 3, 4096
    ctx = torch.tensor([K, K, K], dtype=torch.int32, device="cuda")
    batch = _lib.make_batch(B, P, 1024, ctx)
    rid = np.stack([rng.choice(n_rows, K, replace=False) for _ in range(B)]).astype(np.int32)
    rid[1, 700:] = -1                                   # a short selection
    row_ids = torch.from_numpy(rid.reshape(B, P, K)).cuda()
    if kv == "e4m3":
        q = torch.from_numpy(gen.bf16_bits(rng.standard_normal((L, B, P, Hq, 576))).view(np.int16)).cuda()
        pool = torch.randint(0, 256, (L, n_rows, 576), dtype=torch.uint8, device="cuda")
        pool[(pool & 0x7F) == 0x7F] = 0                 # no NaN codes
        rs = torch.rand((L, n_rows), device="cuda") * 0.02
        qt = "bf16"
    else:
        q = torch.randn((L, B, P, Hq, 576), device="cuda")
        pool = torch.randn((L, n_rows, 576), device="cuda")
        rs = None
        qt = "f32"
    ws = torch.empty(max(_lib.mla_layers_workspace_bytes(B, P, K, Hq, L),
                         _lib.workspace_bytes(_lib.HS_OP_MLA, B, P, 1024, K, Hq), 16),
                     dtype=torch.uint8, device="cuda")
    out1 = torch.empty((L, B, P, Hq, 512), device="cuda")
    lse1 = torch.empty((L, B, P, Hq), device="cuda")
    for l in range(L):
        _lib.sparse_mla_decode(batch, K, Hq, qt, q[l], kv, pool[l], None if rs is None else rs[l],
                               row_ids, 1.0 / 24.0, out1[l], lse1[l], ws)
    outL = torch.empty_like(out1)
    lseL = torch.empty_like(lse1)
    _lib.sparse_mla_decode_layers(batch, K, Hq, L, qt, q, kv, pool, n_rows, rs, row_ids, 1.0 / 24.0,
                                  outL, lseL, ws)
    one = torch.empty_like(out1[0])
    one_lse = torch.empty_like(lse1[0])
    _lib.sparse_mla_decode_layers(batch, K, Hq, 1, qt, q[0], kv, pool[0], n_rows,
                                  None if rs is None else rs[0], row_ids, 1.0 / 24.0, one, one_lse,
                                  ws)
    torch.cuda.synchronize()
    assert torch.equal(one, out1[0]) and torch.equal(one_lse, lse1[0])
    err = ((outL - out1).abs().amax(dim=-1) / out1.abs().amax(dim=-1).clamp_min(1e-30)).max().item()
    assert err <= 1e-5, err
    assert torch.allclose(lseL, lse1, rtol=1e-6, atol=1e-6)
    # the oracle over the same rows, from the same codes and scales
    from oracle import attention as o_attn, numerics as o_num
    tol = 2e-2 if kv == "e4m3" else 1e-5
    qn = q.cpu().numpy()
    qn = qn.view(np.uint16) if kv == "e4m3" else qn
    pn, rsn = pool.cpu().numpy(), None if rs is None else rs.cpu().numpy()
    oL, lL = outL.cpu().numpy(), lseL.cpu().numpy()
    for l in range(L):
        for b in range(B):
            sel = rid[b][rid[b] >= 0]
            x = o_num.to_f64(pn[l][sel], kv)
            if rsn is not None:
                x = x * rsn[l][sel].astype(np.float64)[:, None]
            ro, rl = o_attn.attend(o_num.to_f64(qn[l, b, 0], qt), x, 1.0 / 24.0)
            assert o_attn.max_rel_err(oL[l, b, 0], ro) <= tol, (kv, l, b)
            assert np.all(np.abs(lL[l, b, 0] - rl) <= gc.lse_bound(tol, rl)), (kv, l, b)
