"""GPU parity at the workloads' full sizes, through the C ABI.

Mixed residency at 128K (B=32, T=131072, K=2048) runs as one captured HIP
graph, the launch configuration the benchmark times; the MTP3 mix (B=64, P=4,
4 steps) and the 1M-token no-residency start (B=4, T=2^20, L=4, 16 steps) run
eagerly, step after step from their initial state.

What is checked at these sizes:
  scores     every visible token of every (request, position) against the
             oracle's indexer at 128K (the benchmarked graph), at the first
             MTP3 step and at the first and last 1M steps; at the other steps
             of the sequences a random sample of tokens per row, plus the
             first and last visible token, recomputed one by one;
  top-K      bit-exact against the oracle's top-K of the GPU scores for every
             row; against the oracle's own scores (near-tie swaps only) for
             every row wherever the scores are checked in full;
  resolve    every table, row id, fault list, count, step and error word
             bit-exact for every request; the bytes and scale of every
             faulted row in every layer;
  attention  every output vector against the oracle over the same selection.
"""
import gc as _gc
import sys

import numpy as np
import pytest

from workloads import gen
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
    yield
    _gc.collect()
    torch.cuda.empty_cache()


def _check_step(ds, wl, ost, s, rng, score_sample, oracle_topk_requests=(), attn_tol=2e-2):
    """score_sample None: every visible score, and every row's top-K against
    the oracle's own scores; else sampled scores, and the oracle-score top-K
    check for the listed requests only."""
    q_idx, q = wl.step_inputs(s)
    g = gc.gpu_outputs(ds)
    worst_s, S = gc.check_scores(wl, q_idx, g["scores"], sample=score_sample, rng=rng)
    gc.check_topk_exact(wl, g["scores"], g["topk"])
    if S is not None:
        swaps = gc.check_topk_vs_oracle_scores(wl, S, g["topk"])
        del S
    else:
        swaps = gc.check_topk_vs_oracle_scores_rows(wl, q_idx, g["topk"], oracle_topk_requests)
    new, rr = gc.check_resolve(wl, ost, g["topk"], g)
    if wl.C:
        pool = ds.pool.cpu().numpy()
        rsc = None if ds.row_scale is None else ds.row_scale.cpu().numpy()
        gc.check_copies(wl, rr, pool, rsc)
        del pool
    worst_a = gc.check_attention(wl, q, g["topk"], g["out"], g["lse"], attn_tol)
    return new, rr, {"score_err": worst_s, "attn_err": worst_a, "topk_swaps": swaps,
                     "counts_mean": g["counts"].mean(axis=0).round(1).tolist(),
                     "err": g["err"]}


@pytest.mark.timeout(600)
def test_mixed_128k_full_size_graph():
    """The full-size 128K step as a captured graph replay, against the oracle; then the
    same step launched on its stream (how bench.py times it) from the same state gives
    the same results bit for bit."""
    _say("mixed_128k full size (B=32, T=131072, K=2048), captured graph")
    from decode_indexer_logits_amd.device import DeviceStep
    wl = gen.mixed_128k()
    ds = DeviceStep(wl)
    snap = ds.snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ds.run()                          # warm every kernel before capture
    torch.cuda.synchronize()
    ds.restore(snap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ds.run()
    torch.cuda.synchronize()
    ds.restore(snap)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    replayed = {k: getattr(ds, k).clone() for k in ("topk", "row_ids", "faults", "counts")}
    replayed["out"] = ds.out[0].clone()
    replayed["lse"] = ds.lse[0].clone()
    _say("replayed; checking against the oracle")
    rng = np.random.default_rng(11)
    _, _, info = _check_step(ds, wl, gc.oracle_state(wl), 1, rng, score_sample=None)
    _say(info)
    c = ds.counts.cpu().numpy()
    assert info["err"] == 0
    assert np.all(c[:, 1] >= 900)                     # pre-seeded: about half of the top-K hits
    assert np.all(c[:, 2] > 0) and np.all(c[:, 3] == c[:, 2])
    assert np.all(c[:, 0] + c[:, 1] + c[:, 2] == wl.K)
    _say("the same step launched on the stream")
    ds.restore(snap)
    ds.run()
    torch.cuda.synchronize()
    launched = {k: getattr(ds, k) for k in ("topk", "row_ids", "faults", "counts")}
    launched["out"], launched["lse"] = ds.out[0], ds.lse[0]
    for k, v in replayed.items():
        assert torch.equal(v, launched[k]), f"{k} differs between the replay and the launches"
    del ds, g
    _gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_mtp3_agentic_full_size_four_steps():
    _say("mtp3_agentic full size (B=64, P=4, K=2048, C=10240), 4 steps")
    from decode_indexer_logits_amd.device import DeviceStep
    wl = gen.mtp3_agentic()
    ds = DeviceStep(wl)
    ost = gc.oracle_state(wl)
    rng = np.random.default_rng(12)
    for s in range(1, wl.steps + 1):
        ds.set_queries(s)
        ds.run()
        ost, rr, info = _check_step(ds, wl, ost, s, rng, score_sample=None if s == 1 else 512)
        _say(f"step {s}", info)
        assert info["err"] == 0
        if s == 1:
            assert info["counts_mean"][1] == 0.0        # hot buffers start empty
    del ds
    _gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("append", [False, True])
def test_norescache_1m_full_size_sixteen_steps(append):
    """Sixteen steps at full size; with append, every step but the last is
    followed by a KV append of one token per request (the context grows from
    2^20 to 2^20 + 15), checked against the oracle's append."""
    _say(f"norescache_1m full size (B=4, T=2^20, L=4, K=2048), 16 steps, append={append}")
    from decode_indexer_logits_amd.device import DeviceStep
    wl = gen.norescache_1m(append=append)
    _say("generated")
    ds = DeviceStep(wl)
    ost = gc.oracle_state(wl)
    cs = gc.cache_mirror(wl) if append else None
    rng = np.random.default_rng(13)
    rates = []
    for s in range(1, wl.steps + 1):
        ds.set_queries(s)
        ds.run()
        full = s in (1, wl.steps)
        ost, rr, info = _check_step(ds, wl, ost, s, rng, score_sample=None if full else 2048)
        c = rr.counts
        rate = float(c[:, 1].sum() / max(c[:, 1].sum() + c[:, 2].sum(), 1))
        rates.append(round(rate, 4))
        _say(f"step {s} hit rate {rate:.4f}", info)
        assert info["err"] == 0
        if s == 1:
            assert np.all(c[:, 1] == 0) and np.all(c[:, 2] == wl.K) and np.all(c[:, 3] == 0)
        if append and s < wl.steps:
            ost = gc.append_and_check(ds, wl, ost, cs, s)
    _say("hit rates", rates)
    assert rates[0] == 0.0 and min(rates[1:]) > 0.0
    del ds
    _gc.collect()
    torch.cuda.empty_cache()
