"""Pins of the oracle's composed decode step (CPU only).

``oracle.step.decode_step`` chains the four stages.  What fixes it, apart from
the stage pins: with K at least the context, the sparse step must give dense
softmax attention over every visible token (a result that does not depend on
the selection at all); with K below it, the selection must be the brute-force
stable sort of the scores it returned and the attention the library's softmax
attention over those rows; a caller's scores or selection must be the ones
used; and where rows live (resident, hot or host-only) may change the state
and the counts but never the numbers.
"""
import numpy as np
import torch

from oracle import attention, resolve, step
from workloads import gen


def _state(wl):
    return resolve.ResidencyState(wl.bt, wl.hot_blocks, wl.tok2slot, wl.slot2tok, wl.stamp,
                                  wl.host_bt, wl.step)


def _sdpa(q_h, x, sm_scale):
    """torch's scaled-dot-product attention in float64, MQA by broadcast."""
    qq = torch.from_numpy(q_h)[None, :, None]                       # [1, Hq, 1, 576]
    kk = torch.from_numpy(x)[None, None].expand(1, q_h.shape[0], x.shape[0], 576)
    vv = torch.from_numpy(x[:, :512])[None, None].expand(1, q_h.shape[0], x.shape[0], 512)
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=sm_scale)[0, :, 0].numpy()


def test_k_at_least_context_is_dense_attention():
    wl = gen.tiny_fp32(K=1024, T=500)
    q_idx, q = wl.step_inputs(1)
    r = step.decode_step(wl, _state(wl), q_idx, q)
    T = int(wl.ctx_len[0])
    assert r["topk"][0, 0, :T].tolist() == list(range(T))
    assert np.all(r["topk"][0, 0, T:] == -1)
    do, dl = attention.dense_mla(q[0], wl.q_dtype, wl.lat[0], wl.lat_scale, wl.kv_dtype,
                                 wl.ctx_len, wl.sm_scale)
    so, sl = r["attn"][0]
    assert np.max(np.abs(so - do)) < 1e-12 and np.max(np.abs(sl - dl)) < 1e-12
    # every page resident: each selected token is read in place
    assert r["resolve"].counts.tolist() == [[T, 0, 0, 0]]
    rows = r["resolve"].row_ids[0, 0, :T]
    assert np.array_equal(rows, wl.bt[0, np.arange(T) // 64].astype(np.int64) * 64 + np.arange(T) % 64)
    assert r["state"].step == wl.step + 1


def test_selection_is_brute_force_sort_and_attention_is_library_sdpa():
    wl = gen.tiny_fp32(K=64, T=700)
    q_idx, q = wl.step_inputs(1)
    r = step.decode_step(wl, _state(wl), q_idx, q)
    S = r["scores"][0, 0, :700]
    want = np.sort(np.argsort(-S, kind="stable")[:64])
    assert r["topk"][0, 0].tolist() == want.tolist()
    x = attention.logical_rows(wl.lat[0, 0], None, wl.kv_dtype, want)
    ref = _sdpa(q[0, 0, 0].astype(np.float64), x, wl.sm_scale)
    assert np.max(np.abs(r["attn"][0][0][0, 0] - ref)) < 1e-12


def test_stage_inputs_given_by_the_caller_are_used():
    wl = gen.tiny_fp32(K=32, T=300)
    q_idx, q = wl.step_inputs(1)
    planted = np.zeros((1, 1, wl.T_stride))
    planted[0, 0, :300] = -np.arange(300, dtype=np.float64)      # the best are the first tokens
    r = step.decode_step(wl, _state(wl), q_idx, q, scores=planted)
    assert r["topk"][0, 0].tolist() == list(range(32))
    sel = np.full((1, 1, 32), -1, np.int32)
    sel[0, 0, :3] = [7, 99, 250]
    r = step.decode_step(wl, _state(wl), q_idx, q, selection=sel)
    assert r["topk"] is sel
    assert r["resolve"].counts.tolist() == [[3, 0, 0, 0]]
    x = attention.logical_rows(wl.lat[0, 0], None, wl.kv_dtype, [7, 99, 250])
    ref = _sdpa(q[0, 0, 0].astype(np.float64), x, wl.sm_scale)
    assert np.max(np.abs(r["attn"][0][0][0, 0] - ref)) < 1e-12


def test_residency_changes_state_not_numbers():
    """Two-layer host-only start: the first step faults every selected token
    into both layers' hot slots; the attention equals the same step run on an
    all-resident copy of the state, and the second step hits what the first
    faulted (same queries, same selection)."""
    wl = gen.norescache_1m(B=2, T=4096, K=128, L=2, steps=2)
    q_idx, q = wl.step_inputs(1)
    st0 = _state(wl)
    r1 = step.decode_step(wl, st0, q_idx, q)
    U = [np.unique(r1["topk"][b][r1["topk"][b] >= 0]) for b in range(2)]
    assert r1["resolve"].counts.tolist() == [[0, 0, len(U[b]), 0] for b in range(2)]
    assert r1["resolve"].err == 0
    # all resident: any block table with every page present
    full = _state(wl)
    full.bt = np.arange(full.bt.size, dtype=np.int32).reshape(full.bt.shape)
    rf = step.decode_step(wl, full, q_idx, q)
    assert np.array_equal(rf["topk"], r1["topk"])
    assert rf["resolve"].counts.tolist() == [[len(U[b]), 0, 0, 0] for b in range(2)]
    for l in range(2):
        assert np.array_equal(rf["attn"][l][0], r1["attn"][l][0])
        assert np.array_equal(rf["attn"][l][1], r1["attn"][l][1])
    # the next step over the same selection is all hits, still the same numbers
    r2 = step.decode_step(wl, r1["state"], q_idx, q, selection=r1["topk"])
    assert r2["resolve"].counts.tolist() == [[0, len(U[b]), 0, 0] for b in range(2)]
    for l in range(2):
        assert np.array_equal(r2["attn"][l][0], r1["attn"][l][0])
