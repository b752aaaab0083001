"""GPU parity of the token-sharded top-K, through the C ABI.

hs_topk_sharded against the oracle's sharded selection (which the CPU tests
pin equal to the global one) and against hs_topk on the same scores, bit for
bit: tie-heavy and distinct rows, ragged contexts (empty, shorter than K, on
and off shard boundaries), shard counts from 1 to 64, K from 1 to 8192, and
four rows of 2^20 tokens.
"""
import sys

import numpy as np
import pytest

from oracle import topk as o_topk

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


def _run(S_rows, ctx, K, S):
    from decode_indexer_logits_amd import _lib
    B, Ts = S_rows.shape
    d_ctx = torch.from_numpy(ctx.astype(np.int32)).cuda()
    d_s = torch.from_numpy(S_rows.reshape(B, 1, Ts)).cuda()
    batch = _lib.make_batch(B, 1, Ts, d_ctx)
    out_s = torch.empty((B, 1, K), dtype=torch.int32, device="cuda")
    out_g = torch.empty_like(out_s)
    # the call must not depend on what the workspace holds on entry
    ws_s = torch.full((_lib.topk_sharded_workspace_bytes(B, Ts, K, S),), 0xA5, dtype=torch.uint8,
                      device="cuda")
    ws_g = torch.empty(_lib.workspace_bytes(_lib.HS_OP_TOPK, B, 1, Ts, K), dtype=torch.uint8,
                       device="cuda")
    _lib.topk_sharded(batch, K, S, d_s, out_s, ws_s)
    _lib.topk(batch, K, d_s, out_g, ws_g)
    torch.cuda.synchronize()
    return out_s.cpu().numpy()[:, 0], out_g.cpu().numpy()[:, 0]


def _rows(case, rng, B, Ts):
    if case == "quarter_steps":
        return (np.round(rng.standard_normal((B, Ts)) * 4) / 4).astype(np.float32)
    if case == "signed_zeros":
        s = np.where(rng.random((B, Ts)) < 0.5, np.float32(0.0), np.float32(-0.0))
        pos = rng.random((B, Ts)) < 0.02
        s[pos] = rng.random(int(pos.sum())).astype(np.float32)
        return s.astype(np.float32)
    return rng.standard_normal((B, Ts)).astype(np.float32)


@pytest.mark.parametrize("case", ["quarter_steps", "signed_zeros", "distinct"])
@pytest.mark.parametrize("S,K", [(1, 256), (2, 2048), (8, 2048), (8, 1), (16, 8192), (64, 300)])
def test_sharded_topk_equals_oracle_and_unsharded(case, S, K):
    rng = np.random.default_rng(31 * S + K + ["quarter_steps", "signed_zeros",
                                                  "distinct"].index(case))
    Ts = 64 * S * max(1, 16384 // (64 * S))
    B = 6
    # empty, one token, just under K, one shard, one shard and a token, full
    ctx = np.clip(np.array([0, 1, K - 1, Ts // S, Ts // S + 1, Ts]), 0, Ts)
    rows = _rows(case, rng, B, Ts)
    got_s, got_g = _run(rows, ctx, K, S)
    assert np.array_equal(got_s, got_g)
    for b in range(B):
        want = o_topk.topk_sharded_row(rows[b].astype(np.float64), int(ctx[b]), K, Ts // S)
        assert np.array_equal(got_s[b], want), (b, int(ctx[b]))


def test_sharded_topk_million_token_rows():
    _say("sharded top-K, 4 rows of 2^20 tokens, S = 8")
    rng = np.random.default_rng(77)
    B, Ts, K = 4, 1 << 20, 2048
    rows = (np.round(rng.standard_normal((B, Ts)) * 64) / 64).astype(np.float32)
    ctx = np.array([Ts, Ts - 1, 3 * (Ts // 8) + 5, 700_000])
    got_s, got_g = _run(rows, ctx, K, 8)
    assert np.array_equal(got_s, got_g)
    want = o_topk.topk(rows[:, None, :].astype(np.float64), ctx, K)[:, 0]
    assert np.array_equal(got_s, want)
