"""GPU parity of hs_topk on rows longer than 786432 tokens, through the C ABI.

Such rows take the finalize path that sorts the K selected tokens in LDS (a
bitonic network over the next power of two) instead of laying a bitmap over
the row.  The selection is compared with the oracle's full sort bit for bit:
K from 1 to 8192 including sizes that are not powers of two, tie-heavy and
distinct scores, selections packed into one narrow window, row lengths on both
sides of the switch, and one row of the longest supported context (2^24).
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


def _gpu_topk(rows, ctx, K):
    from decode_indexer_logits_amd import _lib
    B, Ts = rows.shape
    d_ctx = torch.from_numpy(ctx.astype(np.int32)).cuda()
    d_s = torch.from_numpy(rows.reshape(B, 1, Ts)).cuda()
    batch = _lib.make_batch(B, 1, Ts, d_ctx)
    out = torch.empty((B, 1, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(_lib.workspace_bytes(_lib.HS_OP_TOPK, B, 1, Ts, K), dtype=torch.uint8,
                     device="cuda")
    _lib.topk(batch, K, d_s, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()[:, 0]


def _rows(case, rng, B, Ts):
    if case == "quarter_steps":
        return (np.round(rng.standard_normal((B, Ts)) * 4) / 4).astype(np.float32)
    if case == "window":
        # every high score inside one 3000-token window of each row
        s = rng.standard_normal((B, Ts)).astype(np.float32)
        for b in range(B):
            w0 = int(rng.integers(0, Ts - 3000))
            s[b, w0:w0 + 3000] += 50.0
        return s
    return rng.standard_normal((B, Ts)).astype(np.float32)


@pytest.mark.parametrize("case", ["quarter_steps", "distinct", "window"])
@pytest.mark.parametrize("K", [1, 3, 2048, 5000, 8192])
def test_topk_long_rows_equal_oracle(case, K):
    _say(f"top-K long rows: {case}, K={K}")
    rng = np.random.default_rng(1000 + K + 7 * ["quarter_steps", "distinct", "window"].index(case))
    Ts = 1 << 20
    # the last bitmap length, the first sorted one, and longer rows
    ctx = np.array([786432, 786433, 800001, Ts - 3, Ts])
    rows = _rows(case, rng, len(ctx), Ts)
    got = _gpu_topk(rows, ctx, K)
    for b in range(len(ctx)):
        want = o_topk.topk_row(rows[b].astype(np.float64), int(ctx[b]), K)
        assert np.array_equal(got[b], want), (case, K, b, int(ctx[b]))


def test_topk_longest_context():
    _say("top-K: one row of 2^24 tokens, K=8192")
    rng = np.random.default_rng(2024)
    Ts = 1 << 24
    rows = (np.round(rng.standard_normal((1, Ts)) * 16) / 16).astype(np.float32)
    ctx = np.array([Ts])
    got = _gpu_topk(rows, ctx, 8192)
    want = o_topk.topk_row(rows[0].astype(np.float64), Ts, 8192)
    assert np.array_equal(got[0], want)
