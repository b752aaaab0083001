"""The allocation-free indexer + top-K entry point against hs_indexer_topk.

hs_indexer_topk_noalloc runs the same kernels on a static device scratch
array instead of a caller workspace.  Its scores must equal hs_indexer_topk's
bit for bit and its top-K must be identical (and equal the oracle's top-K of
those scores), on calls in a row whose sizes shrink, so that whatever the
previous call left in the shared scratch cannot leak into the next one.
"""
import sys

import numpy as np
import pytest

from workloads import gen

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


def _inputs(seed, ctx, Ts, fp32=False):
    if fp32:
        wl = gen.tiny_fp32(K=256, T=int(ctx[0]))
        x = {"ctx_len": wl.ctx_len, "H": wl.H_idx, "D": wl.D_idx, "q_idx": wl.q_idx, "w": wl.w,
             "idx_pool": wl.idx_pool, "idx_scale": None, "idx_bt": wl.idx_bt, "bias": None,
             "T_stride": wl.T_stride}
        return x, "f32", "f32"
    return gen.indexer_inputs(seed, ctx, Ts), "bf16", "e4m3"


def _both(x, qt, kt, K):
    """(scores, topk) of hs_indexer_topk and of hs_indexer_topk_noalloc."""
    from decode_indexer_logits_amd import _lib
    dev = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).cuda()
           for k, v in x.items() if isinstance(v, np.ndarray)}
    B, Ts = len(x["ctx_len"]), x["T_stride"]
    batch = _lib.make_batch(B, 1, Ts, dev["ctx_len"])
    args = (x["H"], x["D"], qt, dev["q_idx"], dev["w"], kt, dev["idx_pool"], dev.get("idx_scale"),
            dev["idx_bt"], dev.get("bias"))
    s_ref = torch.full((B, 1, Ts), float("nan"), device="cuda")
    t_ref = torch.full((B, 1, K), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(_lib.workspace_bytes(_lib.HS_OP_TOPK, B, 1, Ts, K), dtype=torch.uint8,
                     device="cuda")
    _lib.indexer_topk(batch, *args, s_ref, K, t_ref, ws)
    s = torch.full_like(s_ref, float("nan"))
    t = torch.full_like(t_ref, -7)
    _lib.indexer_topk_noalloc(batch, *args, s, K, t)
    torch.cuda.synchronize()
    return s_ref.cpu().numpy(), t_ref.cpu().numpy(), s.cpu().numpy(), t.cpu().numpy()


def _check(x, qt, kt, K, what):
    from oracle import topk as o_topk
    s_ref, t_ref, s, t = _both(x, qt, kt, K)
    ctx = x["ctx_len"]
    for b in range(len(ctx)):
        n = int(ctx[b])
        assert np.array_equal(s[b, 0, :n].view(np.uint32), s_ref[b, 0, :n].view(np.uint32)), (what, b)
    assert np.array_equal(t, t_ref), what
    ref = o_topk.topk(s.astype(np.float64), ctx, K)
    assert np.array_equal(t, ref), what
    _say(what, "ok")


def test_noalloc_matches_workspace_call_on_shrinking_sizes():
    rng = np.random.default_rng(5)
    # 1: 32 requests of up to 64K tokens (8192-token indexer tiles), K = 2048
    ctx1 = rng.integers(40000, 65537, 32).astype(np.int32)
    ctx1[:3] = [65536, 1, 0]
    x1, qt, kt = _inputs(3100, ctx1, 65536)
    _say("noalloc call 1: B=32, T_stride=65536, K=2048")
    _check(x1, qt, kt, 2048, "call 1")
    # 2: a smaller batch right after, on the same scratch: B=5, T_stride=8192, K=256
    ctx2 = np.array([8192, 300, 64, 5000, 2], dtype=np.int32)
    x2, qt, kt = _inputs(3101, ctx2, 8192)
    _say("noalloc call 2: B=5, T_stride=8192, K=256")
    _check(x2, qt, kt, 256, "call 2")
    # 3: the fp32 path (separate histogram pass), smaller again
    x3, qt, kt = _inputs(0, np.array([3000], np.int32), 3008, fp32=True)
    _say("noalloc call 3: fp32, B=1, T=3000, K=256")
    _check(x3, qt, kt, 256, "call 3")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    from decode_indexer_logits_amd import _lib
    d_ctx = torch.zeros(64, dtype=torch.int32, device="cuda")
    batch = _lib.make_batch(64, 1, 1 << 20, d_ctx)
    one = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.HsError) as e:
        _lib.indexer_topk_noalloc(batch, 64, 128, "bf16", one, one, "e4m3", one, one,
                                  one.view(torch.int32), None, one, 2048, one.view(torch.int32))
    assert e.value.status == 5 and "static scratch" in str(e.value)
