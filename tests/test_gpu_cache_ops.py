"""GPU parity of KV append, pre-copy and demotion, through the C ABI.

A small batch (ragged contexts, two latent layers of E4M3 rows, E4M3 indexer
keys with block scales, a pinned host pool) goes through a seeded sequence of
the three operations, including calls that must fail as a whole.  After every
call the device state is compared bit for bit with the oracle's: context
lengths, both block tables, host table, both free lists, every pool byte and
scale, every host byte and scale, and the error bits of that call.
"""
import sys

import numpy as np
import pytest

from oracle import cache_ops as co

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


class _Dev:
    """Device copy of a CacheState, with the C ABI structs that point into it."""

    def __init__(self, st: co.CacheState, P: int, interleaved: bool = False):
        """interleaved: the host pool keeps the L rows of a token together
        ([tokens, L, 576], host_row_pitch = L) instead of one plane per layer."""
        from decode_indexer_logits_amd import _lib
        self.lib = _lib
        cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        B, MB = st.bt.shape
        self.T_stride = MB * 64
        self.ctx = cu(st.ctx_len)
        self.bt, self.idx_bt, self.host_bt = cu(st.bt), cu(st.idx_bt), cu(st.host_bt)
        self.pool, self.row_scale = cu(st.pool), cu(st.row_scale)
        self.idx_pool, self.idx_scale = cu(st.idx_pool), cu(st.idx_scale)
        self.inter = interleaved
        hr, hs = (st.host_rows.transpose(1, 0, 2), st.host_scale.T) if interleaved else \
            (st.host_rows, st.host_scale)
        self.host_rows = torch.from_numpy(np.ascontiguousarray(hr)).pin_memory()
        self.host_scale = cu(hs)
        cap = st.free_capacity
        self.free = torch.zeros(cap, dtype=torch.int32, device="cuda")
        self.free[:len(st.free)] = torch.tensor(st.free, dtype=torch.int32)
        self.free_n = torch.tensor([len(st.free)], dtype=torch.int32, device="cuda")
        self.ifree = torch.zeros(len(st.idx_free) + 8, dtype=torch.int32, device="cuda")
        self.ifree[:len(st.idx_free)] = torch.tensor(st.idx_free, dtype=torch.int32)
        self.ifree_n = torch.tensor([len(st.idx_free)], dtype=torch.int32, device="cuda")
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.step = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.ws = torch.empty(_lib.workspace_bytes(_lib.HS_OP_CACHE, B, P, self.T_stride, 1),
                              dtype=torch.uint8, device="cuda")
        self.batch = _lib.make_batch(B, P, self.T_stride, self.ctx)
        L, n_rows = st.pool.shape[:2]
        pitch, layer_rows = (L, 1) if interleaved else (0, B * self.T_stride)
        self.res = _lib.Residency(0, L, _lib.HS_E4M3, pitch, n_rows, layer_rows,
                                  self.bt.data_ptr(), None, None, None, None,
                                  self.step.data_ptr(), self.err.data_ptr(), self.pool.data_ptr(),
                                  self.row_scale.data_ptr(), _lib.host_device_ptr(self.host_rows),
                                  self.host_scale.data_ptr(), self.host_bt.data_ptr())
        self.idx = _lib.IndexCache(_lib.HS_E4M3, st.idx_pool.shape[2], self.idx_pool.data_ptr(),
                                   self.idx_scale.data_ptr(), self.idx_bt.data_ptr())
        self.cap = cap
        self.P = P

    def free_list(self, capacity=None):
        return self.lib.FreeList(self.free.data_ptr(), self.free_n.data_ptr(),
                                 self.cap if capacity is None else capacity, 0)

    def idx_free_list(self):
        return self.lib.FreeList(self.ifree.data_ptr(), self.ifree_n.data_ptr(),
                                 self.ifree.numel(), 0)

    def compare(self, st: co.CacheState, what: str):
        torch.cuda.synchronize()
        eq = lambda d, h, name: np.testing.assert_array_equal(d.cpu().numpy(), h,
                                                              err_msg=f"{what}: {name}")
        eq(self.ctx, st.ctx_len, "ctx_len")
        eq(self.bt, st.bt, "bt")
        eq(self.idx_bt, st.idx_bt, "idx_bt")
        eq(self.host_bt, st.host_bt, "host_bt")
        n = int(self.free_n.item())
        assert self.free[:n].cpu().numpy().tolist() == st.free, what
        m = int(self.ifree_n.item())
        assert self.ifree[:m].cpu().numpy().tolist() == st.idx_free, what
        eq(self.pool, st.pool, "pool")
        eq(self.row_scale.view(torch.int32), st.row_scale.view(np.int32), "row_scale")
        eq(self.idx_pool, st.idx_pool, "idx_pool")
        eq(self.idx_scale.view(torch.int32), st.idx_scale.view(np.int32), "idx_scale")
        hr = self.host_rows.numpy()
        np.testing.assert_array_equal(hr.transpose(1, 0, 2) if self.inter else hr, st.host_rows,
                                      err_msg=what)
        hs = self.host_scale.view(torch.int32).cpu().numpy()
        np.testing.assert_array_equal(hs.T if self.inter else hs, st.host_scale.view(np.int32),
                                      err_msg=f"{what}: host_scale")


def _initial(rng, B=5, T_stride=1024, L=2, D=576, Dk=128, spare=10, spare_idx=12):
    MB = T_stride // 64
    ctx = np.array([0, 1, 63, 64, 700], dtype=np.int32)[:B]
    in_use = sum(-(-int(t) // 64) for t in ctx)
    nb, ni = in_use + spare, in_use + spare_idx
    order, iorder = list(rng.permutation(nb)), list(rng.permutation(ni))
    bt = np.full((B, MB), -1, np.int32)
    ibt = np.full((B, MB), -1, np.int32)
    for b in range(B):
        for p in range(-(-int(ctx[b]) // 64)):
            bt[b, p] = order.pop()
            ibt[b, p] = iorder.pop()
    return co.CacheState(
        ctx_len=ctx, bt=bt, idx_bt=ibt, host_bt=np.full((B, MB), -1, np.int64),
        pool=rng.integers(0, 256, (L, nb * 64, D)).astype(np.uint8),
        row_scale=rng.random((L, nb * 64)).astype(np.float32),
        idx_pool=rng.integers(0, 256, (ni, 64, Dk)).astype(np.uint8),
        idx_scale=rng.random(ni).astype(np.float32),
        host_rows=np.zeros((L, B * T_stride, D), np.uint8),
        host_scale=np.zeros((L, B * T_stride), np.float32),
        free=order, idx_free=iorder, free_capacity=nb)


@pytest.mark.parametrize("seed,layout", [(0, "layer_major"), (1, "layer_major"),
                                         (2, "interleaved")])
def test_cache_operations_against_oracle(seed, layout):
    from decode_indexer_logits_amd import _lib
    rng = np.random.default_rng(500 + seed)
    P = 4
    st = _initial(rng)
    dev = _Dev(st, P, interleaved=layout == "interleaved")
    dev.compare(st, "initial")
    B = len(st.ctx_len)
    L, _, D = st.pool.shape
    Dk = st.idx_pool.shape[2]
    seen = {"append": 0, "append_err": 0, "precopy": 0, "demote": 0, "demote_err": 0}
    for k in range(36):
        dev.err.zero_()
        op = ["append", "append", "precopy", "demote"][int(rng.integers(0, 4))]
        if k in (0, 29, 32):
            op = "precopy"                                     # pages to demote later
        if k == 1:
            op = "precopy_all"
        if k in (2, 30, 33):
            op = "demote_small" if k == 2 else "append_bad"
        if k in (31, 34):
            op = "demote_small"
        if op.startswith("append"):
            n_new = rng.integers(0, P + 1, B).astype(np.int32)
            if op == "append_bad":
                n_new[int(rng.integers(0, B))] = P + 1         # more than P: nothing appended
            rows = rng.integers(0, 256, (B, P, L, D)).astype(np.uint8)
            rsc = rng.random((B, P, L)).astype(np.float32)
            keys = rng.integers(0, 256, (B, P, Dk)).astype(np.uint8)
            ksc = rng.random((B, P)).astype(np.float32)
            want = co.append_tokens(st, n_new, rows, rsc, keys, ksc)
            cu = lambda a: torch.from_numpy(a).cuda()
            _lib.append_tokens(dev.batch, dev.ctx, cu(n_new), dev.res, cu(rows), cu(rsc), dev.idx,
                               cu(keys), cu(ksc), dev.free_list(), dev.idx_free_list(), dev.ws)
            seen["append_err" if want else "append"] += 1
        elif op.startswith("precopy"):
            mp = 1024 if op == "precopy_all" else int(rng.integers(1, 4))
            got = co.precopy_pages(st, mp)
            _lib.precopy_pages(dev.batch, dev.res, mp)
            want = 0
            seen["precopy"] += len(got)
        else:
            n_dem = rng.integers(0, 4, B).astype(np.int32)
            tail = int(rng.integers(1, 4))
            cap = st.free_capacity
            if op == "demote_small":
                n_dem[:] = 3
                tail = 1
                cap = len(st.free)                             # no room: nothing demoted
            saved = st.free_capacity
            st.free_capacity = cap
            want, plan = co.demote_pages(st, n_dem, tail)
            st.free_capacity = saved
            _lib.demote_pages(dev.batch, dev.res, torch.from_numpy(n_dem).cuda(), tail,
                              dev.free_list(cap), dev.ws)
            seen["demote_err" if want else "demote"] += 1 if want else len(plan)
        dev.compare(st, f"op {k} ({op})")
        assert int(dev.err.item()) == want, (k, op, int(dev.err.item()), want)
    _say(seen, "ctx", st.ctx_len.tolist(), "free", len(st.free), "idx free", len(st.idx_free))
    assert all(v > 0 for v in seen.values()), seen
