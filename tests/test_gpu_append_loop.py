"""Decode loop with KV append on the GPU, checked step by step against the oracle.

A small no-residency workload (two requests of 8192 tokens, two layers, hot
buffers of 2K rows) runs five decode steps; after each of the first four every
request appends one token through hs_append_tokens, so the context grows from
8192 to 8196 and the first append opens a new page (a latent block and an
indexer block popped from the free lists).  After every append the device's
tables, free lists, indexer cache and the appended latent rows equal the
oracle's append (oracle/cache_ops.py) run on the oracle's own copy of those
tables; every step is checked stage by stage (scores, top-K, resolve with the
new page resident, fault copies, attention) against the oracle on the grown
context.
"""
import sys

import numpy as np
import pytest

import gpu_check as gc
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


@pytest.mark.parametrize("layout", ["interleaved", "layer_major"])
def test_append_loop_against_oracle(layout):
    from decode_indexer_logits_amd.device import DeviceStep
    _say(f"decode loop with append, host pool {layout}")
    wl = gen.norescache_1m(B=2, T=8192, K=256, L=2, steps=5, append=True)
    ds = DeviceStep(wl, host_layout=layout)
    ost = gc.oracle_state(wl)
    cs = gc.cache_mirror(wl)
    for s in range(1, wl.steps + 1):
        ds.set_queries(s)
        ds.run()
        ost, rr, info = gc.full_check(ds, wl, ost, s=s, attn_tol=2e-2)
        c = info["counts"]
        _say(s, "ctx", wl.ctx_len.tolist(), "counts", c.tolist())
        if s < wl.steps:
            ost = gc.append_and_check(ds, wl, ost, cs, s)
    assert wl.ctx_len.tolist() == [8192 + wl.steps - 1] * wl.B
