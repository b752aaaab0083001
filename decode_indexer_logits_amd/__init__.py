"""MI355X-native decode step of indexer-driven sparse MLA attention with hybrid
GPU/host KV residency.

The compute path is the HIP library ``libhisparse.so`` (C ABI in
include/hs.h): indexer scores, top-K, fused resolve with single-row faults from
pinned host memory, and sparse MLA attention, all on gfx950.  ``_lib`` binds it
with ctypes; ``device`` holds the torch plumbing (device tensors, pinned host
pool, streams) that drives one step.
"""

from ._lib import (HsError, load, abi_version, workspace_bytes, host_device_ptr,  # noqa: F401
                   indexer_scores, topk, resolve_rows, sparse_mla_decode, make_batch, Batch,
                   Residency, HS_OP_TOPK, HS_OP_MLA)
