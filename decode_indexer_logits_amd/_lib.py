"""ctypes binding of ``libhisparse.so`` (the C ABI declared in include/hs.h).

Argument marshalling only: every function takes torch tensors (device memory,
or pinned host memory for the host pool), passes their addresses and sizes to
the library, and raises ``HsError`` on a nonzero status.  All work runs in the
library's HIP kernels on the given stream (torch's current stream by
default).  Loading fails loudly if the library has not been built.
"""

from __future__ import annotations

import ctypes
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libhisparse.so"

HS_F32, HS_BF16, HS_E4M3 = 0, 1, 2
DTYPES = {"f32": HS_F32, "bf16": HS_BF16, "e4m3": HS_E4M3}
HS_OP_INDEXER, HS_OP_TOPK, HS_OP_RESOLVE, HS_OP_MLA, HS_OP_CACHE = 0, 1, 2, 3, 4
DEVERR_VICTIMS, DEVERR_NO_HOST = 1, 2
DEVERR_APPEND_RANGE, DEVERR_APPEND_NO_BLOCK, DEVERR_DEMOTE_FULL = 4, 8, 16

EXPORTS = ["hs_indexer_scores", "hs_quantize_queries", "hs_topk", "hs_indexer_topk",
           "hs_indexer_topk_noalloc", "hs_indexer_topk_scores", "hs_indexer_topk_select",
           "hs_resolve_rows", "hs_resolve_tables", "hs_copy_faults", "hs_copy_faults_layers",
           "hs_sparse_mla_decode", "hs_sparse_mla_decode_layers", "hs_mla_layers_workspace_bytes",
           "hs_topk_sharded", "hs_topk_sharded_workspace_bytes",
           "hs_sparse_mla_decode_sharded", "hs_mla_sharded_workspace_bytes",
           "hs_indexer_topk_select_resolve",
           "hs_append_tokens", "hs_precopy_pages", "hs_demote_pages",
           "hs_workspace_bytes", "hs_host_device_ptr", "hs_last_error", "hs_abi_version"]


class HsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hs status {status}: {msg}")
        self.status = status


class Batch(ctypes.Structure):
    _fields_ = [("B", c_int32), ("P", c_int32), ("T_stride", c_int32), ("max_blocks", c_int32),
                ("ctx_len", c_void_p)]


class Residency(ctypes.Structure):
    _fields_ = [("C", c_int32), ("L", c_int32), ("kv_t", c_int32), ("host_row_pitch", c_int32),
                ("pool_layer_rows", c_int64), ("host_layer_rows", c_int64),
                ("bt", c_void_p), ("hot_blocks", c_void_p), ("tok2slot", c_void_p),
                ("slot2tok", c_void_p), ("stamp", c_void_p), ("step", c_void_p),
                ("err", c_void_p), ("pool", c_void_p), ("row_scale", c_void_p),
                ("host_rows", c_void_p), ("host_scale", c_void_p), ("host_bt", c_void_p)]


class FreeList(ctypes.Structure):
    _fields_ = [("blocks", c_void_p), ("count", c_void_p), ("capacity", c_int32),
                ("pad_", c_int32)]


class IndexCache(ctypes.Structure):
    _fields_ = [("k_t", c_int32), ("D_idx", c_int32), ("pool", c_void_p), ("scale", c_void_p),
                ("bt", c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    """The loaded library (raises ImportError if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} not found: build it with "
                          "`python -m decode_indexer_logits_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(str(LIB_PATH))
    P = c_void_p
    lib.hs_indexer_scores.argtypes = [P, c_int32, c_int32, c_int32, P, P, c_int32, P, P, P, P, P, P]
    lib.hs_quantize_queries.argtypes = [P, c_int32, c_int32, P, P, P, P, P]
    lib.hs_topk.argtypes = [P, c_int32, P, P, P, c_size_t, P]
    lib.hs_indexer_topk.argtypes = [P, c_int32, c_int32, c_int32, P, P, c_int32, P, P, P, P, P,
                                    c_int32, P, P, c_size_t, P]
    lib.hs_indexer_topk_noalloc.argtypes = [P, c_int32, c_int32, c_int32, P, P, c_int32, P, P, P,
                                            P, P, c_int32, P, P]
    lib.hs_indexer_topk_scores.argtypes = [P, c_int32, c_int32, c_int32, P, P, c_int32, P, P, P,
                                           P, P, c_int32, P, c_size_t, P]
    lib.hs_indexer_topk_select.argtypes = [P, c_int32, c_int32, P, P, P, c_size_t, P]
    lib.hs_resolve_rows.argtypes = [P, c_int32, P, P, P, P, P, P, c_size_t, P]
    lib.hs_resolve_tables.argtypes = [P, c_int32, P, P, P, P, P, P]
    lib.hs_indexer_topk_select_resolve.argtypes = [P, c_int32, c_int32, P, P, P, c_size_t, P, P,
                                                   P, P, P]
    lib.hs_copy_faults.argtypes = [P, c_int32, P, P, P, c_int32, P]
    lib.hs_copy_faults_layers.argtypes = [P, c_int32, P, P, P, c_int32, c_int32, c_int32, P]
    lib.hs_sparse_mla_decode.argtypes = [P, c_int32, c_int32, c_int32, P, c_int32, P, P, P,
                                         c_float, P, P, P, c_size_t, P]
    lib.hs_sparse_mla_decode_layers.argtypes = [P, c_int32, c_int32, c_int32, c_int32, P, c_int32,
                                                P, c_int64, P, P, c_float, P, P, P, c_size_t, P]
    lib.hs_sparse_mla_decode_layers.restype = c_int32
    lib.hs_mla_layers_workspace_bytes.argtypes = [c_int32] * 5
    lib.hs_mla_layers_workspace_bytes.restype = c_size_t
    lib.hs_sparse_mla_decode_sharded.argtypes = [P, c_int32, c_int32, c_int32, c_int32, P, c_int32,
                                                 P, P, P, P, c_float, P, P, P, P, P, c_size_t, P]
    lib.hs_sparse_mla_decode_sharded.restype = c_int32
    lib.hs_mla_sharded_workspace_bytes.argtypes = [c_int32] * 5
    lib.hs_mla_sharded_workspace_bytes.restype = c_size_t
    lib.hs_topk_sharded.argtypes = [P, c_int32, c_int32, P, P, P, c_size_t, P]
    lib.hs_topk_sharded.restype = c_int32
    lib.hs_topk_sharded_workspace_bytes.argtypes = [c_int32] * 4
    lib.hs_topk_sharded_workspace_bytes.restype = c_size_t
    lib.hs_append_tokens.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, c_size_t, P]
    lib.hs_precopy_pages.argtypes = [P, P, c_int32, P]
    lib.hs_demote_pages.argtypes = [P, P, P, c_int32, P, P, c_size_t, P]
    for f in ("hs_append_tokens", "hs_precopy_pages", "hs_demote_pages"):
        getattr(lib, f).restype = c_int32
    for f in ("hs_indexer_scores", "hs_quantize_queries", "hs_topk", "hs_indexer_topk",
              "hs_indexer_topk_noalloc", "hs_indexer_topk_scores", "hs_indexer_topk_select",
              "hs_resolve_rows", "hs_resolve_tables", "hs_copy_faults", "hs_copy_faults_layers",
              "hs_sparse_mla_decode", "hs_host_device_ptr"):
        getattr(lib, f).restype = c_int32
    lib.hs_workspace_bytes.argtypes = [c_int32] * 6
    lib.hs_workspace_bytes.restype = c_size_t
    lib.hs_host_device_ptr.argtypes = [P, ctypes.POINTER(c_void_p)]
    lib.hs_last_error.restype = ctypes.c_char_p
    lib.hs_abi_version.restype = c_int32
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(st: int):
    if st != 0:
        raise HsError(st, load().hs_last_error().decode())


def abi_version() -> int:
    return load().hs_abi_version()


def last_error() -> str:
    return load().hs_last_error().decode()


def workspace_bytes(op: int, B: int, P: int, T_stride: int, K: int, Hq: int = 16) -> int:
    return load().hs_workspace_bytes(op, B, P, T_stride, K, Hq)


def host_device_ptr(pinned) -> int:
    out = c_void_p()
    _check(load().hs_host_device_ptr(pinned.data_ptr(), ctypes.byref(out)))
    return out.value


def make_batch(B: int, P: int, T_stride: int, ctx_len) -> Batch:
    """The batch struct; it keeps a reference to ctx_len, whose address it holds."""
    b = Batch(B, P, T_stride, T_stride // 64, _ptr(ctx_len))
    b._ctx_len_ref = ctx_len
    return b


def indexer_scores(batch: Batch, H: int, D: int, q_t: str, q_idx, w, k_t: str, idx_pool,
                   idx_scale, idx_bt, bias, scores, stream=None):
    _check(load().hs_indexer_scores(ctypes.byref(batch), H, D, DTYPES[q_t], _ptr(q_idx), _ptr(w),
                                    DTYPES[k_t], _ptr(idx_pool), _ptr(idx_scale), _ptr(idx_bt),
                                    _ptr(bias), _ptr(scores), _stream(stream)))


def quantize_queries(batch: Batch, H: int, D: int, q_idx, w, q8, w_scaled, stream=None):
    _check(load().hs_quantize_queries(ctypes.byref(batch), H, D, _ptr(q_idx), _ptr(w), _ptr(q8),
                                      _ptr(w_scaled), _stream(stream)))


def topk(batch: Batch, K: int, scores, out, ws, stream=None):
    _check(load().hs_topk(ctypes.byref(batch), K, _ptr(scores), _ptr(out), _ptr(ws),
                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def indexer_topk(batch: Batch, H: int, D: int, q_t: str, q_idx, w, k_t: str, idx_pool, idx_scale,
                 idx_bt, bias, scores, K: int, out, ws, stream=None):
    _check(load().hs_indexer_topk(ctypes.byref(batch), H, D, DTYPES[q_t], _ptr(q_idx), _ptr(w),
                                  DTYPES[k_t], _ptr(idx_pool), _ptr(idx_scale), _ptr(idx_bt),
                                  _ptr(bias), _ptr(scores), K, _ptr(out), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(stream)))


def indexer_topk_scores(batch: Batch, H: int, D: int, q_t: str, q_idx, w, k_t: str, idx_pool,
                        idx_scale, idx_bt, bias, scores, K: int, ws, stream=None):
    _check(load().hs_indexer_topk_scores(ctypes.byref(batch), H, D, DTYPES[q_t], _ptr(q_idx),
                                         _ptr(w), DTYPES[k_t], _ptr(idx_pool), _ptr(idx_scale),
                                         _ptr(idx_bt), _ptr(bias), _ptr(scores), K, _ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size(),
                                         _stream(stream)))


def indexer_topk_select(batch: Batch, q_t: str, K: int, scores, out, ws, stream=None):
    _check(load().hs_indexer_topk_select(ctypes.byref(batch), DTYPES[q_t], K, _ptr(scores),
                                         _ptr(out), _ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size(),
                                         _stream(stream)))


def indexer_topk_noalloc(batch: Batch, H: int, D: int, q_t: str, q_idx, w, k_t: str, idx_pool,
                         idx_scale, idx_bt, bias, scores, K: int, out, stream=None):
    _check(load().hs_indexer_topk_noalloc(ctypes.byref(batch), H, D, DTYPES[q_t], _ptr(q_idx),
                                          _ptr(w), DTYPES[k_t], _ptr(idx_pool), _ptr(idx_scale),
                                          _ptr(idx_bt), _ptr(bias), _ptr(scores), K, _ptr(out),
                                          _stream(stream)))


def resolve_rows(batch: Batch, K: int, topk_t, res: Residency, row_ids, faults, counts,
                 stream=None):
    _check(load().hs_resolve_rows(ctypes.byref(batch), K, _ptr(topk_t), ctypes.byref(res),
                                  _ptr(row_ids), _ptr(faults), _ptr(counts), None, 0,
                                  _stream(stream)))


def resolve_tables(batch: Batch, K: int, topk_t, res: Residency, row_ids, faults, counts,
                   stream=None):
    _check(load().hs_resolve_tables(ctypes.byref(batch), K, _ptr(topk_t), ctypes.byref(res),
                                    _ptr(row_ids), _ptr(faults), _ptr(counts), _stream(stream)))


def indexer_topk_select_resolve(batch: Batch, q_t: str, K: int, scores, topk_t, ws,
                                res: Residency, row_ids, faults, counts, stream=None):
    _check(load().hs_indexer_topk_select_resolve(
        ctypes.byref(batch), DTYPES[q_t], K, _ptr(scores), _ptr(topk_t), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), ctypes.byref(res), _ptr(row_ids),
        _ptr(faults), _ptr(counts), _stream(stream)))


def copy_faults(batch: Batch, K: int, res: Residency, faults, counts, workgroups: int = 0,
                stream=None):
    _check(load().hs_copy_faults(ctypes.byref(batch), K, ctypes.byref(res), _ptr(faults),
                                 _ptr(counts), workgroups, _stream(stream)))


def copy_faults_layers(batch: Batch, K: int, res: Residency, faults, counts, layer0: int,
                       n_layers: int, workgroups: int = 0, stream=None):
    _check(load().hs_copy_faults_layers(ctypes.byref(batch), K, ctypes.byref(res), _ptr(faults),
                                        _ptr(counts), layer0, n_layers, workgroups,
                                        _stream(stream)))


def sparse_mla_decode(batch: Batch, K: int, Hq: int, q_t: str, q, kv_t: str, pool, row_scale,
                      row_ids, sm_scale: float, out, lse, ws, stream=None):
    _check(load().hs_sparse_mla_decode(ctypes.byref(batch), K, Hq, DTYPES[q_t], _ptr(q),
                                       DTYPES[kv_t], _ptr(pool), _ptr(row_scale), _ptr(row_ids),
                                       float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                       0 if ws is None else ws.numel() * ws.element_size(),
                                       _stream(stream)))


def sparse_mla_decode_layers(batch: Batch, K: int, Hq: int, L: int, q_t: str, q, kv_t: str, pool,
                             pool_layer_rows: int, row_scale, row_ids, sm_scale: float, out, lse,
                             ws, stream=None):
    _check(load().hs_sparse_mla_decode_layers(
        ctypes.byref(batch), K, Hq, L, DTYPES[q_t], _ptr(q), DTYPES[kv_t], _ptr(pool),
        int(pool_layer_rows), _ptr(row_scale), _ptr(row_ids), float(sm_scale), _ptr(out),
        _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def mla_layers_workspace_bytes(B: int, P: int, K: int, Hq: int, L: int) -> int:
    return load().hs_mla_layers_workspace_bytes(B, P, K, Hq, L)


def sparse_mla_decode_sharded(batch: Batch, K: int, S: int, Hq: int, q_t: str, q, kv_t: str, pool,
                              row_scale, topk, row_ids, sm_scale: float, shard_out, shard_lse,
                              out, lse, ws, stream=None):
    _check(load().hs_sparse_mla_decode_sharded(
        ctypes.byref(batch), K, S, Hq, DTYPES[q_t], _ptr(q), DTYPES[kv_t], _ptr(pool),
        _ptr(row_scale), _ptr(topk), _ptr(row_ids), float(sm_scale), _ptr(shard_out),
        _ptr(shard_lse), _ptr(out), _ptr(lse), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def mla_sharded_workspace_bytes(B: int, P: int, K: int, S: int, Hq: int) -> int:
    return load().hs_mla_sharded_workspace_bytes(B, P, K, S, Hq)


def append_tokens(batch: Batch, ctx_len, n_new, res: Residency, new_rows, new_row_scale,
                  idx: IndexCache, new_keys, new_key_scale, latent_free: FreeList,
                  idx_free: FreeList, ws, stream=None):
    _check(load().hs_append_tokens(ctypes.byref(batch), _ptr(ctx_len), _ptr(n_new),
                                   ctypes.byref(res), _ptr(new_rows), _ptr(new_row_scale),
                                   ctypes.byref(idx), _ptr(new_keys), _ptr(new_key_scale),
                                   ctypes.byref(latent_free), ctypes.byref(idx_free), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(stream)))


def precopy_pages(batch: Batch, res: Residency, max_pages: int, stream=None):
    _check(load().hs_precopy_pages(ctypes.byref(batch), ctypes.byref(res), max_pages,
                                   _stream(stream)))


def demote_pages(batch: Batch, res: Residency, n_demote, tail_pages: int, latent_free: FreeList,
                 ws, stream=None):
    _check(load().hs_demote_pages(ctypes.byref(batch), ctypes.byref(res), _ptr(n_demote),
                                  tail_pages, ctypes.byref(latent_free), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(stream)))


def topk_sharded_workspace_bytes(B: int, T_stride: int, K: int, S: int) -> int:
    return load().hs_topk_sharded_workspace_bytes(B, T_stride, K, S)


def topk_sharded(batch: Batch, K: int, S: int, scores, out, ws, stream=None):
    _check(load().hs_topk_sharded(ctypes.byref(batch), K, S, _ptr(scores), _ptr(out), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(stream)))
