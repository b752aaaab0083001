"""The C-ABI library: loads, exports every declared symbol, validates on the
host, and its struct layouts match the binding (CPU only, no compute calls)."""
import ctypes
import os
import re
import subprocess

import pytest

from decode_indexer_logits_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hs.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = _lib.load()
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", str(_lib.LIB_PATH)], capture_output=True,
                         text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n
    assert _lib.abi_version() == 1


def test_probe_library_is_separate_and_loads():
    """The benchmark's bandwidth probes live in their own library; the decode-step
    library exports none of them."""
    probe = _lib.LIB_PATH.parent / "libhsprobe.so"
    lib = ctypes.CDLL(str(probe))
    for n in ("hsp_read_stream", "hsp_read_pages", "hsp_host_gather"):
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", str(_lib.LIB_PATH)], capture_output=True,
                         text=True).stdout
    assert "hsp_" not in out


def test_struct_layout_matches_header(tmp_path):
    c = tmp_path / "probe.c"
    c.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "hs.h"\n'
                 "int main(void){printf(\"%zu %zu %zu %zu %zu %zu\\n\", sizeof(hs_batch),"
                 " offsetof(hs_batch, ctx_len), sizeof(hs_residency),"
                 " offsetof(hs_residency, pool_layer_rows), offsetof(hs_residency, bt),"
                 " offsetof(hs_residency, host_bt));"
                 " printf(\"%zu %zu %zu %zu %zu\\n\", sizeof(hs_free_list), offsetof(hs_free_list, capacity),"
                 " sizeof(hs_index_cache), offsetof(hs_index_cache, pool), offsetof(hs_index_cache, bt));"
                 " return 0;}\n")
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)], check=True)
    vals = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()))
    assert vals == [ctypes.sizeof(_lib.Batch), _lib.Batch.ctx_len.offset,
                    ctypes.sizeof(_lib.Residency), _lib.Residency.pool_layer_rows.offset,
                    _lib.Residency.bt.offset, _lib.Residency.host_bt.offset,
                    ctypes.sizeof(_lib.FreeList), _lib.FreeList.capacity.offset,
                    ctypes.sizeof(_lib.IndexCache), _lib.IndexCache.pool.offset,
                    _lib.IndexCache.bt.offset]


def test_host_validation_rejects_bad_arguments_without_launching():
    lib = _lib.load()
    fake = ctypes.c_void_p(16)            # never dereferenced: validation fails first
    b = _lib.Batch(2, 1, 1024, 16, 16)
    assert lib.hs_topk(None, 8, fake, fake, fake, 1 << 30, None) == 1
    assert lib.hs_topk(ctypes.byref(b), 0, fake, fake, fake, 1 << 30, None) == 2
    assert lib.hs_topk(ctypes.byref(b), 9000, fake, fake, fake, 1 << 30, None) == 2
    assert lib.hs_topk(ctypes.byref(b), 8, fake, fake, fake, 10, None) == 5
    assert "workspace" in _lib.last_error()
    assert lib.hs_topk(ctypes.byref(b), 8, ctypes.c_void_p(20), fake, fake, 1 << 30, None) == 6
    assert "scores" in _lib.last_error()
    bad = _lib.Batch(2, 5, 1024, 16, 16)
    assert lib.hs_topk(ctypes.byref(bad), 8, fake, fake, fake, 1 << 30, None) == 2
    # the allocation-free variant refuses sizes beyond its static scratch
    big = _lib.Batch(64, 1, 1 << 20, (1 << 20) // 64, 16)
    assert lib.hs_indexer_topk_noalloc(ctypes.byref(big), 64, 128, 1, fake, fake, 2, fake, fake,
                                       fake, None, fake, 2048, fake, None) == 5
    assert "static scratch" in _lib.last_error()
    bad = _lib.Batch(2, 1, 1000, 15, 16)
    assert lib.hs_topk(ctypes.byref(bad), 8, fake, fake, fake, 1 << 30, None) == 2
    # indexer dtype and shape checks
    assert lib.hs_indexer_scores(ctypes.byref(b), 64, 96, 1, fake, fake, 2, fake, None, fake,
                                 None, fake, None) == 2
    assert lib.hs_indexer_scores(ctypes.byref(b), 64, 128, 1, fake, fake, 0, fake, None, fake,
                                 None, fake, None) == 3
    assert lib.hs_indexer_scores(ctypes.byref(b), 24, 128, 1, fake, fake, 2, fake, None, fake,
                                 None, fake, None) == 2
    assert lib.hs_indexer_scores(ctypes.byref(b), 64, 128, 1, ctypes.c_void_p(17), fake, 2, fake,
                                 None, fake, None, fake, None) == 6
    # E4M3 queries: E4M3 keys and D = 128 only
    assert lib.hs_indexer_scores(ctypes.byref(b), 64, 64, 2, fake, fake, 2, fake, None, fake,
                                 None, fake, None) == 2
    assert lib.hs_indexer_scores(ctypes.byref(b), 64, 128, 2, fake, fake, 1, fake, None, fake,
                                 None, fake, None) == 3
    assert lib.hs_indexer_scores(ctypes.byref(b), 40, 128, 2, fake, fake, 2, fake, None, fake,
                                 None, fake, None) == 2
    # query quantization
    assert lib.hs_quantize_queries(ctypes.byref(b), 64, 128, fake, fake, None, fake, None) == 1
    assert lib.hs_quantize_queries(ctypes.byref(b), 64, 96, fake, fake, fake, fake, None) == 2
    assert lib.hs_quantize_queries(ctypes.byref(b), 65, 128, fake, fake, fake, fake, None) == 2
    assert lib.hs_quantize_queries(ctypes.byref(b), 64, 128, ctypes.c_void_p(18), fake, fake,
                                   fake, None) == 6
    # resolve: capacity rule C >= P*K
    res = _lib.Residency(128, 1, 2, 0, 0, 0, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16)
    assert lib.hs_resolve_rows(ctypes.byref(b), 256, fake, ctypes.byref(res), fake, fake, fake,
                               None, 0, None) == 4
    assert "C=128" in _lib.last_error()
    res.C = 100
    assert lib.hs_resolve_rows(ctypes.byref(b), 64, fake, ctypes.byref(res), fake, fake, fake,
                               None, 0, None) == 2
    # layer-range copies: the range must lie inside [0, L)
    res.C = 128
    for l0, nl in ((1, 1), (0, 2), (-1, 1), (0, 0)):
        assert lib.hs_copy_faults_layers(ctypes.byref(b), 64, ctypes.byref(res), fake, fake, l0,
                                         nl, 0, None) == 2, (l0, nl)
        assert "layers" in _lib.last_error()
    # attention: heads in groups of 16, at most 128; workspace
    for bad_hq in (8, 24, 144):
        assert lib.hs_sparse_mla_decode(ctypes.byref(b), 2048, bad_hq, 1, fake, 2, fake, fake,
                                        fake, 0.1, fake, None, None, 0, None) == 2
    for hq in (16, 32, 128):
        assert lib.hs_sparse_mla_decode(ctypes.byref(b), 2048, hq, 1, fake, 2, fake, fake, fake,
                                        0.1, fake, None, None, 0, None) == 5
    assert lib.hs_mla_layers_workspace_bytes(8, 1, 2048, 24, 1) == 0
    # token-sharded attention: S in [1, 64] dividing T_stride, outputs required
    def sharded(K=2048, S=4, Hq=16, q_t=1, kv_t=2, rs=fake, so=fake, ws=None, ws_bytes=0):
        return lib.hs_sparse_mla_decode_sharded(ctypes.byref(b), K, S, Hq, q_t, fake, kv_t, fake,
                                                rs, fake, fake, 0.1, so, fake, fake, None, ws,
                                                ws_bytes, None)
    assert sharded(S=0) == 2 and sharded(S=65) == 2 and sharded(S=3) == 2
    assert sharded(Hq=40) == 2 and sharded(K=8193) == 2
    assert sharded(so=None) == 1
    assert sharded() == 5
    need = lib.hs_mla_sharded_workspace_bytes(2, 1, 2048, 4, 16)
    assert need > 0 and lib.hs_mla_sharded_workspace_bytes(8, 1, 2048, 65, 16) == 0
    big = ctypes.c_void_p(1 << 20)
    assert sharded(ws=big, ws_bytes=need - 1) == 5
    assert sharded(q_t=0, ws=big, ws_bytes=need) == 3
    assert sharded(q_t=0, kv_t=0, ws=big, ws_bytes=need) == 3     # F32 rows take no scale
    assert sharded(rs=None, ws=big, ws_bytes=need) == 1           # E4M3 rows need scales


def test_cache_operations_validate_on_the_host():
    lib = _lib.load()
    fake = ctypes.c_void_p(16)
    ctx = ctypes.c_void_p(32)
    b = _lib.Batch(2, 1, 1024, 16, 32)
    res = _lib.Residency(0, 1, 2, 0, 1 << 20, 2048, 16, None, None, None, None, 16, 16, 16, 16,
                         16, 16, 16)
    idx = _lib.IndexCache(2, 128, 16, 16, 16)
    fl = _lib.FreeList(16, 16, 8, 0)
    ws_n = _lib.workspace_bytes(_lib.HS_OP_CACHE, 2, 1, 1024, 1)
    assert ws_n >= (2 + 4) * 4
    args = lambda c, w=ws_n: (ctypes.byref(b), c, fake, ctypes.byref(res), fake, fake,
                              ctypes.byref(idx), fake, fake, ctypes.byref(fl), ctypes.byref(fl),
                              fake, w, None)
    assert lib.hs_append_tokens(*args(fake)) == 2                 # ctx_len is not the batch's
    assert lib.hs_append_tokens(*args(ctx, 4)) == 5               # workspace too small
    bad = _lib.FreeList(16, None, 8, 0)
    assert lib.hs_append_tokens(ctypes.byref(b), ctx, fake, ctypes.byref(res), fake, fake,
                                ctypes.byref(idx), fake, fake, ctypes.byref(bad),
                                ctypes.byref(fl), fake, ws_n, None) == 1
    idx64 = _lib.IndexCache(2, 96, 16, 16, 16)
    assert lib.hs_append_tokens(ctypes.byref(b), ctx, fake, ctypes.byref(res), fake, fake,
                                ctypes.byref(idx64), fake, fake, ctypes.byref(fl),
                                ctypes.byref(fl), fake, ws_n, None) == 2
    assert lib.hs_precopy_pages(ctypes.byref(b), ctypes.byref(res), 0, None) == 2
    assert lib.hs_precopy_pages(ctypes.byref(b), ctypes.byref(res), 2000, None) == 2
    # two layers of a 2 x 1024-token host pool: planes of 2048 rows, or the two rows of a
    # token side by side (pitch 2, layer stride 1) are accepted; overlapping layouts are not
    def two_layers(pitch, layer_rows):
        return _lib.Residency(0, 2, 2, pitch, 1 << 20, layer_rows, 16, None, None, None, None, 16,
                              16, 16, 16, 16, 16, 16)
    bad_layouts = [(0, 2047), (1, 1000), (2, 2), (3, 2), (-1, 2048)]
    for pitch, lr in bad_layouts:
        r2 = two_layers(pitch, lr)
        assert lib.hs_precopy_pages(ctypes.byref(b), ctypes.byref(r2), 4, None) == 2, (pitch, lr)
    assert lib.hs_demote_pages(ctypes.byref(b), ctypes.byref(res), fake, 0, ctypes.byref(fl),
                               fake, ws_n, None) == 2            # the tail must stay
    assert lib.hs_demote_pages(ctypes.byref(b), ctypes.byref(res), None, 1, ctypes.byref(fl),
                               fake, ws_n, None) == 1


def test_attention_layers_validates_on_the_host():
    lib = _lib.load()
    fake = ctypes.c_void_p(16)
    b = _lib.Batch(2, 1, 1024, 16, 32)
    call = lambda K, Hq, L, plr, ws_n: lib.hs_sparse_mla_decode_layers(
        ctypes.byref(b), K, Hq, L, _lib.HS_BF16, fake, _lib.HS_E4M3, fake, plr, fake, fake,
        ctypes.c_float(0.05), fake, None, fake, ws_n, None)
    assert call(2048, 16, 0, 4096, 1 << 30) == 2            # L out of range
    assert call(2048, 16, 17, 4096, 1 << 30) == 2
    assert call(2048, 16, 4, 0, 1 << 30) == 2               # no layer stride for L > 1
    assert call(2048, 8, 4, 4096, 1 << 30) == 2             # one shard of 16 heads
    need = _lib.mla_layers_workspace_bytes(2, 1, 2048, 16, 4)
    assert need > 0 and call(2048, 16, 4, 4096, need - 1) == 5
    assert _lib.mla_layers_workspace_bytes(2, 1, 2048, 16, 1) == \
        _lib.workspace_bytes(_lib.HS_OP_MLA, 2, 1, 1024, 2048, 16)


def test_workspace_sizes():
    assert _lib.workspace_bytes(_lib.HS_OP_TOPK, 32, 1, 131072, 2048) >= 32 * 131072 * 8
    assert _lib.workspace_bytes(_lib.HS_OP_RESOLVE, 32, 1, 131072, 2048) == 0
    # 32 positions x 2048 rows split over many workgroups -> partials needed
    assert _lib.workspace_bytes(_lib.HS_OP_MLA, 32, 1, 131072, 2048) > 0
