// Host-side check of the C ABI's argument validation, built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code only.  Every call here is
// rejected before any launch (fake device pointers never reach a kernel), and
// the pure functions (workspace sizes, error text, version) run on extreme
// sizes.  Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/hs.h"

static int g_fail = 0;

#define EXPECT(call, code)                                                                 \
  do {                                                                                     \
    const hs_status st_ = (call);                                                          \
    if (st_ != (code)) {                                                                   \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call,  \
                   (int)st_, (int)(code), hs_last_error());                                \
      ++g_fail;                                                                            \
    }                                                                                      \
  } while (0)
#define CHECK(cond)                                                                        \
  do {                                                                                     \
    if (!(cond)) {                                                                         \
      std::fprintf(stderr, "line %d: %s failed\n", __LINE__, #cond);                       \
      ++g_fail;                                                                            \
    }                                                                                      \
  } while (0)

int main() {
  CHECK(hs_abi_version() == HS_ABI_VERSION);
  CHECK(std::strcmp(hs_last_error(), "") == 0);
  // fake device addresses: 16-byte aligned, never dereferenced
  void* f = reinterpret_cast<void*>(uintptr_t(1) << 20);
  void* odd = reinterpret_cast<void*>((uintptr_t(1) << 20) + 4);
  const int32_t* ctx = static_cast<const int32_t*>(f);
  float* ff = static_cast<float*>(f);
  int32_t* fi = static_cast<int32_t*>(f);

  // ---- batch geometry
  hs_batch b = {2, 1, 1024, 16, ctx};
  hs_batch bad = b;
  EXPECT(hs_topk(nullptr, 64, ff, fi, f, 1 << 30, nullptr), HS_ERR_NULL);
  bad.B = 0;
  EXPECT(hs_topk(&bad, 64, ff, fi, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  bad = b; bad.P = 5;
  EXPECT(hs_topk(&bad, 64, ff, fi, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  bad = b; bad.T_stride = 100;
  EXPECT(hs_topk(&bad, 64, ff, fi, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  bad = b; bad.max_blocks = 15;
  EXPECT(hs_topk(&bad, 64, ff, fi, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  bad = b; bad.ctx_len = nullptr;
  EXPECT(hs_topk(&bad, 64, ff, fi, f, 1 << 30, nullptr), HS_ERR_NULL);
  bad = b; bad.T_stride = 1 << 25; bad.max_blocks = (1 << 25) / 64;
  EXPECT(hs_topk(&bad, 64, ff, fi, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  CHECK(std::strlen(hs_last_error()) > 0);

  // ---- indexer
  EXPECT(hs_indexer_scores(&b, 64, 128, HS_BF16, nullptr, ff, HS_E4M3, f, ff, fi, nullptr, ff,
                           nullptr), HS_ERR_NULL);
  EXPECT(hs_indexer_scores(&b, 65, 128, HS_BF16, f, ff, HS_E4M3, f, ff, fi, nullptr, ff, nullptr),
         HS_ERR_SHAPE);
  EXPECT(hs_indexer_scores(&b, 64, 96, HS_BF16, f, ff, HS_E4M3, f, ff, fi, nullptr, ff, nullptr),
         HS_ERR_SHAPE);
  EXPECT(hs_indexer_scores(&b, 64, 128, HS_BF16, f, ff, HS_F32, f, nullptr, fi, nullptr, ff,
                           nullptr), HS_ERR_DTYPE);
  EXPECT(hs_indexer_scores(&b, 64, 128, HS_BF16, odd, ff, HS_E4M3, f, ff, fi, nullptr, ff,
                           nullptr), HS_ERR_ALIGN);
  EXPECT(hs_quantize_queries(&b, 64, 96, f, ff, static_cast<uint8_t*>(f), ff, nullptr),
         HS_ERR_SHAPE);
  void* odd2 = reinterpret_cast<void*>((uintptr_t(1) << 20) + 2);   // queries need 4 bytes here
  EXPECT(hs_quantize_queries(&b, 64, 128, odd2, ff, static_cast<uint8_t*>(f), ff, nullptr),
         HS_ERR_ALIGN);

  // ---- top-K and its fused / sharded / allocation-free forms
  const size_t tk = hs_workspace_bytes(HS_OP_TOPK, 2, 1, 1024, 64, 16);
  CHECK(tk > 0);
  EXPECT(hs_topk(&b, 0, ff, fi, f, tk, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_topk(&b, 8193, ff, fi, f, tk, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_topk(&b, 64, nullptr, fi, f, tk, nullptr), HS_ERR_NULL);
  EXPECT(hs_topk(&b, 64, reinterpret_cast<float*>(odd), fi, f, tk, nullptr), HS_ERR_ALIGN);
  EXPECT(hs_topk(&b, 64, ff, fi, f, tk - 1, nullptr), HS_ERR_WORKSPACE);
  hs_batch b4 = {2, 4, 1024, 16, ctx};
  EXPECT(hs_topk_sharded(&b4, 64, 4, ff, fi, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_topk_sharded(&b, 64, 0, ff, fi, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_topk_sharded(&b, 64, 65, ff, fi, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_topk_sharded(&b, 64, 32, ff, fi, f, 1 << 30, nullptr), HS_ERR_SHAPE);   // 1024 % 2048
  EXPECT(hs_topk_sharded(&b, 64, 4, ff, fi, f, 16, nullptr), HS_ERR_WORKSPACE);
  EXPECT(hs_indexer_topk(&b, 64, 128, HS_BF16, f, ff, HS_E4M3, f, ff, fi, nullptr, ff, 64, fi, f,
                         tk - 1, nullptr), HS_ERR_WORKSPACE);
  EXPECT(hs_indexer_topk_select(&b, HS_BF16, 64, ff, fi, f, tk - 1, nullptr), HS_ERR_WORKSPACE);
  hs_batch huge = {65535, 4, 1 << 24, (1 << 24) / 64, ctx};
  EXPECT(hs_indexer_topk_noalloc(&huge, 64, 128, HS_BF16, f, ff, HS_E4M3, f, ff, fi, nullptr, ff,
                                 2048, fi, nullptr), HS_ERR_WORKSPACE);

  // ---- resolve and copies
  hs_residency r;
  std::memset(&r, 0, sizeof r);
  r.C = 128; r.L = 1; r.kv_t = HS_E4M3; r.pool_layer_rows = 1 << 20; r.host_layer_rows = 1 << 20;
  r.bt = fi; r.hot_blocks = fi; r.tok2slot = fi; r.slot2tok = fi; r.stamp = fi; r.step = fi;
  r.err = fi; r.pool = f; r.row_scale = ff; r.host_rows = f; r.host_scale = ff;
  r.host_bt = static_cast<const int64_t*>(f);
  EXPECT(hs_resolve_rows(&b, 256, fi, &r, fi, fi, fi, nullptr, 0, nullptr), HS_ERR_CAPACITY);
  EXPECT(hs_resolve_rows(&b, 64, fi, nullptr, fi, fi, fi, nullptr, 0, nullptr), HS_ERR_NULL);
  hs_residency r2 = r;
  r2.C = 100;
  EXPECT(hs_resolve_tables(&b, 64, fi, &r2, fi, fi, fi, nullptr), HS_ERR_SHAPE);
  r2 = r; r2.L = 17;
  EXPECT(hs_resolve_tables(&b, 64, fi, &r2, fi, fi, fi, nullptr), HS_ERR_SHAPE);
  r2 = r; r2.kv_t = HS_F32;
  EXPECT(hs_resolve_tables(&b, 64, fi, &r2, fi, fi, fi, nullptr), HS_ERR_DTYPE);
  EXPECT(hs_copy_faults(&b, 64, &r, fi, fi, 2000, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_copy_faults_layers(&b, 64, &r, fi, fi, 1, 1, 0, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_copy_faults_layers(&b, 64, &r, fi, fi, 0, 0, 0, nullptr), HS_ERR_SHAPE);
  // selection half + resolve tables: each half's checks
  EXPECT(hs_indexer_topk_select_resolve(&b, HS_BF16, 64, ff, fi, f, tk - 1, &r, fi, fi, fi,
                                        nullptr), HS_ERR_WORKSPACE);
  EXPECT(hs_indexer_topk_select_resolve(&b, HS_BF16, 64, nullptr, fi, f, tk, &r, fi, fi, fi,
                                        nullptr), HS_ERR_NULL);
  EXPECT(hs_indexer_topk_select_resolve(&b, HS_BF16, 64, ff, fi, f, tk, &r, nullptr, fi, fi,
                                        nullptr), HS_ERR_NULL);
  EXPECT(hs_indexer_topk_select_resolve(&b, HS_BF16, 64, ff, fi, f, tk, &r2, fi, fi, fi,
                                        nullptr), HS_ERR_DTYPE);
  EXPECT(hs_indexer_topk_select_resolve(&b, HS_BF16, 256, ff, fi, f, 1 << 30, &r, fi, fi, fi,
                                        nullptr), HS_ERR_CAPACITY);

  // ---- attention
  EXPECT(hs_sparse_mla_decode(&b, 2048, 24, HS_BF16, f, HS_E4M3, f, ff, fi, 0.1f, ff, nullptr,
                              nullptr, 0, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_sparse_mla_decode(&b, 2048, 64, HS_BF16, f, HS_E4M3, f, ff, fi, 0.1f, ff, nullptr,
                              nullptr, 0, nullptr), HS_ERR_WORKSPACE);
  EXPECT(hs_sparse_mla_decode(&b, 0, 16, HS_BF16, f, HS_E4M3, f, ff, fi, 0.1f, ff, nullptr,
                              nullptr, 0, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_sparse_mla_decode_layers(&b, 2048, 16, 17, HS_BF16, f, HS_E4M3, f, 1 << 20, ff, fi,
                                     0.1f, ff, ff, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_sparse_mla_decode_layers(&b, 2048, 16, 2, HS_BF16, f, HS_E4M3, f, 0, ff, fi, 0.1f,
                                     ff, ff, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_sparse_mla_decode_sharded(&b, 2048, 3, 16, HS_BF16, f, HS_E4M3, f, ff, fi, fi, 0.1f,
                                      ff, ff, ff, nullptr, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_sparse_mla_decode_sharded(&b, 2048, 4, 16, HS_BF16, f, HS_E4M3, f, ff, fi, fi, 0.1f,
                                      nullptr, ff, ff, nullptr, f, 1 << 30, nullptr), HS_ERR_NULL);
  EXPECT(hs_sparse_mla_decode_sharded(&b, 2048, 4, 16, HS_F32, f, HS_F32, f, ff, fi, fi, 0.1f,
                                      ff, ff, ff, nullptr, f, 1 << 30, nullptr), HS_ERR_DTYPE);

  // ---- cache operations
  hs_free_list fl = {fi, fi, 0, 0};
  hs_index_cache ic = {HS_E4M3, 128, f, ff, fi};
  EXPECT(hs_append_tokens(&b, fi, fi, &r, f, ff, &ic, f, ff, &fl, &fl, f, 1 << 30, nullptr),
         HS_ERR_SHAPE);
  EXPECT(hs_append_tokens(&b, fi, fi, &r, f, ff, &ic, f, ff, nullptr, &fl, f, 1 << 30, nullptr),
         HS_ERR_NULL);
  EXPECT(hs_precopy_pages(&b, &r, 0, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_precopy_pages(&b, &r, 5000, nullptr), HS_ERR_SHAPE);
  fl.capacity = 8;
  EXPECT(hs_demote_pages(&b, &r, fi, 0, &fl, f, 1 << 30, nullptr), HS_ERR_SHAPE);
  EXPECT(hs_host_device_ptr(nullptr, nullptr), HS_ERR_NULL);

  // ---- workspace sizes at the extremes (no overflow, no trap)
  const int ops[] = {HS_OP_INDEXER, HS_OP_TOPK, HS_OP_RESOLVE, HS_OP_MLA, HS_OP_CACHE};
  for (int op : ops) {
    (void)hs_workspace_bytes(op, 65535, 4, 1 << 24, 8192, 128);
    (void)hs_workspace_bytes(op, 1, 1, 64, 1, 16);
    (void)hs_workspace_bytes(op, 0, 0, 0, 0, 0);
    (void)hs_workspace_bytes(op, -1, -1, -1, -1, -1);
  }
  CHECK(hs_workspace_bytes(HS_OP_TOPK, 65535, 4, 1 << 24, 8192, 16) >
        (size_t)65535 * 4 * (1 << 24) * 8);
  CHECK(hs_mla_layers_workspace_bytes(65535, 4, 8192, 128, 16) > 0);
  CHECK(hs_mla_layers_workspace_bytes(4, 1, 2048, 24, 1) == 0);
  CHECK(hs_mla_sharded_workspace_bytes(65535, 4, 8192, 64, 128) > 0);
  CHECK(hs_mla_sharded_workspace_bytes(4, 1, 2048, 65, 16) == 0);
  CHECK(hs_topk_sharded_workspace_bytes(65535, 1 << 24, 8192, 64) > 0);
  CHECK(hs_topk_sharded_workspace_bytes(4, 1000, 64, 4) == 0);

  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("all checks passed\n");
  return 0;
}
