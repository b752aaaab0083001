// C ABI of the decode step: host-side argument checks, then kernel launches.
// Nothing here allocates, synchronizes, reads device memory or issues a
// memset, so every entry point can be recorded into a HIP graph.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/hs.h"
#include "hs_launch.h"

namespace {

thread_local char g_err[512] = "";

hs_status fail(hs_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hs_status check_batch(const hs_batch* b, hs::BatchDims* d) {
  if (!b) return fail(HS_ERR_NULL, "batch is NULL");
  if (!b->ctx_len) return fail(HS_ERR_NULL, "batch.ctx_len is NULL");
  if (b->B < 1 || b->B > 65535) return fail(HS_ERR_SHAPE, "B=%d out of [1, 65535]", b->B);
  if (b->P < 1 || b->P > 4) return fail(HS_ERR_SHAPE, "P=%d out of [1, 4]", b->P);
  if (b->T_stride < 64 || b->T_stride > (1 << 24) || b->T_stride % 64)
    return fail(HS_ERR_SHAPE, "T_stride=%d must be a multiple of 64 in [64, 2^24]", b->T_stride);
  if (b->max_blocks != b->T_stride / 64)
    return fail(HS_ERR_SHAPE, "max_blocks=%d must equal T_stride/64=%d", b->max_blocks,
                b->T_stride / 64);
  d->B = b->B;
  d->P = b->P;
  d->T_stride = b->T_stride;
  d->max_blocks = b->max_blocks;
  d->ctx_len = b->ctx_len;
  return HS_OK;
}

hs_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(HS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = 0;
  return HS_OK;
}

}  // namespace

namespace {

enum class IdxPath { kBf16E4m3, kE4m3E4m3, kF32 };

hs_status check_indexer(const hs::BatchDims& d, int32_t H_idx, int32_t D_idx, hs_dtype q_t,
                        const void* q_idx, const float* w, hs_dtype k_t, const void* idx_pool,
                        const float* idx_scale, const int32_t* idx_bt, float* scores,
                        IdxPath* path) {
  (void)d;
  if (!q_idx || !w || !idx_pool || !idx_bt || !scores)
    return fail(HS_ERR_NULL, "indexer: q_idx, w, idx_pool, idx_bt and scores are required");
  if (D_idx != 64 && D_idx != 128) return fail(HS_ERR_SHAPE, "D_idx=%d must be 64 or 128", D_idx);
  if (!aligned16(q_idx) || !aligned16(idx_pool) || !aligned16(scores))
    return fail(HS_ERR_ALIGN, "indexer: q_idx, idx_pool and scores need 16-byte alignment");
  if (q_t != HS_F32 && !aligned16(w))
    return fail(HS_ERR_ALIGN, "indexer: w needs 16-byte alignment on the matrix-core paths");
  if (q_t == HS_BF16 && k_t == HS_E4M3) {
    if (H_idx < 16 || H_idx > 64 || H_idx % 16)
      return fail(HS_ERR_SHAPE, "H_idx=%d must be 16, 32, 48 or 64 on the bf16/e4m3 path", H_idx);
    *path = IdxPath::kBf16E4m3;
    return HS_OK;
  }
  if (q_t == HS_E4M3 && k_t == HS_E4M3) {
    if (D_idx != 128) return fail(HS_ERR_SHAPE, "D_idx=%d must be 128 on the e4m3/e4m3 path", D_idx);
    if (H_idx < 16 || H_idx > 64 || H_idx % 16)
      return fail(HS_ERR_SHAPE, "H_idx=%d must be 16, 32, 48 or 64 on the e4m3/e4m3 path", H_idx);
    *path = IdxPath::kE4m3E4m3;
    return HS_OK;
  }
  if (q_t == HS_F32 && k_t == HS_F32) {
    if (H_idx < 1 || H_idx > 64) return fail(HS_ERR_SHAPE, "H_idx=%d out of [1, 64]", H_idx);
    if (idx_scale) return fail(HS_ERR_DTYPE, "fp32 keys take no scale (idx_scale must be NULL)");
    *path = IdxPath::kF32;
    return HS_OK;
  }
  return fail(HS_ERR_DTYPE, "indexer supports (q, k) = (BF16, E4M3), (E4M3, E4M3) or (F32, F32)");
}

hipError_t launch_indexer(const hs::BatchDims& d, IdxPath path, int32_t H_idx, int32_t D_idx,
                          const void* q_idx, const float* w, const void* idx_pool,
                          const float* idx_scale, const int32_t* idx_bt, const float* bias,
                          float* scores, uint32_t* hist, hipStream_t s) {
  if (path == IdxPath::kBf16E4m3)
    return hs::launch_indexer_bf16_e4m3(d, H_idx, D_idx, static_cast<const uint16_t*>(q_idx), w,
                                        static_cast<const uint8_t*>(idx_pool), idx_scale, idx_bt,
                                        bias, scores, hist, s);
  if (path == IdxPath::kE4m3E4m3)
    return hs::launch_indexer_e4m3(d, H_idx, static_cast<const uint8_t*>(q_idx), w,
                                   static_cast<const uint8_t*>(idx_pool), idx_scale, idx_bt,
                                   bias, scores, hist, s);
  return hs::launch_indexer_f32(d, H_idx, D_idx, static_cast<const float*>(q_idx), w,
                                static_cast<const float*>(idx_pool), idx_bt, bias, scores, s);
}

hs_status check_topk(const hs::BatchDims& d, int32_t K, int32_t* topk, void* ws, size_t ws_bytes) {
  if (!topk) return fail(HS_ERR_NULL, "top-K: topk is required");
  if (K < 1 || K > 8192) return fail(HS_ERR_SHAPE, "K=%d out of [1, 8192]", K);
  const size_t need = hs::topk_workspace_bytes(d.B, d.P, d.T_stride, K);
  if (!ws || ws_bytes < need)
    return fail(HS_ERR_WORKSPACE, "top-K needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (!aligned16(ws)) return fail(HS_ERR_ALIGN, "workspace needs 16-byte alignment");
  return HS_OK;
}

// First half of the fused indexer + top-K: the indexer, with the first top-K
// radix pass (every row's histogram) added into the workspace in its
// epilogue.  The histogram and counter area must be zero on entry (the second
// half leaves it so); `clear` zeroes it first with a kernel, for a workspace
// in an unknown state.  The fp32 indexer has no fused histogram.
hipError_t launch_indexer_topk_scores(const hs::BatchDims& d, IdxPath path, int32_t H_idx,
                                      int32_t D_idx, const void* q_idx, const float* w,
                                      const void* idx_pool, const float* idx_scale,
                                      const int32_t* idx_bt, const float* bias, float* scores,
                                      int32_t K, void* ws, bool clear, hipStream_t s) {
  if (path == IdxPath::kF32)
    return launch_indexer(d, path, H_idx, D_idx, q_idx, w, idx_pool, idx_scale, idx_bt, bias,
                          scores, nullptr, s);
  uint32_t* hist = hs::topk_histograms(ws);
  if (clear) {
    hipError_t e = hs::launch_topk_zero(d, K, ws, &hist, s);
    if (e != hipSuccess) return e;
  }
  return launch_indexer(d, path, H_idx, D_idx, q_idx, w, idx_pool, idx_scale, idx_bt, bias,
                        scores, hist, s);
}

// Second half: the rest of the selection (after the fp32 indexer, the whole
// of hs_topk, histogram pass included).  Leaves the histogram and counter
// area zero.
hipError_t launch_indexer_topk_select(const hs::BatchDims& d, bool fused_hist, const float* scores,
                                      int32_t K, int32_t* topk, void* ws, hipStream_t s) {
  if (!fused_hist) return hs::launch_topk(d, K, scores, topk, ws, s);
  return hs::launch_topk_select(d, K, scores, topk, ws, s);
}

hs_status launch_indexer_topk(const hs::BatchDims& d, IdxPath path, int32_t H_idx, int32_t D_idx,
                              const void* q_idx, const float* w, const void* idx_pool,
                              const float* idx_scale, const int32_t* idx_bt, const float* bias,
                              float* scores, int32_t K, int32_t* topk, void* ws, bool clear,
                              hipStream_t s) {
  hipError_t e = launch_indexer_topk_scores(d, path, H_idx, D_idx, q_idx, w, idx_pool, idx_scale,
                                            idx_bt, bias, scores, K, ws, clear, s);
  if (e == hipSuccess)
    e = launch_indexer_topk_select(d, path != IdxPath::kF32, scores, K, topk, ws, s);
  return launched(e, "indexer + top-K");
}

// Scratch of hs_indexer_topk_noalloc, for callers that cannot allocate: one
// copy per GPU, created with the code object and held until the process ends.
// Host code never uses the array's name as an address: static_scratch() looks
// up this device's copy once and every launch takes that pointer.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hs_status static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HS_ERR_HIP, "device %d is beyond the %d the scratch table tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HS_OK;
}

}  // namespace

extern "C" {

hs_status hs_indexer_scores(const hs_batch* batch, int32_t H_idx, int32_t D_idx, hs_dtype q_t,
                            const void* q_idx, const float* w, hs_dtype k_t,
                            const void* idx_pool, const float* idx_scale, const int32_t* idx_bt,
                            const float* bias, float* scores, void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  IdxPath path;
  if (hs_status st = check_indexer(d, H_idx, D_idx, q_t, q_idx, w, k_t, idx_pool, idx_scale,
                                   idx_bt, scores, &path))
    return st;
  return launched(launch_indexer(d, path, H_idx, D_idx, q_idx, w, idx_pool, idx_scale, idx_bt,
                                 bias, scores, nullptr, static_cast<hipStream_t>(stream)),
                  "indexer");
}

hs_status hs_quantize_queries(const hs_batch* batch, int32_t H_idx, int32_t D_idx,
                              const void* q_idx, const float* w, uint8_t* q8, float* w_scaled,
                              void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!q_idx || !w || !q8 || !w_scaled)
    return fail(HS_ERR_NULL, "quantize: q_idx, w, q8 and w_scaled are required");
  if (D_idx != 64 && D_idx != 128) return fail(HS_ERR_SHAPE, "D_idx=%d must be 64 or 128", D_idx);
  if (H_idx < 1 || H_idx > 64) return fail(HS_ERR_SHAPE, "H_idx=%d out of [1, 64]", H_idx);
  if ((reinterpret_cast<uintptr_t>(q_idx) & 3u) || (reinterpret_cast<uintptr_t>(q8) & 1u))
    return fail(HS_ERR_ALIGN, "quantize: q_idx needs 4-byte and q8 2-byte alignment");
  const int rows = d.B * d.P * H_idx;
  return launched(hs::launch_quantize_queries(rows, D_idx, static_cast<const uint16_t*>(q_idx), w,
                                              q8, w_scaled, static_cast<hipStream_t>(stream)),
                  "quantize queries");
}

hs_status hs_indexer_topk(const hs_batch* batch, int32_t H_idx, int32_t D_idx, hs_dtype q_t,
                          const void* q_idx, const float* w, hs_dtype k_t, const void* idx_pool,
                          const float* idx_scale, const int32_t* idx_bt, const float* bias,
                          float* scores, int32_t K, int32_t* topk, void* ws, size_t ws_bytes,
                          void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  IdxPath path;
  if (hs_status st = check_indexer(d, H_idx, D_idx, q_t, q_idx, w, k_t, idx_pool, idx_scale,
                                   idx_bt, scores, &path))
    return st;
  if (hs_status st = check_topk(d, K, topk, ws, ws_bytes)) return st;
  return launch_indexer_topk(d, path, H_idx, D_idx, q_idx, w, idx_pool, idx_scale, idx_bt, bias,
                             scores, K, topk, ws, false, static_cast<hipStream_t>(stream));
}

hs_status hs_indexer_topk_scores(const hs_batch* batch, int32_t H_idx, int32_t D_idx,
                                 hs_dtype q_t, const void* q_idx, const float* w, hs_dtype k_t,
                                 const void* idx_pool, const float* idx_scale,
                                 const int32_t* idx_bt, const float* bias, float* scores,
                                 int32_t K, void* ws, size_t ws_bytes, void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  IdxPath path;
  if (hs_status st = check_indexer(d, H_idx, D_idx, q_t, q_idx, w, k_t, idx_pool, idx_scale,
                                   idx_bt, scores, &path))
    return st;
  int32_t unused_topk = 0;
  if (hs_status st = check_topk(d, K, &unused_topk, ws, ws_bytes)) return st;
  return launched(launch_indexer_topk_scores(d, path, H_idx, D_idx, q_idx, w, idx_pool, idx_scale,
                                             idx_bt, bias, scores, K, ws, false,
                                             static_cast<hipStream_t>(stream)),
                  "indexer (fused top-K histogram)");
}

hs_status hs_indexer_topk_select(const hs_batch* batch, hs_dtype q_t, int32_t K,
                                 const float* scores, int32_t* topk, void* ws, size_t ws_bytes,
                                 void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!scores) return fail(HS_ERR_NULL, "hs_indexer_topk_select: scores is required");
  if (!aligned16(scores))
    return fail(HS_ERR_ALIGN, "hs_indexer_topk_select: scores need 16-byte alignment");
  if (q_t != HS_F32 && q_t != HS_BF16 && q_t != HS_E4M3)
    return fail(HS_ERR_DTYPE, "hs_indexer_topk_select: q_t=%d is not a query type", (int)q_t);
  if (hs_status st = check_topk(d, K, topk, ws, ws_bytes)) return st;
  return launched(launch_indexer_topk_select(d, q_t != HS_F32, scores, K, topk, ws,
                                             static_cast<hipStream_t>(stream)),
                  "top-K selection");
}

hs_status hs_indexer_topk_noalloc(const hs_batch* batch, int32_t H_idx, int32_t D_idx,
                                  hs_dtype q_t, const void* q_idx, const float* w, hs_dtype k_t,
                                  const void* idx_pool, const float* idx_scale,
                                  const int32_t* idx_bt, const float* bias, float* scores,
                                  int32_t K, int32_t* topk, void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  IdxPath path;
  if (hs_status st = check_indexer(d, H_idx, D_idx, q_t, q_idx, w, k_t, idx_pool, idx_scale,
                                   idx_bt, scores, &path))
    return st;
  if (!topk) return fail(HS_ERR_NULL, "top-K: topk is required");
  if (K < 1 || K > 8192) return fail(HS_ERR_SHAPE, "K=%d out of [1, 8192]", K);
  const size_t need = hs::topk_workspace_bytes(d.B, d.P, d.T_stride, K);
  if (need > kStaticScratchBytes)
    return fail(HS_ERR_WORKSPACE,
                "hs_indexer_topk_noalloc: these sizes need %zu bytes of scratch; the library's "
                "static scratch holds %zu (use hs_indexer_topk with a workspace)",
                need, kStaticScratchBytes);
  void* ws = nullptr;
  if (hs_status st = static_scratch(&ws)) return st;
  return launch_indexer_topk(d, path, H_idx, D_idx, q_idx, w, idx_pool, idx_scale, idx_bt, bias,
                             scores, K, topk, ws, true, static_cast<hipStream_t>(stream));
}

size_t hs_topk_sharded_workspace_bytes(int32_t B, int32_t T_stride, int32_t K, int32_t S) {
  if (B < 1 || K < 1 || S < 1 || S > 64 || T_stride < 64 * S || T_stride % (64 * S)) return 0;
  return hs::topk_sharded_workspace_bytes(B, T_stride, K, S);
}

hs_status hs_topk_sharded(const hs_batch* batch, int32_t K, int32_t S, const float* scores,
                          int32_t* topk, void* ws, size_t ws_bytes, void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!scores || !topk) return fail(HS_ERR_NULL, "hs_topk_sharded: scores and topk are required");
  if (d.P != 1) return fail(HS_ERR_SHAPE, "hs_topk_sharded: one query position (P=%d)", d.P);
  if (K < 1 || K > 8192) return fail(HS_ERR_SHAPE, "K=%d out of [1, 8192]", K);
  if (S < 1 || S > 64 || d.T_stride % (64 * S))
    return fail(HS_ERR_SHAPE, "S=%d must be in [1, 64] and T_stride=%d a multiple of 64*S", S,
                d.T_stride);
  if (!aligned16(scores)) return fail(HS_ERR_ALIGN, "hs_topk_sharded: scores need 16-byte alignment");
  const size_t need = hs::topk_sharded_workspace_bytes(d.B, d.T_stride, K, S);
  if (!ws || ws_bytes < need)
    return fail(HS_ERR_WORKSPACE, "sharded top-K needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (!aligned16(ws)) return fail(HS_ERR_ALIGN, "workspace needs 16-byte alignment");
  return launched(hs::launch_topk_sharded(d, K, S, scores, topk, ws, static_cast<hipStream_t>(stream)),
                  "sharded top-K");
}

hs_status hs_topk(const hs_batch* batch, int32_t K, const float* scores, int32_t* topk, void* ws,
                  size_t ws_bytes, void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!scores) return fail(HS_ERR_NULL, "hs_topk: scores is required");
  if (!aligned16(scores)) return fail(HS_ERR_ALIGN, "hs_topk: scores need 16-byte alignment");
  if (hs_status st = check_topk(d, K, topk, ws, ws_bytes)) return st;
  return launched(hs::launch_topk(d, K, scores, topk, ws, static_cast<hipStream_t>(stream)), "topk");
}

}  // extern "C"

namespace {

hs_status check_residency(const hs::BatchDims& d, int32_t K, const hs_residency* res,
                          hs::ResidencyArgs* r) {
  if (!res) return fail(HS_ERR_NULL, "residency is NULL");
  if (K < 1 || d.P * K > 8192) return fail(HS_ERR_SHAPE, "P*K=%d out of [1, 8192]", d.P * K);
  if (!res->bt || !res->step || !res->err || !res->pool)
    return fail(HS_ERR_NULL, "residency: bt, step, err and pool are required");
  if (res->L < 1 || res->L > 16) return fail(HS_ERR_SHAPE, "L=%d out of [1, 16]", res->L);
  if (res->C < 0 || res->C % 64 || res->C > 16384)
    return fail(HS_ERR_SHAPE, "C=%d must be a multiple of 64 in [0, 16384] (0 = no hot buffers)",
                res->C);
  if (res->C > 0 && res->C < d.P * K)
    return fail(HS_ERR_CAPACITY, "C=%d below P*K=%d: a step's faults could exceed its victims",
                res->C, d.P * K);
  if (res->C > 0 && (!res->hot_blocks || !res->tok2slot || !res->slot2tok || !res->stamp))
    return fail(HS_ERR_NULL, "residency: hot_blocks, tok2slot, slot2tok and stamp are required when C > 0");
  int kv_bytes;
  if (res->kv_t == HS_E4M3) {
    kv_bytes = 1;
    if (!res->row_scale) return fail(HS_ERR_NULL, "E4M3 rows need row_scale");
    if (res->host_rows && !res->host_scale) return fail(HS_ERR_NULL, "E4M3 host rows need host_scale");
  } else if (res->kv_t == HS_F32) {
    kv_bytes = 4;
    if (res->row_scale || res->host_scale) return fail(HS_ERR_DTYPE, "F32 rows take no scales");
  } else {
    return fail(HS_ERR_DTYPE, "residency kv_t must be E4M3 or F32");
  }
  if (res->host_rows && !res->host_bt) return fail(HS_ERR_NULL, "host_rows given without host_bt");
  if (res->C > 0 && res->host_bt && !res->host_rows)
    return fail(HS_ERR_NULL, "host_bt given without host_rows");
  if (!aligned16(res->pool) || (res->host_rows && !aligned16(res->host_rows)))
    return fail(HS_ERR_ALIGN, "pool and host_rows need 16-byte alignment");
  if (res->pool_layer_rows < 0 || res->host_layer_rows < 0)
    return fail(HS_ERR_SHAPE, "layer strides must be non-negative");
  if (res->host_row_pitch < 0)
    return fail(HS_ERR_SHAPE, "host_row_pitch=%d must be non-negative", res->host_row_pitch);
  r->C = res->C;
  r->L = res->L;
  r->kv_bytes = kv_bytes;
  r->pool_layer_rows = res->pool_layer_rows;
  r->host_layer_rows = res->host_layer_rows;
  r->host_row_pitch = res->host_row_pitch > 1 ? res->host_row_pitch : 1;
  r->bt = res->bt;
  r->hot_blocks = res->hot_blocks;
  r->tok2slot = res->tok2slot;
  r->slot2tok = res->slot2tok;
  r->stamp = res->stamp;
  r->step = res->step;
  r->err = res->err;
  r->pool = res->pool;
  r->row_scale = res->row_scale;
  r->host_rows = res->host_rows;
  r->host_scale = res->host_scale;
  r->host_bt = res->host_bt;
  return HS_OK;
}

}  // namespace

extern "C" {

hs_status hs_resolve_tables(const hs_batch* batch, int32_t K, const int32_t* topk,
                            const hs_residency* res, int32_t* row_ids, int32_t* faults,
                            int32_t* counts, void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!topk || !row_ids || !faults || !counts)
    return fail(HS_ERR_NULL, "resolve: topk, row_ids, faults and counts are required");
  hs::ResidencyArgs r;
  if (hs_status st = check_residency(d, K, res, &r)) return st;
  return launched(hs::launch_resolve_tables(d, K, topk, r, row_ids, faults, counts,
                                            static_cast<hipStream_t>(stream)),
                  "resolve");
}

hs_status hs_indexer_topk_select_resolve(const hs_batch* batch, hs_dtype q_t, int32_t K,
                                         const float* scores, int32_t* topk, void* ws,
                                         size_t ws_bytes, const hs_residency* res,
                                         int32_t* row_ids, int32_t* faults, int32_t* counts,
                                         void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!scores) return fail(HS_ERR_NULL, "hs_indexer_topk_select_resolve: scores is required");
  if (!aligned16(scores))
    return fail(HS_ERR_ALIGN, "hs_indexer_topk_select_resolve: scores need 16-byte alignment");
  if (q_t != HS_F32 && q_t != HS_BF16 && q_t != HS_E4M3)
    return fail(HS_ERR_DTYPE, "hs_indexer_topk_select_resolve: q_t=%d is not a query type",
                (int)q_t);
  if (hs_status st = check_topk(d, K, topk, ws, ws_bytes)) return st;
  if (!row_ids || !faults || !counts)
    return fail(HS_ERR_NULL,
                "hs_indexer_topk_select_resolve: row_ids, faults and counts are required");
  hs::ResidencyArgs r;
  if (hs_status st = check_residency(d, K, res, &r)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_t == HS_F32) {
    // no histogram from the indexer: the whole selection, then the tables
    hipError_t e = hs::launch_topk(d, K, scores, topk, ws, s);
    if (e == hipSuccess) e = hs::launch_resolve_tables(d, K, topk, r, row_ids, faults, counts, s);
    return launched(e, "top-K + resolve");
  }
  hipError_t e = hs::launch_topk_filter(d, K, scores, ws, s);
  if (e == hipSuccess)
    e = hs::launch_finalize_resolve(d, K, topk, ws, r, row_ids, faults, counts, s);
  return launched(e, "top-K + resolve");
}

hs_status hs_copy_faults_layers(const hs_batch* batch, int32_t K, const hs_residency* res,
                                const int32_t* faults, const int32_t* counts, int32_t layer0,
                                int32_t n_layers, int32_t workgroups, void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!faults || !counts) return fail(HS_ERR_NULL, "hs_copy_faults: faults and counts are required");
  if (workgroups < 0 || workgroups > 1024)
    return fail(HS_ERR_SHAPE, "hs_copy_faults: workgroups=%d out of [0, 1024]", workgroups);
  hs::ResidencyArgs r;
  if (hs_status st = check_residency(d, K, res, &r)) return st;
  if (layer0 < 0 || n_layers < 1 || layer0 + n_layers > r.L)
    return fail(HS_ERR_SHAPE, "hs_copy_faults_layers: layers [%d, %d) outside [0, L=%d)", layer0,
                layer0 + n_layers, r.L);
  return launched(hs::launch_fault_copy(d, K, r, faults, counts, layer0, n_layers, workgroups,
                                        static_cast<hipStream_t>(stream)),
                  "fault copy");
}

hs_status hs_copy_faults(const hs_batch* batch, int32_t K, const hs_residency* res,
                         const int32_t* faults, const int32_t* counts, int32_t workgroups,
                         void* stream) {
  const int32_t L = res ? res->L : 1;
  return hs_copy_faults_layers(batch, K, res, faults, counts, 0, L, workgroups, stream);
}

hs_status hs_resolve_rows(const hs_batch* batch, int32_t K, const int32_t* topk,
                          const hs_residency* res, int32_t* row_ids, int32_t* faults,
                          int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (hs_status st = hs_resolve_tables(batch, K, topk, res, row_ids, faults, counts, stream))
    return st;
  return hs_copy_faults(batch, K, res, faults, counts, 0, stream);
}

}  // extern "C"

namespace {

hs_status sparse_mla(const char* name, const hs_batch* batch, int32_t K, int32_t Hq, int32_t L,
                     hs_dtype q_t, const void* q, hs_dtype kv_t, const void* pool,
                     int64_t pool_layer_rows, const float* row_scale, const int32_t* row_ids,
                     float sm_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                     void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!q || !pool || !row_ids || !out)
    return fail(HS_ERR_NULL, "%s: q, pool, row_ids and out are required", name);
  if (K < 1 || K > 8192) return fail(HS_ERR_SHAPE, "K=%d out of [1, 8192]", K);
  if (Hq < 16 || Hq > 128 || Hq % 16)
    return fail(HS_ERR_SHAPE, "Hq=%d must be a multiple of 16 in [16, 128]", Hq);
  if (L < 1 || L > 16) return fail(HS_ERR_SHAPE, "L=%d out of [1, 16]", L);
  if (L > 1 && pool_layer_rows < 1)
    return fail(HS_ERR_SHAPE, "pool_layer_rows=%lld must be positive for L > 1",
                (long long)pool_layer_rows);
  if (!aligned16(q) || !aligned16(pool) || !aligned16(out))
    return fail(HS_ERR_ALIGN, "q, pool and out need 16-byte alignment");
  const size_t need = hs::mla_workspace_bytes(d.B, d.P, K, Hq, L);
  if (need && (!ws || ws_bytes < need))
    return fail(HS_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu", name, need, ws_bytes);
  if (need && !aligned16(ws)) return fail(HS_ERR_ALIGN, "workspace needs 16-byte alignment");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_t == HS_BF16 && kv_t == HS_E4M3) {
    if (!row_scale) return fail(HS_ERR_NULL, "E4M3 rows need row_scale");
    return launched(hs::launch_mla_bf16_e4m3(d, K, L, Hq, pool_layer_rows,
                                             static_cast<const uint16_t*>(q),
                                             static_cast<const uint8_t*>(pool), row_scale, row_ids,
                                             sm_scale, out, lse, ws, s),
                    name);
  }
  if (q_t == HS_F32 && kv_t == HS_F32) {
    if (row_scale) return fail(HS_ERR_DTYPE, "F32 rows take no row_scale");
    return launched(hs::launch_mla_f32(d, K, L, Hq, pool_layer_rows, static_cast<const float*>(q),
                                       static_cast<const float*>(pool), row_ids, sm_scale, out,
                                       lse, ws, s),
                    name);
  }
  return fail(HS_ERR_DTYPE, "sparse MLA supports (q, kv) = (BF16, E4M3) or (F32, F32)");
}

}  // namespace

extern "C" {

hs_status hs_sparse_mla_decode(const hs_batch* batch, int32_t K, int32_t Hq, hs_dtype q_t,
                               const void* q, hs_dtype kv_t, const void* pool,
                               const float* row_scale, const int32_t* row_ids, float sm_scale,
                               float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return sparse_mla("hs_sparse_mla_decode", batch, K, Hq, 1, q_t, q, kv_t, pool, 0, row_scale,
                    row_ids, sm_scale, out, lse, ws, ws_bytes, stream);
}

hs_status hs_sparse_mla_decode_layers(const hs_batch* batch, int32_t K, int32_t Hq, int32_t L,
                                      hs_dtype q_t, const void* q, hs_dtype kv_t,
                                      const void* pool, int64_t pool_layer_rows,
                                      const float* row_scale, const int32_t* row_ids,
                                      float sm_scale, float* out, float* lse, void* ws,
                                      size_t ws_bytes, void* stream) {
  return sparse_mla("hs_sparse_mla_decode_layers", batch, K, Hq, L, q_t, q, kv_t, pool,
                    pool_layer_rows, row_scale, row_ids, sm_scale, out, lse, ws, ws_bytes, stream);
}

size_t hs_mla_layers_workspace_bytes(int32_t B, int32_t P, int32_t K, int32_t Hq, int32_t L) {
  if (B < 1 || P < 1 || K < 1 || L < 1 || Hq < 16 || Hq % 16) return 0;
  return hs::mla_workspace_bytes(B, P, K, Hq, L);
}

size_t hs_mla_sharded_workspace_bytes(int32_t B, int32_t P, int32_t K, int32_t S, int32_t Hq) {
  if (B < 1 || P < 1 || K < 1 || K > 8192 || S < 1 || S > 64 || Hq < 16 || Hq > 128 || Hq % 16)
    return 0;
  return hs::mla_sharded_workspace_bytes(B, P, K, S, Hq);
}

hs_status hs_sparse_mla_decode_sharded(const hs_batch* batch, int32_t K, int32_t S, int32_t Hq,
                                       hs_dtype q_t, const void* q, hs_dtype kv_t,
                                       const void* pool, const float* row_scale,
                                       const int32_t* topk, const int32_t* row_ids,
                                       float sm_scale, float* shard_out, float* shard_lse,
                                       float* out, float* lse, void* ws, size_t ws_bytes,
                                       void* stream) {
  const char* name = "hs_sparse_mla_decode_sharded";
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!q || !pool || !topk || !row_ids || !shard_out || !shard_lse || !out)
    return fail(HS_ERR_NULL, "%s: q, pool, topk, row_ids, shard_out, shard_lse and out are required",
                name);
  if (K < 1 || K > 8192) return fail(HS_ERR_SHAPE, "K=%d out of [1, 8192]", K);
  if (S < 1 || S > 64 || d.T_stride % S)
    return fail(HS_ERR_SHAPE, "S=%d must be in [1, 64] and divide T_stride=%d", S, d.T_stride);
  if (Hq < 16 || Hq > 128 || Hq % 16)
    return fail(HS_ERR_SHAPE, "Hq=%d must be a multiple of 16 in [16, 128]", Hq);
  if (!aligned16(q) || !aligned16(pool) || !aligned16(out) || !aligned16(shard_out))
    return fail(HS_ERR_ALIGN, "q, pool, shard_out and out need 16-byte alignment");
  const size_t need = hs::mla_sharded_workspace_bytes(d.B, d.P, K, S, Hq);
  if (!ws || ws_bytes < need)
    return fail(HS_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu", name, need, ws_bytes);
  if (!aligned16(ws)) return fail(HS_ERR_ALIGN, "workspace needs 16-byte alignment");
  bool f32;
  if (q_t == HS_BF16 && kv_t == HS_E4M3) {
    if (!row_scale) return fail(HS_ERR_NULL, "E4M3 rows need row_scale");
    f32 = false;
  } else if (q_t == HS_F32 && kv_t == HS_F32) {
    if (row_scale) return fail(HS_ERR_DTYPE, "F32 rows take no row_scale");
    f32 = true;
  } else {
    return fail(HS_ERR_DTYPE, "sparse MLA supports (q, kv) = (BF16, E4M3) or (F32, F32)");
  }
  return launched(hs::launch_mla_sharded(d, K, S, Hq, f32, q, pool, row_scale, topk, row_ids,
                                         sm_scale, shard_out, shard_lse, out, lse, ws,
                                         static_cast<hipStream_t>(stream)),
                  name);
}

size_t hs_workspace_bytes(int32_t op, int32_t B, int32_t P, int32_t T_stride, int32_t K,
                          int32_t Hq) {
  if (op == HS_OP_CACHE) return B < 1 ? 0 : hs::cache_workspace_bytes(B);
  if (B < 1 || P < 1 || K < 1) return 0;
  switch (op) {
    case HS_OP_TOPK: return hs::topk_workspace_bytes(B, P, T_stride, K);
    case HS_OP_MLA: return hs::mla_workspace_bytes(B, P, K, Hq, 1);
    default: return 0;
  }
}

static_assert(HS_DEVERR_APPEND_RANGE == hs::kDevErrAppendRange &&
                  HS_DEVERR_APPEND_NO_BLOCK == hs::kDevErrAppendNoBlock &&
                  HS_DEVERR_DEMOTE_FULL == hs::kDevErrDemoteFull,
              "device error bits");

}  // extern "C"

namespace {

hs_status check_free_list(const hs_free_list* f, const char* what, hs::FreeListArgs* out) {
  if (!f || !f->blocks || !f->count) return fail(HS_ERR_NULL, "%s free list is incomplete", what);
  if (f->capacity < 1) return fail(HS_ERR_SHAPE, "%s free list capacity=%d", what, f->capacity);
  out->blocks = f->blocks;
  out->count = f->count;
  out->capacity = f->capacity;
  return HS_OK;
}

hs_status check_cache_ws(const hs::BatchDims& d, void* ws, size_t ws_bytes) {
  const size_t need = hs::cache_workspace_bytes(d.B);
  if (!ws || ws_bytes < need)
    return fail(HS_ERR_WORKSPACE, "cache operations need %zu workspace bytes, got %zu", need,
                ws_bytes);
  if (!aligned16(ws)) return fail(HS_ERR_ALIGN, "workspace needs 16-byte alignment");
  return HS_OK;
}

}  // namespace

extern "C" {

hs_status hs_append_tokens(const hs_batch* batch, int32_t* ctx_len, const int32_t* n_new,
                           const hs_residency* res, const void* new_rows,
                           const float* new_row_scale, const hs_index_cache* idx,
                           const void* new_keys, const float* new_key_scale,
                           const hs_free_list* latent_free, const hs_free_list* idx_free,
                           void* ws, size_t ws_bytes, void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!ctx_len || ctx_len != batch->ctx_len)
    return fail(HS_ERR_SHAPE, "hs_append_tokens: ctx_len must be batch->ctx_len");
  if (!n_new || !new_rows || !idx || !new_keys)
    return fail(HS_ERR_NULL, "hs_append_tokens: n_new, new_rows, idx and new_keys are required");
  hs::ResidencyArgs r;
  if (hs_status st = check_residency(d, 1, res, &r)) return st;
  if (res->kv_t == HS_E4M3 && !new_row_scale)
    return fail(HS_ERR_NULL, "E4M3 rows need new_row_scale");
  if (res->kv_t == HS_F32 && new_row_scale)
    return fail(HS_ERR_DTYPE, "F32 rows take no new_row_scale");
  if (!idx->pool || !idx->bt) return fail(HS_ERR_NULL, "indexer cache: pool and bt are required");
  if (idx->D_idx != 64 && idx->D_idx != 128)
    return fail(HS_ERR_SHAPE, "D_idx=%d must be 64 or 128", idx->D_idx);
  int key_bytes;
  if (idx->k_t == HS_E4M3) {
    key_bytes = idx->D_idx;
    if (!idx->scale || !new_key_scale)
      return fail(HS_ERR_NULL, "E4M3 keys need the block scales and new_key_scale");
  } else if (idx->k_t == HS_F32) {
    key_bytes = 4 * idx->D_idx;
    if (idx->scale || new_key_scale) return fail(HS_ERR_DTYPE, "F32 keys take no scales");
  } else {
    return fail(HS_ERR_DTYPE, "indexer keys must be E4M3 or F32");
  }
  if (!aligned16(new_rows) || !aligned16(new_keys) || !aligned16(idx->pool))
    return fail(HS_ERR_ALIGN, "new_rows, new_keys and the indexer pool need 16-byte alignment");
  hs::FreeListArgs lf, fi;
  if (hs_status st = check_free_list(latent_free, "latent", &lf)) return st;
  if (hs_status st = check_free_list(idx_free, "indexer", &fi)) return st;
  if (hs_status st = check_cache_ws(d, ws, ws_bytes)) return st;
  return launched(hs::launch_append_tokens(d, ctx_len, n_new, r, new_rows, new_row_scale,
                                           key_bytes, idx->pool, idx->scale, idx->bt, new_keys,
                                           new_key_scale, lf, fi, ws,
                                           static_cast<hipStream_t>(stream)),
                  "append");
}

hs_status hs_precopy_pages(const hs_batch* batch, const hs_residency* res, int32_t max_pages,
                           void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  hs::ResidencyArgs r;
  if (hs_status st = check_residency(d, 1, res, &r)) return st;
  if (!res->host_rows || !res->host_bt || (res->kv_t == HS_E4M3 && !res->host_scale))
    return fail(HS_ERR_NULL, "pre-copy needs host_rows, host_bt (and host_scale for E4M3)");
  if (max_pages < 1 || max_pages > hs::precopy_max_pages())
    return fail(HS_ERR_SHAPE, "max_pages=%d out of [1, %d]", max_pages, hs::precopy_max_pages());
  // host slot of page j of request b: tokens b*T_stride + 64j ..; the layers'
  // rows must not overlap: planes of B*T_stride tokens, or the L rows of a
  // token inside its pitch
  const int64_t n_tok = (int64_t)d.B * d.T_stride;
  if (res->L > 1 && r.host_layer_rows < n_tok * r.host_row_pitch &&
      (r.host_layer_rows < 1 || r.host_row_pitch < (int64_t)res->L * r.host_layer_rows))
    return fail(HS_ERR_SHAPE,
                "host pool of B*T_stride=%lld tokens: layers overlap (host_layer_rows=%lld, "
                "host_row_pitch=%lld; need host_layer_rows >= B*T_stride*pitch or pitch >= "
                "L*host_layer_rows)",
                (long long)n_tok, (long long)r.host_layer_rows, (long long)r.host_row_pitch);
  return launched(hs::launch_precopy_pages(d, r, max_pages, static_cast<hipStream_t>(stream)),
                  "pre-copy");
}

hs_status hs_demote_pages(const hs_batch* batch, const hs_residency* res,
                          const int32_t* n_demote, int32_t tail_pages,
                          const hs_free_list* latent_free, void* ws, size_t ws_bytes,
                          void* stream) {
  hs::BatchDims d;
  if (hs_status st = check_batch(batch, &d)) return st;
  if (!n_demote) return fail(HS_ERR_NULL, "hs_demote_pages: n_demote is required");
  hs::ResidencyArgs r;
  if (hs_status st = check_residency(d, 1, res, &r)) return st;
  if (!res->host_bt) return fail(HS_ERR_NULL, "demotion needs host_bt");
  if (tail_pages < 1 || tail_pages > d.max_blocks)
    return fail(HS_ERR_SHAPE, "tail_pages=%d out of [1, %d]", tail_pages, d.max_blocks);
  hs::FreeListArgs lf;
  if (hs_status st = check_free_list(latent_free, "latent", &lf)) return st;
  if (hs_status st = check_cache_ws(d, ws, ws_bytes)) return st;
  return launched(hs::launch_demote_pages(d, r, n_demote, tail_pages, lf, ws,
                                          static_cast<hipStream_t>(stream)),
                  "demotion");
}

hs_status hs_host_device_ptr(const void* pinned_host, const void** dev_ptr) {
  if (!pinned_host || !dev_ptr) return fail(HS_ERR_NULL, "hs_host_device_ptr: NULL argument");
  void* dp = nullptr;
  hipError_t e = hipHostGetDevicePointer(&dp, const_cast<void*>(pinned_host), 0);
  if (e != hipSuccess) return fail(HS_ERR_HIP, "hipHostGetDevicePointer: %s", hipGetErrorString(e));
  *dev_ptr = dp;
  g_err[0] = 0;
  return HS_OK;
}

const char* hs_last_error(void) { return g_err; }

int32_t hs_abi_version(void) { return HS_ABI_VERSION; }

}  // extern "C"
