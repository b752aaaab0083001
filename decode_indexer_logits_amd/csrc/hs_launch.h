// Internal launchers of the decode-step kernels (host side).  Argument checks
// happen in hs_api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hs {

struct BatchDims {
  int B, P, T_stride, max_blocks;
  const int32_t* ctx_len;
};

// Indexer: bf16 queries x E4M3 keys on the matrix cores.  With `hist`, the
// 11-bit score-key histogram of every (request, position) is added to it.
hipError_t launch_indexer_bf16_e4m3(const BatchDims& d, int H, int DK, const uint16_t* q,
                                   const float* w, const uint8_t* pool, const float* scale,
                                   const int32_t* bt, const float* bias, float* scores,
                                   uint32_t* hist, hipStream_t s);
// Indexer: E4M3 queries x E4M3 keys (D = 128) on the fp8 matrix cores.
hipError_t launch_indexer_e4m3(const BatchDims& d, int H, const uint8_t* q8, const float* w,
                               const uint8_t* pool, const float* scale, const int32_t* bt,
                               const float* bias, float* scores, uint32_t* hist, hipStream_t s);
// Per-head E4M3 quantization of `rows` bf16 query vectors of DK (64 or 128).
hipError_t launch_quantize_queries(int rows, int DK, const uint16_t* q, const float* w,
                                   uint8_t* q8, float* w_scaled, hipStream_t s);
// Indexer: fp32 queries x fp32 keys on the vector ALUs.
hipError_t launch_indexer_f32(const BatchDims& d, int H, int DK, const float* q, const float* w,
                              const float* pool, const int32_t* bt, const float* bias,
                              float* scores, hipStream_t s);

size_t topk_workspace_bytes(int B, int P, int T_stride, int K);
hipError_t launch_topk(const BatchDims& d, int K, const float* scores, int32_t* topk, void* ws,
                       hipStream_t s);
size_t topk_sharded_workspace_bytes(int B, int T_stride, int K, int S);
hipError_t launch_topk_sharded(const BatchDims& d, int K, int S, const float* scores,
                               int32_t* topk, void* ws, hipStream_t s);
// The pieces of the fused indexer + top-K: the histogram area the indexer
// fills (at the start of the workspace), a kernel that zeroes it with the
// counters (the selection leaves both zero, so only a workspace in an unknown
// state needs it), and the selection from that histogram.
uint32_t* topk_histograms(void* ws);
hipError_t launch_topk_zero(const BatchDims& d, int K, void* ws, uint32_t** hist, hipStream_t s);
hipError_t launch_topk_select(const BatchDims& d, int K, const float* scores, int32_t* topk,
                              void* ws, hipStream_t s);
// The histogram pass of hs_topk alone, into a workspace whose histograms and
// counters are zero (a selection leaves them so).
hipError_t launch_topk_hist(const BatchDims& d, int K, const float* scores, void* ws,
                            hipStream_t s);
// The filter pass of the selection alone (the finalize then runs on its own or
// fused with the resolve tables).
hipError_t launch_topk_filter(const BatchDims& d, int K, const float* scores, void* ws,
                              hipStream_t s);

struct ResidencyArgs {
  int C, L, kv_bytes;               // kv_bytes: bytes per latent element (1 or 4)
  int64_t pool_layer_rows, host_layer_rows;
  int64_t host_row_pitch;           // rows from one host token to the next (>= 1)
  const int32_t* bt;
  const int32_t* hot_blocks;
  int32_t* tok2slot;
  int32_t* slot2tok;
  int32_t* stamp;
  int32_t* step;
  int32_t* err;
  void* pool;
  float* row_scale;
  const void* host_rows;
  const float* host_scale;
  const int64_t* host_bt;
};
hipError_t launch_resolve_tables(const BatchDims& d, int K, const int32_t* topk,
                                 const ResidencyArgs& r, int32_t* row_ids, int32_t* faults,
                                 int32_t* counts, hipStream_t s);
// The top-K finalize followed by the resolve tables, after the filter pass
// (launch_topk_filter) on a workspace laid out as topk_workspace_bytes says:
// one kernel for one query position, the two launches otherwise.
hipError_t launch_finalize_resolve(const BatchDims& d, int K, int32_t* topk, void* topk_ws,
                                   const ResidencyArgs& r, int32_t* row_ids, int32_t* faults,
                                   int32_t* counts, hipStream_t s);
hipError_t launch_topk_finalize(const BatchDims& d, int K, int32_t* topk, void* ws,
                                hipStream_t s);
// Layers l0 .. l0 + nl - 1 of every fault (the call with l0 + nl == L advances
// the step); workgroups = 0: the default grid (every CU)
hipError_t launch_fault_copy(const BatchDims& d, int K, const ResidencyArgs& r,
                             const int32_t* faults, const int32_t* counts, int l0, int nl,
                             int workgroups, hipStream_t s);

// Device error bits of the cache operations (the HS_DEVERR_* values of hs.h).
constexpr int kDevErrAppendRange = 4;
constexpr int kDevErrAppendNoBlock = 8;
constexpr int kDevErrDemoteFull = 16;
struct FreeListArgs {
  int32_t* blocks;
  int32_t* count;
  int capacity;
};
size_t cache_workspace_bytes(int B);
int precopy_max_pages();
hipError_t launch_append_tokens(const BatchDims& d, int32_t* ctx_len, const int32_t* n_new,
                                const ResidencyArgs& r, const void* new_rows,
                                const float* new_row_scale, int key_bytes, void* idx_pool,
                                float* idx_scale, int32_t* idx_bt, const void* new_keys,
                                const float* new_key_scale, const FreeListArgs& lat,
                                const FreeListArgs& idx, void* ws, hipStream_t s);
hipError_t launch_precopy_pages(const BatchDims& d, const ResidencyArgs& r, int max_pages,
                                hipStream_t s);
hipError_t launch_demote_pages(const BatchDims& d, const ResidencyArgs& r,
                               const int32_t* n_demote, int tail_pages,
                               const FreeListArgs& lat, void* ws, hipStream_t s);
// Sparse MLA over L layers that share the row ids: queries [L, B, P, Hq, 576],
// layer l's pool rows at l * pool_layer_rows, outputs [L, B, P, Hq, 512];
// Hq a multiple of 16 (G = Hq / 16 head groups).
int mla_num_splits(int B, int P, int K, int L, int G);
size_t mla_workspace_bytes(int B, int P, int K, int Hq, int L);
hipError_t launch_mla_bf16_e4m3(const BatchDims& d, int K, int L, int Hq, int64_t pool_layer_rows,
                                const uint16_t* q, const uint8_t* pool, const float* row_scale,
                                const int32_t* row_ids, float sm_scale, float* out, float* lse,
                                void* ws, hipStream_t s);
hipError_t launch_mla_f32(const BatchDims& d, int K, int L, int Hq, int64_t pool_layer_rows,
                          const float* q, const float* pool, const int32_t* row_ids,
                          float sm_scale, float* out, float* lse, void* ws, hipStream_t s);
// Token-sharded attention: S shards of T_stride / S tokens; per-shard outputs
// [B, P, S, Hq, 512] and log-sum-exp [B, P, S, Hq], merged into out / lse.
size_t mla_sharded_workspace_bytes(int B, int P, int K, int S, int Hq);
hipError_t launch_mla_sharded(const BatchDims& d, int K, int S, int Hq, bool f32, const void* q,
                              const void* pool, const float* row_scale, const int32_t* topk,
                              const int32_t* row_ids, float sm_scale, float* shard_out,
                              float* shard_lse, float* out, float* lse, void* ws, hipStream_t s);

}  // namespace hs
