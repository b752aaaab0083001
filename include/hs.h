/*
 * hs.h -- C ABI of one decode step of indexer-driven sparse MLA attention with
 * hybrid GPU/host KV residency, for AMD Instinct MI355X (gfx950).
 *
 * The step (page "Un contexte d'un million sur huit H200", sections "Ce qui se
 * passe" and "Les trois états de résidence"):
 *
 *   hs_indexer_scores    the indexer scores every cached token of every request
 *   hs_topk              the K best tokens of each query position are selected
 *   hs_resolve_rows      the fused resolve maps each selected token to a pool row:
 *                        resident page in place / hot slot with an LRU refresh /
 *                        single-row fault copied from pinned host memory
 *   hs_sparse_mla_decode sparse MLA attention over the selected latent rows
 *                        (hs_sparse_mla_decode_layers: several layers, one launch)
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise; host
 *     pools are pinned host memory passed by their device-accessible address
 *     (see hs_host_device_ptr).  The caller owns every buffer, including the
 *     workspace; the library allocates nothing and keeps no state between calls
 *     except the thread-local error message, a per-device memo of how many
 *     workgroups of each multi-position indexer kernel fit the GPU at once
 *     (from the runtime's occupancy query; it sizes their tiles and changes no
 *     result), and the static workspace of hs_indexer_topk_noalloc.
 *   - Every call only enqueues kernels on `stream` (a hipStream_t; NULL = the
 *     default stream).  No call synchronizes, reads device memory on the host,
 *     allocates, or issues a memset, so a whole step can be captured in a HIP
 *     graph: nothing on the decode path waits for a CPU decision, as the page
 *     above requires of the fused resolve.
 *   - Arguments are validated on the host only (null pointers, shapes, types,
 *     alignment, capacity).  A failed check returns a nonzero hs_status, enqueues
 *     nothing and sets the message returned by hs_last_error().  Device contents
 *     (block tables, lengths, token ids) are trusted; the resolve step reports
 *     inconsistent residency tables through its device error word.
 *   - Layouts are dense row-major; the block (page) size is 64 tokens.
 */
#ifndef HS_H
#define HS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HS_ABI_VERSION 1
#define HS_BLOCK 64        /* tokens per page of every paged cache          */
#define HS_D_LATENT 576    /* latent row: 512 compressed + 64 rotary values  */
#define HS_D_VALUE 512     /* value part of a latent row                     */

typedef int32_t hs_status;
enum {
  HS_OK = 0,
  HS_ERR_NULL = 1,       /* a required pointer is NULL                      */
  HS_ERR_SHAPE = 2,      /* a size is out of the supported range            */
  HS_ERR_DTYPE = 3,      /* unsupported element-type combination            */
  HS_ERR_CAPACITY = 4,   /* hot capacity below P*K                          */
  HS_ERR_WORKSPACE = 5,  /* workspace missing or smaller than required      */
  HS_ERR_ALIGN = 6,      /* a pointer is not 16-byte aligned                */
  HS_ERR_HIP = 7         /* the HIP runtime rejected a launch               */
};

typedef enum {
  HS_F32 = 0,    /* IEEE binary32                                          */
  HS_BF16 = 1,   /* bfloat16                                               */
  HS_E4M3 = 2    /* OCP FP8 E4M3FN code (bias 7, no infinity, max 448)     */
} hs_dtype;

/* Error bits the resolve step ORs into hs_residency.err (device). */
#define HS_DEVERR_VICTIMS 1   /* more faults than replaceable hot slots      */
#define HS_DEVERR_APPEND_RANGE 4    /* hs_append_tokens: a request would pass
                                       T_stride or take more than P tokens, or
                                       the page receiving its first new token is
                                       not resident; nothing was appended      */
#define HS_DEVERR_APPEND_NO_BLOCK 8 /* hs_append_tokens: a free list holds fewer
                                       blocks than the pages to open; nothing
                                       was appended                            */
#define HS_DEVERR_DEMOTE_FULL 16    /* hs_demote_pages: the free list cannot take
                                       the blocks; nothing was demoted         */
#define HS_DEVERR_NO_HOST 2   /* a selected token is neither resident, hot,
                                 nor present in the host pool                */

/* Batch geometry shared by all calls.
 * B requests with P query positions each.  Request b has T_b = ctx_len[b]
 * cached tokens (0 <= T_b <= T_stride); query position p (0 <= p < P) sees the
 * tokens 0 .. T_b - P + p (the P newest tokens are the P positions of a
 * multi-token-prediction step; P = 4 for three speculative tokens, page "Un
 * contexte d'un million sur huit H200", section "Les chiffres").
 * T_stride is the row stride of every per-token array and a multiple of 64;
 * every block table has max_blocks = T_stride / 64 columns. */
typedef struct hs_batch {
  int32_t B;               /* 1 .. 65535                                     */
  int32_t P;               /* 1 .. 4                                         */
  int32_t T_stride;        /* multiple of 64, 64 .. 2^24                     */
  int32_t max_blocks;      /* T_stride / 64                                  */
  const int32_t* ctx_len;  /* device [B] int32                               */
} hs_batch;

/* Indexer scores (page "Un contexte d'un million sur huit H200", section
 * "Ce qui se passe": an indexer selects the tokens sparse MLA attends to; its
 * cache stays resident and is much smaller than the latent cache).  The pages
 * give no formula; the one computed is
 *
 *   scores[b,p,t] = sum_h w[b,p,h] * max(0, sum_d q[b,p,h,d] * k[b,t,d]) + bias[b,t]
 *
 * for 0 <= t <= T_b - P + p, with one key per token shared by all heads.
 *   q_idx     [B, P, H_idx, D_idx]   q_t = HS_BF16 (with k_t = HS_E4M3),
 *                                    HS_E4M3 (with k_t = HS_E4M3; D_idx = 128;
 *                                    codes from hs_quantize_queries) or
 *                                    HS_F32 (with k_t = HS_F32)
 *   w         [B, P, H_idx] fp32, non-negative values need not hold
 *   idx_pool  [N_blocks, 64, D_idx]  key of token t of request b is row t % 64
 *                                    of block idx_bt[b, t / 64]
 *   idx_scale [N_blocks] fp32 per-block dequantization scale, > 0, or NULL (= 1);
 *             must be NULL for HS_F32 keys
 *   idx_bt    [B, max_blocks] int32; entries for pages past T_b are never read
 *   bias      [B, T_stride] fp32 or NULL
 *   scores    [B, P, T_stride] fp32 output; entries past a position's visible
 *             limit are left unspecified (hs_topk never reads them)
 * Supported: D_idx in {64, 128}; H_idx a multiple of 16 up to 64 on the
 * HS_BF16/HS_E4M3 path (bf16 matrix cores, fp32 accumulation) and on the
 * HS_E4M3/HS_E4M3 path (fp8 matrix cores, exact products, fp32 accumulation;
 * D_idx = 128 only), 1 .. 64 on HS_F32.
 * Keys, queries and scores need 16-byte alignment, and so does w on the
 * matrix-core paths. */
hs_status hs_indexer_scores(const hs_batch* batch, int32_t H_idx, int32_t D_idx,
                            hs_dtype q_t, const void* q_idx, const float* w,
                            hs_dtype k_t, const void* idx_pool, const float* idx_scale,
                            const int32_t* idx_bt, const float* bias, float* scores,
                            void* stream);

/* Per-head E4M3 quantization of bf16 indexer queries, for the HS_E4M3 query
 * path of hs_indexer_scores / hs_indexer_topk.  The pages keep the KV cache in
 * FP8 (page "Un contexte d'un million sur huit H200", section "Les chiffres")
 * and leave the indexer's query precision open; this is an optional variant
 * that puts both operands of the q.k contraction in FP8.  For every row
 * r = (b, p, h) of D_idx values:
 *   amax = max_d |q[r, d]|;  if amax < 2^-64 the row's codes and s are 0,
 *   else inv = 448 / amax, q8[r, d] = E4M3(q[r, d] * inv) (binary32 division
 *   and product, round to nearest, ties to even), s = amax / 448;
 *   w_scaled[r] = w[r] * s   (binary32).
 * Because s >= 0 it leaves the ReLU, so scores computed from (q8, w_scaled)
 * approximate those of (q, w) with the queries rounded to 4 significant bits.
 *   q_idx    [B, P, H_idx, D_idx] bf16, finite; w [B, P, H_idx] fp32
 *   q8       [B, P, H_idx, D_idx] E4M3 codes (output; may not alias q_idx)
 *   w_scaled [B, P, H_idx] fp32 (output; may alias w)
 * D_idx in {64, 128}; 1 <= H_idx <= 64. */
hs_status hs_quantize_queries(const hs_batch* batch, int32_t H_idx, int32_t D_idx,
                              const void* q_idx, const float* w, uint8_t* q8, float* w_scaled,
                              void* stream);

/* Top-K per query position (page "Un contexte d'un million sur huit H200",
 * section "Ce qui se passe"; K = 2048 on "vLLM sert GLM-5.3 en contexte 1M sur
 * 16 H200", section "Comment s'y prendre").  For each (b, p): the K largest
 * scores among the visible tokens, ties going to the lower token index; written
 * in ascending token order.  A position that sees n <= K tokens selects all n,
 * followed by -1.  Scores must not be NaN; -0.0 equals +0.0.
 *   scores [B, P, T_stride] fp32 (16-byte aligned), topk [B, P, K] int32 output.
 * 1 <= K <= 8192.  Workspace: hs_workspace_bytes(HS_OP_TOPK, ...), 16-byte
 * aligned; its contents on entry do not matter (the call clears what it
 * needs), and it is left zero-filled. */
hs_status hs_topk(const hs_batch* batch, int32_t K, const float* scores, int32_t* topk,
                  void* ws, size_t ws_bytes, void* stream);

/* Token-sharded top-K: the selection as a cache split across GPUs by tokens
 * makes it (page "vLLM sert GLM-5.3 en contexte 1M sur 16 H200", section "Le
 * mécanisme": DCP splits the KV cache by tokens across GPUs and gathers the
 * fragments at every layer), emulated on one GPU.  Each
 * request's tokens are cut into S contiguous shards of T_stride/S tokens; each
 * shard keeps its own top-K, and the K best of the union of those candidates
 * are kept, with the same order and tie rule.  The result equals hs_topk's
 * (every token of the global top-K is in its shard's top-K); a few long rows
 * become S times as many short ones for the radix select.
 * One query position (batch->P == 1); 1 <= S <= 64 and T_stride a multiple of
 * 64*S; 1 <= K <= 8192; scores 16-byte aligned.  Workspace:
 * hs_topk_sharded_workspace_bytes(B, T_stride, K, S), 16-byte aligned; its
 * contents on entry do not matter (the call clears what it needs). */
hs_status hs_topk_sharded(const hs_batch* batch, int32_t K, int32_t S, const float* scores,
                          int32_t* topk, void* ws, size_t ws_bytes, void* stream);
size_t hs_topk_sharded_workspace_bytes(int32_t B, int32_t T_stride, int32_t K, int32_t S);

/* hs_indexer_scores followed by hs_topk, with the first pass of the top-K
 * radix select (the per-row histogram of the top 11 score-key bits) built in
 * the indexer's epilogue instead of a separate pass over the scores.  Same
 * arguments and outputs as the two calls; scores are still written.
 * Workspace: hs_workspace_bytes(HS_OP_TOPK, ...) bytes, 16-byte aligned, and
 * ZERO-FILLED before its first use: the histograms are added into it.  Every
 * call (and every hs_topk call) returns every word it wrote to zero, so a
 * workspace zeroed once can be reused as it is by any later call, whatever
 * its batch geometry. */
hs_status hs_indexer_topk(const hs_batch* batch, int32_t H_idx, int32_t D_idx, hs_dtype q_t,
                          const void* q_idx, const float* w, hs_dtype k_t, const void* idx_pool,
                          const float* idx_scale, const int32_t* idx_bt, const float* bias,
                          float* scores, int32_t K, int32_t* topk, void* ws, size_t ws_bytes,
                          void* stream);

/* The two halves of hs_indexer_topk, for callers that schedule or time them
 * apart:
 *   hs_indexer_topk_scores  the indexer: scores, and every row's histogram
 *                           added into the (zeroed) workspace (none for
 *                           HS_F32 queries);
 *   hs_indexer_topk_select  the rest of the selection from those scores and
 *                           histograms (for q_t = HS_F32 the whole of
 *                           hs_topk); it returns the workspace to zero.
 * Enqueued in this order on one stream, with the same batch, K, scores and
 * workspace, they are hs_indexer_topk.  A scores half must be followed by its
 * select half before the workspace is used again. */
hs_status hs_indexer_topk_scores(const hs_batch* batch, int32_t H_idx, int32_t D_idx,
                                 hs_dtype q_t, const void* q_idx, const float* w, hs_dtype k_t,
                                 const void* idx_pool, const float* idx_scale,
                                 const int32_t* idx_bt, const float* bias, float* scores,
                                 int32_t K, void* ws, size_t ws_bytes, void* stream);
hs_status hs_indexer_topk_select(const hs_batch* batch, hs_dtype q_t, int32_t K,
                                 const float* scores, int32_t* topk, void* ws, size_t ws_bytes,
                                 void* stream);

/* hs_indexer_topk for callers that cannot allocate device memory: code under
 * HIP graph capture that may not call hipMalloc, tight serving loops, and
 * harnesses that forbid allocation.  Same arguments and results as
 * hs_indexer_topk without ws/ws_bytes: the workspace is a static device
 * array inside the library, 64 MiB per GPU, created when the library's code
 * object is loaded on that GPU and held until the process ends.  The call
 * allocates nothing; it clears the part of the array that must start at zero
 * with a kernel on `stream`.  Sizes whose hs_workspace_bytes(HS_OP_TOPK, ...)
 * exceed 64 MiB are rejected with HS_ERR_WORKSPACE (B*P*T_stride up to about
 * 8.3 million tokens: the 128K batch of 32 and the 1M batch of 4 fit).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialized by the
 * caller. */
hs_status hs_indexer_topk_noalloc(const hs_batch* batch, int32_t H_idx, int32_t D_idx,
                                  hs_dtype q_t, const void* q_idx, const float* w, hs_dtype k_t,
                                  const void* idx_pool, const float* idx_scale,
                                  const int32_t* idx_bt, const float* bias, float* scores,
                                  int32_t K, int32_t* topk, void* stream);

/* Residency state of a batch: one shared paged pool of latent rows on the GPU,
 * per-request hot buffers made of ordinary pool blocks (page "Un contexte d'un
 * million sur huit H200", section "Les trois états de résidence", last
 * paragraph) and a pinned host pool.  The tables are read and updated in place
 * by hs_resolve_rows. */
typedef struct hs_residency {
  int32_t C;                  /* hot rows per request: 0, or a multiple of 64 up to 16384,
                                 with C >= P*K (the pages' default is 2K, and
                                 (num_speculative_tokens + 2) K with MTP,
                                 section "Ce qu'il faut en retenir")         */
  int32_t L;                  /* latent layers sharing this state, 1 .. 16   */
  hs_dtype kv_t;              /* HS_E4M3 (row_scale/host_scale required) or
                                 HS_F32 (scales must be NULL)                */
  int32_t host_row_pitch;     /* rows from one host token to the next in
                                 host_rows / host_scale: 0 or 1 = consecutive
                                 (layer-major [L, host_layer_rows, 576]); L
                                 with host_layer_rows = 1 interleaves the
                                 layers ([tokens, L, 576]), so the L rows of
                                 one fault are one contiguous read           */
  int64_t pool_layer_rows;    /* rows from one layer to the next in pool and
                                 row_scale (>= rows used by the block ids)   */
  int64_t host_layer_rows;    /* same for host_rows / host_scale             */
  const int32_t* bt;          /* [B, max_blocks] pool block of a resident
                                 page, -1 = page not resident               */
  const int32_t* hot_blocks;  /* [B, C/64] pool blocks of the hot buffer;
                                 slot v is row hot_blocks[b, v/64]*64 + v%64 */
  int32_t* tok2slot;          /* [B, T_stride] hot slot of a token, -1 = none */
  int32_t* slot2tok;          /* [B, C] token in a slot, -1 = empty          */
  int32_t* stamp;             /* [B, C] last step that used the slot, 0 = never */
  int32_t* step;              /* [1] step counter, incremented per call      */
  int32_t* err;               /* [1] device error bits (HS_DEVERR_*), OR-ed  */
  void* pool;                 /* [L, pool_layer_rows, 576] rows             */
  float* row_scale;           /* [L, pool_layer_rows] per-row fp32 scale     */
  const void* host_rows;      /* pinned host rows of 576 values, given by its
                                 device-accessible address: token h of layer
                                 l is row l*host_layer_rows + h*pitch (pitch =
                                 max(host_row_pitch, 1)); may be NULL when no
                                 page is host-only                           */
  const float* host_scale;    /* scale of each host row, same indexing;
                                 any device-accessible memory.  Device memory
                                 is preferable: the table is small, and reading
                                 it from the host costs one link transaction
                                 per fault                                  */
  const int64_t* host_bt;     /* [B, max_blocks] host token index h of token
                                 64*j of page j (its row in layer l is
                                 l*host_layer_rows + h*pitch), -1 = page has
                                 no host copy                                */
} hs_residency;

/* Fused resolve (page "Un contexte d'un million sur huit H200", section "Les
 * trois états de résidence": resident tokens are read in place, hot tokens
 * refresh their LRU entry, a fault copies one row from pinned host memory, and
 * no CPU decision sits on the path).  The pages give no LRU policy; the one
 * implemented, bit-exact with the oracle:
 *   s = step + 1 for the call.  Per request, U = the sorted distinct tokens of
 *   topk[b]; each t in U (page j = t/64) is RESIDENT if bt[b,j] >= 0, a HIT if
 *   tok2slot[b,t] >= 0 (its stamp becomes s), else a FAULT (ascending order).
 *   Victims are the slots with stamp < s ordered by (stamp, slot); the i-th
 *   fault takes the i-th victim, evicting its previous token, and host row
 *   l*host_layer_rows + (host_bt[b,j] + t%64)*pitch (576 values) and its scale
 *   are copied to the slot's pool row in every layer l.  step becomes s.
 * Outputs:
 *   row_ids [B, P, K] int32: pool row of topk[b,p,k], -1 for -1 entries
 *   faults  [B, P*K, 2] int32: (token, slot) of each served fault, ascending
 *           tokens; entries past counts[b][2] are unspecified
 *   counts  [B, 4] int32: resident, hits, faults served, evictions (over U)
 * Faults beyond the replaceable slots and tokens with no copy anywhere get row
 * -1 and set HS_DEVERR_* bits; with C >= P*K and a host copy of every
 * non-resident page neither can happen.  P*K <= 8192.  No workspace is needed
 * (ws may be NULL, ws_bytes 0). */
hs_status hs_resolve_rows(const hs_batch* batch, int32_t K, const int32_t* topk,
                          const hs_residency* res, int32_t* row_ids, int32_t* faults,
                          int32_t* counts, void* ws, size_t ws_bytes, void* stream);

/* The two halves of hs_resolve_rows, for callers that overlap the host-link
 * copies with other work (the copies are bound by the host link, the rest of
 * the step by HBM):
 *   hs_resolve_tables  everything but the copies: tables, row ids, fault list
 *                      and counts (the same outputs as hs_resolve_rows);
 *   hs_copy_faults     copies the rows listed in faults/counts (as written by
 *                      the preceding hs_resolve_tables on the same batch and
 *                      state) from the host pool into their slots in every
 *                      layer, with their scales, and advances res->step.
 * Enqueued on one stream in this order they are hs_resolve_rows.  The copy may
 * run on another stream behind an event recorded after hs_resolve_tables;
 * then nothing may read the faulted slots before it completes, and the next
 * hs_resolve_tables on the same state (and step counter) must wait for it.
 * `workgroups` bounds the copy's grid: 0 lets it use the whole GPU (fastest
 * alone); a small grid (e.g. 32) leaves most compute units to HBM-bound work
 * running concurrently on another stream, at nearly the same link rate.
 * 0 <= workgroups <= 1024. */
hs_status hs_resolve_tables(const hs_batch* batch, int32_t K, const int32_t* topk,
                            const hs_residency* res, int32_t* row_ids, int32_t* faults,
                            int32_t* counts, void* stream);
hs_status hs_copy_faults(const hs_batch* batch, int32_t K, const hs_residency* res,
                         const int32_t* faults, const int32_t* counts, int32_t workgroups,
                         void* stream);

/* hs_indexer_topk_select followed by hs_resolve_tables, the fused resolve
 * step of page "Un contexte d'un million sur huit H200", section "Les trois
 * états de résidence", right behind the selection it consumes: with one query
 * position (batch->P == 1) each request's workgroup finishes its top-K and
 * resolves that list in the same kernel, so no launch separates the two; with
 * several positions it enqueues the two calls.  Arguments as the two calls
 * (q_t, K, scores, topk, ws, ws_bytes of hs_indexer_topk_select after the
 * matching hs_indexer_topk_scores; res, row_ids, faults, counts of
 * hs_resolve_tables), with the same results: topk, the workspace returned to
 * zero, tables, row ids, fault list and counts.  hs_copy_faults then follows
 * as after hs_resolve_tables. */
hs_status hs_indexer_topk_select_resolve(const hs_batch* batch, hs_dtype q_t, int32_t K,
                                         const float* scores, int32_t* topk, void* ws,
                                         size_t ws_bytes, const hs_residency* res,
                                         int32_t* row_ids, int32_t* faults, int32_t* counts,
                                         void* stream);

/* hs_copy_faults for layers layer0 .. layer0 + n_layers - 1 of every fault
 * only, for callers that let a layer's attention start as soon as its rows
 * are in (IndexShare on page "Un contexte d'un million sur huit H200",
 * section "Ce qui se passe": one selection feeds several attention layers, so
 * layer l's attention needs only layer l's faulted rows).  Calls that cover
 * every layer once, in any grouping, do what one hs_copy_faults does; the
 * call whose range ends at layer L - 1 advances res->step, so it comes last
 * (or the next hs_resolve_tables waits for all of them).
 * 0 <= layer0, 1 <= n_layers, layer0 + n_layers <= res->L. */
hs_status hs_copy_faults_layers(const hs_batch* batch, int32_t K, const hs_residency* res,
                                const int32_t* faults, const int32_t* counts, int32_t layer0,
                                int32_t n_layers, int32_t workgroups, void* stream);

/* Sparse MLA decode attention in the absorbed (MQA) form that the
 * sparse_mla_force_mqa option keeps on the sparse kernel (page "vLLM sert
 * GLM-5.3 en contexte 1M sur 16 H200", section "Comment s'y prendre"): all Hq
 * heads attend over the same selected latent rows x (576 values), which are
 * the keys; the values are their first 512 values:
 *   z_j = sm_scale * row_scale[r_j] * (q[b,p,h,:] . code(r_j))
 *   out[b,p,h,:] = sum_j softmax(z)_j * row_scale[r_j] * code(r_j)[0:512]
 *   lse[b,p,h]   = ln sum_j exp(z_j)
 * over the rows r_j = row_ids[b,p,j] >= 0, j ascending; -1 entries are skipped.
 * With no valid row the output is 0 and lse is -inf.  The reduction order
 * depends only on the order of row_ids, never on the row addresses.
 *   q       [B, P, Hq, 576]   HS_BF16 with kv_t = HS_E4M3, or HS_F32 with HS_F32
 *   pool    [rows, 576] one layer's rows; row_scale [rows] fp32 (E4M3 only,
 *           NULL for F32)
 *   out     [B, P, Hq, 512] fp32; lse [B, P, Hq] fp32 or NULL
 * Hq is a multiple of 16 in [16, 128]: the heads one GPU holds, taken by the
 * kernels in groups of 16 that share every row gather.  1 <= K <= 8192.
 * Workspace: hs_workspace_bytes(HS_OP_MLA, ...). */
hs_status hs_sparse_mla_decode(const hs_batch* batch, int32_t K, int32_t Hq, hs_dtype q_t,
                               const void* q, hs_dtype kv_t, const void* pool,
                               const float* row_scale, const int32_t* row_ids,
                               float sm_scale, float* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream);

/* The same attention for L layers that share one selection (the IndexShare
 * reuse on page "Un contexte d'un million sur huit H200", section "Ce qui se
 * passe": one indexer pass and one top-K set feed several attention layers), in
 * one launch: the grid spans the layers, so layers that are each too small to
 * fill the GPU run side by side, and one combine merges every layer's slices.
 *   q         [L, B, P, Hq, 576]    layer l's queries
 *   pool      [L, pool_layer_rows, 576], row_scale [L, pool_layer_rows]: layer
 *             l's row r is at l * pool_layer_rows + r (row_ids index every layer)
 *   out       [L, B, P, Hq, 512], lse [L, B, P, Hq] (NULL = not written)
 *   ws        hs_mla_layers_workspace_bytes(B, P, K, Hq, L) bytes, 16-byte
 *             aligned (0 = none needed)
 * L = 1 computes the same as hs_sparse_mla_decode.  For L > 1 the K rows are cut
 * into fewer slices per layer, so the fp32 summation order (and the last bits)
 * can differ from L calls of hs_sparse_mla_decode; it depends only on row_ids. */
hs_status hs_sparse_mla_decode_layers(const hs_batch* batch, int32_t K, int32_t Hq, int32_t L,
                                      hs_dtype q_t, const void* q, hs_dtype kv_t,
                                      const void* pool, int64_t pool_layer_rows,
                                      const float* row_scale, const int32_t* row_ids,
                                      float sm_scale, float* out, float* lse, void* ws,
                                      size_t ws_bytes, void* stream);
size_t hs_mla_layers_workspace_bytes(int32_t B, int32_t P, int32_t K, int32_t Hq, int32_t L);

/* Token-sharded attention: the attention as a KV cache split across GPUs by
 * tokens computes it (page "vLLM sert GLM-5.3 en contexte 1M sur 16 H200",
 * section "Le mécanisme": DCP splits the KV cache by tokens across GPUs and
 * gathers the fragments at every layer), emulated on one GPU.  Each request's
 * tokens are cut into S contiguous shards of T_stride / S tokens; shard s
 * attends over the selected tokens it holds and hands over its fragment, and
 * the fragments are merged in shard order by their log-sum-exp:
 *   shard_out[b,p,s,h,:], shard_lse[b,p,s,h]: hs_sparse_mla_decode's out and
 *       lse over the entries j of topk[b,p,:] with topk[b,p,j] / (T_stride/S)
 *       = s (0 and -inf for a shard with none);
 *   lse[b,p,h] = ln sum_s exp(shard_lse[b,p,s,h]),
 *   out[b,p,h,:] = sum_s exp(shard_lse[b,p,s,h] - lse[b,p,h]) shard_out[b,p,s,h,:]
 * which is the unsharded attention up to rounding.
 *   topk    [B, P, K] token ids in ascending order, -1 entries last (hs_topk's
 *           or hs_topk_sharded's output): they say which shard holds each row;
 *           another order gives unspecified (but in-bounds) results
 *   row_ids [B, P, K] pool rows of those tokens (-1 = skipped), as for
 *           hs_sparse_mla_decode; q, pool, row_scale, out, lse likewise
 *   shard_out [B, P, S, Hq, 512] fp32 output, shard_lse [B, P, S, Hq] fp32 output
 * 1 <= S <= 64 and S divides T_stride; Hq a multiple of 16 in [16, 128];
 * 1 <= K <= 8192.  Workspace: hs_mla_sharded_workspace_bytes(B, P, K, S, Hq),
 * 16-byte aligned; its contents on entry do not matter. */
hs_status hs_sparse_mla_decode_sharded(const hs_batch* batch, int32_t K, int32_t S, int32_t Hq,
                                       hs_dtype q_t, const void* q, hs_dtype kv_t,
                                       const void* pool, const float* row_scale,
                                       const int32_t* topk, const int32_t* row_ids,
                                       float sm_scale, float* shard_out, float* shard_lse,
                                       float* out, float* lse, void* ws, size_t ws_bytes,
                                       void* stream);
size_t hs_mla_sharded_workspace_bytes(int32_t B, int32_t P, int32_t K, int32_t S, int32_t Hq);

#define HS_OP_INDEXER 0
#define HS_OP_TOPK 1
#define HS_OP_RESOLVE 2
#define HS_OP_MLA 3
#define HS_OP_CACHE 4

/* Device workspace in bytes needed by `op` for these sizes (0 if none). */
size_t hs_workspace_bytes(int32_t op, int32_t B, int32_t P, int32_t T_stride, int32_t K,
                          int32_t Hq);

/* ---- Around the decode step: KV append, pre-copy, demotion ----
 * Page "Un contexte d'un million sur huit H200", section "Les trois états de
 * résidence": with full residency completed prefix pages are copied to the
 * host ahead of time, so that their block can be given up later without a
 * copy; with mixed residency the tail stays on the GPU and older pages live
 * only on the host; the indexer's cache stays resident (section "Ce qui se
 * passe").  Every decision is taken on the device and is deterministic, so
 * the calls are graph-capturable and reproducible.
 *
 * A free list is a stack of pool blocks in device memory: blocks[0 .. *count-1]
 * are free, the top is blocks[*count - 1]. */
typedef struct hs_free_list {
  int32_t* blocks;     /* device [capacity]                                 */
  int32_t* count;      /* device [1]                                        */
  int32_t capacity;
  int32_t pad_;
} hs_free_list;

/* The indexer's paged key cache (as passed to hs_indexer_scores). */
typedef struct hs_index_cache {
  hs_dtype k_t;        /* HS_E4M3 (scale per block) or HS_F32 (no scale)    */
  int32_t D_idx;       /* 64 or 128                                         */
  void* pool;          /* [N_idx_blocks, 64, D_idx]                         */
  float* scale;        /* [N_idx_blocks] or NULL                            */
  int32_t* bt;         /* [B, max_blocks]                                   */
} hs_index_cache;

/* Append n_new[b] (0 .. P) tokens to request b after its last token: the
 * latent row of every layer with its scale, and the indexer key.  A token at
 * a page start (t % 64 == 0) opens a page: a latent block and an indexer block
 * are popped from the two free lists (request order, then token order) and
 * the indexer block's scale is set to that token's new_key_scale.  Then
 * ctx_len[b] += n_new[b].  All-or-nothing: on a range or capacity problem the
 * call appends nothing and sets HS_DEVERR_APPEND_* in res->err.
 *   ctx_len       the batch's ctx_len (batch->ctx_len), updated in place
 *   n_new         device [B] int32
 *   res           latent pool, row_scale, bt (updated), err, L, kv_t
 *   new_rows      device [B, P, L, 576] in kv_t; new_row_scale [B, P, L] fp32
 *                 (E4M3) or NULL (F32)
 *   idx           indexer cache (pool, scale and bt updated)
 *   new_keys      device [B, P, D_idx] in idx->k_t; new_key_scale [B, P] fp32
 *                 (E4M3) or NULL (F32)
 *   ws            hs_workspace_bytes(HS_OP_CACHE, B, ...) bytes, 16-byte aligned
 * Pointers to row data need 16-byte alignment. */
hs_status hs_append_tokens(const hs_batch* batch, int32_t* ctx_len, const int32_t* n_new,
                           const hs_residency* res, const void* new_rows,
                           const float* new_row_scale, const hs_index_cache* idx,
                           const void* new_keys, const float* new_key_scale,
                           const hs_free_list* latent_free, const hs_free_list* idx_free,
                           void* ws, size_t ws_bytes, void* stream);

/* Pre-copy: for every request, its lowest completed pages (all 64 tokens below
 * T_b) that are resident and have no host copy, at most max_pages (1 .. 1024)
 * per request, are copied (rows and scales of every layer) to their host slot,
 * host row b*T_stride + 64p, and host_bt records it.  Writes res->host_rows
 * (pinned host memory, zero-copy), res->host_scale and res->host_bt, which must
 * all be given; the host pool holds B*T_stride rows per layer
 * (res->host_layer_rows >= B*T_stride).  Bound by the host link (writes). */
hs_status hs_precopy_pages(const hs_batch* batch, const hs_residency* res, int32_t max_pages,
                           void* stream);

/* Demotion under pressure: request b gives up the blocks of its lowest
 * n_demote[b] pages that are resident, have a host copy and lie outside its
 * last tail_pages pages (tail_pages >= 1: the tail, counted from the page of
 * its last token, is never demoted).  bt becomes -1 for them and their blocks
 * are pushed on latent_free (request order, then page order).  All-or-nothing
 * if the free list would pass its capacity (HS_DEVERR_DEMOTE_FULL).
 *   n_demote  device [B] int32;  ws as for hs_append_tokens. */
hs_status hs_demote_pages(const hs_batch* batch, const hs_residency* res,
                          const int32_t* n_demote, int32_t tail_pages,
                          const hs_free_list* latent_free, void* ws, size_t ws_bytes,
                          void* stream);

/* Device-accessible address of pinned host memory allocated with
 * hipHostMalloc (or torch pin_memory); HS_ERR_HIP if it is not pinned. */
hs_status hs_host_device_ptr(const void* pinned_host, const void** dev_ptr);

/* Message of the last failed call on this thread ("" if none). */
const char* hs_last_error(void);

/* HS_ABI_VERSION of the loaded library. */
int32_t hs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HS_H */
