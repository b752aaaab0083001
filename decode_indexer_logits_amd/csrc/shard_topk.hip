// Token-sharded top-K on one GPU: the way a cache split across GPUs by tokens
// selects (page "vLLM sert GLM-5.3 en contexte 1M sur 16 H200", section "Le
// mécanisme": DCP splits the KV cache by tokens across GPUs).  Each request's visible
// tokens are cut into S contiguous shards of T_stride/S tokens; every shard
// keeps its own top-K (a row of its own for the radix select, so a few long
// rows become many short ones), the candidates of all shards are gathered
// with their scores in ascending token order, and a second select keeps the
// K best of them.  Every token of the global top-K is in its shard's top-K,
// and the candidate order is the token order, so ties break the same way:
// the result equals the unsharded top-K.
//
// One query position per request (with P = 1 the score rows of the shards
// are consecutive rows of T_stride/S scores, so the shard view is the same
// array with another row length).
#include "hs_common.h"
#include "hs_launch.h"
#include "topk_select.h"

namespace hs {
namespace {

constexpr int kNT = 256;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int cand_stride(int S, int K) { return (S * K + kBlock - 1) / kBlock * kBlock; }

struct ShardWs {
  int32_t* ctx_s;      // [B*S] visible tokens of each shard
  int32_t* topk_s;     // [B*S, K] shard-local selections
  int32_t* cand_tok;   // [B, Tc] candidate tokens, ascending
  float* cand_score;   // [B, Tc] their scores
  int32_t* cand_n;     // [B] candidates per request
  int32_t* sel;        // [B, K] selected candidate indices
  void* inner;         // workspace of the two selects, used one after the other
};

ShardWs shard_ws(void* ws, int B, int S, int K) {
  const int Tc = cand_stride(S, K);
  char* p = static_cast<char*>(ws);
  ShardWs w;
  w.ctx_s = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * S * 4);
  w.topk_s = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * S * K * 4);
  w.cand_tok = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * Tc * 4);
  w.cand_score = reinterpret_cast<float*>(p);
  p += align256((size_t)B * Tc * 4);
  w.cand_n = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * 4);
  w.sel = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * K * 4);
  w.inner = p;
  return w;
}

__device__ __forceinline__ int shard_visible(int T, int s, int Ts) {
  return min(max(T - s * Ts, 0), Ts);
}

// One workgroup per shard row r = b * S + s: the row's visible tokens, and its
// histogram and counters of the shard-level select zeroed (the workspace may
// hold anything on entry).
__global__ __launch_bounds__(kNT) void shard_ctx_zero_kernel(int S, int Ts,
                                                             const int32_t* __restrict__ ctx_len,
                                                             int32_t* __restrict__ ctx_s,
                                                             topk_sel::TopkWs w) {
  const int r = blockIdx.x;
  uint4* h = reinterpret_cast<uint4*>(w.hist + (size_t)r * topk_sel::kBins1);
  for (int i = threadIdx.x; i < topk_sel::kBins1 / 4; i += kNT) h[i] = make_uint4(0, 0, 0, 0);
  if (threadIdx.x < topk_sel::kCnt) w.cnt[r * topk_sel::kCnt + threadIdx.x] = 0;
  if (threadIdx.x == 0) ctx_s[r] = shard_visible(ctx_len[r / S], r % S, Ts);
}

// One workgroup per (request, shard): its valid selections, shifted to
// request tokens, with their scores, at the shard's offset in the candidate
// row (the offset is the sum of min(K, visible) over the shards before it).
// It also adds its candidates to the candidate row's first-level histogram of
// the second select (the pass that hs_topk runs on its own): LDS counts, then
// one 64-bit atomic per non-empty pair of bins.  That histogram is zero on
// entry because the shard-level select, which ran just before, returned its
// own histograms and counters (which cover it) to zero.  Rows of at most K
// candidates need no histogram; their counts are cleared by the selection.
__global__ __launch_bounds__(kNT) void shard_gather_kernel(
    int S, int Ts, int T_stride, int K, int Tc, const int32_t* __restrict__ ctx_len,
    const float* __restrict__ scores, const int32_t* __restrict__ topk_s,
    int32_t* __restrict__ cand_tok, float* __restrict__ cand_score,
    int32_t* __restrict__ cand_n, uint32_t* __restrict__ hist2) {
  __shared__ uint32_t h[topk_sel::kBins1];
  const int b = blockIdx.x / S, s = blockIdx.x % S;
  for (int i = threadIdx.x; i < topk_sel::kBins1; i += kNT) h[i] = 0;
  const int T = ctx_len[b];
  int off = 0, total = 0;
  for (int u = 0; u < S; ++u) {
    const int v = min(K, shard_visible(T, u, Ts));
    if (u < s) off += v;
    total += v;
  }
  const int nv = min(K, shard_visible(T, s, Ts));
  const int32_t* src = topk_s + (size_t)(b * S + s) * K;
  __syncthreads();
  for (int i = threadIdx.x; i < nv; i += kNT) {
    const int t = src[i] + s * Ts;
    const float sc = scores[(size_t)b * T_stride + t];
    cand_tok[(size_t)b * Tc + off + i] = t;
    cand_score[(size_t)b * Tc + off + i] = sc;
    atomicAdd(&h[score_key(sc) >> 21], 1u);
  }
  if (s == 0 && threadIdx.x == 0) cand_n[b] = total;
  __syncthreads();
  uint32_t* hrow = hist2 + (size_t)b * topk_sel::kBins1;
  for (int i = threadIdx.x; i < topk_sel::kBins1 / 2; i += kNT)
    if (h[2 * i] | h[2 * i + 1])
      atomicAdd(reinterpret_cast<unsigned long long*>(hrow + 2 * i),
                (unsigned long long)h[2 * i] | ((unsigned long long)h[2 * i + 1] << 32));
}

__global__ __launch_bounds__(kNT) void shard_map_kernel(int B, int K, int Tc,
                                                        const int32_t* __restrict__ sel,
                                                        const int32_t* __restrict__ cand_tok,
                                                        int32_t* __restrict__ topk) {
  const int i = blockIdx.x * kNT + threadIdx.x;
  if (i >= B * K) return;
  const int j = sel[i];
  topk[i] = j >= 0 ? cand_tok[(size_t)(i / K) * Tc + j] : -1;
}

}  // namespace

size_t topk_sharded_workspace_bytes(int B, int T_stride, int K, int S) {
  const int Tc = cand_stride(S, K);
  const size_t own = align256((size_t)B * S * 4) + align256((size_t)B * S * K * 4) +
                     2 * align256((size_t)B * Tc * 4) + align256((size_t)B * 4) +
                     align256((size_t)B * K * 4);
  const size_t a = topk_workspace_bytes(B * S, 1, T_stride / S, K);
  const size_t c = topk_workspace_bytes(B, 1, Tc, K);
  return own + (a > c ? a : c);
}

// Eight launches: shard contexts with the shard select's zeroing, its histogram,
// filter and finalize, the gather with the candidate select's histogram, that
// select's filter and finalize, and the map back to tokens.  Both selects use
// the one inner workspace; the candidate select's histogram rows and counters
// lie inside the shard select's histogram area (B rows of kBins1 words plus
// B * kCnt counters against B * S rows, S >= 2; the same rows when S = 1),
// which that select's finalize leaves zero.
hipError_t launch_topk_sharded(const BatchDims& d, int K, int S, const float* scores,
                               int32_t* topk, void* ws, hipStream_t s) {
  const int Ts = d.T_stride / S, Tc = cand_stride(S, K);
  ShardWs w = shard_ws(ws, d.B, S, K);
  const topk_sel::TopkWs w1 = topk_sel::topk_ws(w.inner, d.B * S, Ts, K);
  const topk_sel::TopkWs w2 = topk_sel::topk_ws(w.inner, d.B, Tc, K);
  hipLaunchKernelGGL(shard_ctx_zero_kernel, dim3(d.B * S), dim3(kNT), 0, s, S, Ts, d.ctx_len,
                     w.ctx_s, w1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const BatchDims ds{d.B * S, 1, Ts, Ts / kBlock, w.ctx_s};
  e = launch_topk_hist(ds, K, scores, w.inner, s);
  if (e == hipSuccess) e = launch_topk_select(ds, K, scores, w.topk_s, w.inner, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shard_gather_kernel, dim3(d.B * S), dim3(kNT), 0, s, S, Ts, d.T_stride, K,
                     Tc, d.ctx_len, scores, w.topk_s, w.cand_tok, w.cand_score, w.cand_n, w2.hist);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const BatchDims dc{d.B, 1, Tc, Tc / kBlock, w.cand_n};
  e = launch_topk_select(dc, K, w.cand_score, w.sel, w.inner, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shard_map_kernel, dim3((d.B * K + kNT - 1) / kNT), dim3(kNT), 0, s, d.B, K,
                     Tc, w.sel, w.cand_tok, topk);
  return hipGetLastError();
}

}  // namespace hs
