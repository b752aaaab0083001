// Exact top-K per query position on gfx950 (K best tokens of the indexer,
// page "Un contexte d'un million sur huit H200", section "Ce qui se passe";
// K = 2048 on "vLLM sert GLM-5.3 en contexte 1M sur 16 H200", section
// "Comment s'y prendre").
//
// Scores map to order-preserving uint32 keys.  A row (one request position,
// up to 2^24 tokens) is spread over many workgroups so that both few long rows
// and many short ones fill the chip:
//   1. zero       per-row histogram and counters (hs_topk only: the finalize
//                 pass below returns every word of the workspace the call
//                 wrote to zero, so hs_indexer_topk, whose workspace is zeroed
//                 once by its owner, needs no clearing launch)
//   2. histogram  of the top 11 key bits, per 8192-token chunk: LDS counts,
//                 then one global atomic per non-empty bin (the fused path of
//                 hs_indexer_topk builds it in the indexer's epilogue instead)
//   3. filter     one wave of every 4096-token workgroup (8192 on rows over
//                 2^18 tokens, 1024 when few rows would leave the chip idle)
//                 finds the bin b1
//                 holding the K-th largest key from the row's histogram; keys
//                 above b1 are selected outright, keys in b1 become candidates;
//                 the workgroup reserves its output ranges with one pair of
//                 global atomics
//   4. finalize   one workgroup per row stages the candidates in LDS, goes on
//                 with the radix select over them (key bits 20..10, then 9..0),
//                 sends ties at the threshold to the lower token (radix select
//                 on the token index), and writes the K tokens in ascending
//                 order: an LDS bitmap per 786432 tokens, each selected token
//                 placed by the popcounts before it.
// Passes 3 and 4 stay separate kernels: handing a row from many workgroups to
// one inside a kernel needs a device-scope release per workgroup, which on a
// multi-die GPU writes back L2 and costs far more than a kernel boundary.
// A row is not finished by one workgroup from the start either: at 2^17 tokens
// per row the per-token work alone keeps one CU busy for tens of microseconds.
// The selection is exact: the same tokens as a full sort by (score desc,
// token asc), written in ascending token order, -1 padded for short rows.
#include "hs_common.h"
#include "hs_launch.h"
#include "topk_select.h"

namespace hs {
namespace {

using namespace topk_sel;

// The same search from the top over a row's 2048-bin histogram in global
// memory, by one wave: lane l reads bins 32l .. 32l+31 (eight 16-byte loads),
// a suffix sum over the lanes places each lane's range, and the lane holding
// the k-th largest key walks its bins.  Only the finding lane writes.
__device__ void wave_find_bin_top(const uint32_t* __restrict__ hrow, uint32_t k, int* d_out,
                                  uint32_t* before_out) {
  const int lane = lane_id();
  uint4 q[8];
  const uint4* src = reinterpret_cast<const uint4*>(hrow) + lane * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = src[j];
  uint32_t c[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    c[4 * j] = q[j].x;
    c[4 * j + 1] = q[j].y;
    c[4 * j + 2] = q[j].z;
    c[4 * j + 3] = q[j].w;
  }
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) local += c[j];
  // sum over the lanes above this one (higher bins come first): the wave total
  // less the inclusive prefix (DPP scan; the whole wave is active here)
  const int pre = wave_inclusive_scan_i32((int)local);
  uint32_t before = (uint32_t)(__builtin_amdgcn_readlane(pre, kWave - 1) - pre);
  if (before < k && before + local >= k) {
#pragma unroll
    for (int j = 31; j >= 0; --j) {
      if (before < k && before + c[j] >= k) {
        *d_out = lane * 32 + j;
        *before_out = before;
      }
      before += c[j];
    }
  }
}

__global__ __launch_bounds__(kScanNT) void topk_zero_kernel(TopkWs ws) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < kBins1; i += kScanNT) ws.hist[(size_t)r * kBins1 + i] = 0;
  if (threadIdx.x < kCnt) ws.cnt[r * kCnt + threadIdx.x] = 0;
}

__global__ __launch_bounds__(kScanNT) void topk_hist_kernel(const int32_t* __restrict__ ctx_len,
                                                            int P, int T_stride, int K,
                                                            const float* __restrict__ scores,
                                                            TopkWs ws) {
  constexpr int kPer = kChunk / kScanNT;
  __shared__ uint32_t h[kBins1];
  const int r = blockIdx.y;
  const int n = row_visible(ctx_len, P, r);
  const int base = blockIdx.x * kChunk;
  if (n <= K || base >= n) return;
  for (int i = threadIdx.x; i < kBins1; i += kScanNT) h[i] = 0;
  const float* row = scores + (size_t)r * T_stride;
  const int end = min(base + kChunk, n);
  uint32_t bins[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int t = base + i * kScanNT + threadIdx.x;
    bins[i] = t < end ? (score_key(row[t]) >> 21) : 0xFFFFFFFFu;
  }
  __syncthreads();
  // all loads were issued above; only the LDS adds remain
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (bins[i] != 0xFFFFFFFFu) atomicAdd(&h[bins[i]], 1u);
  __syncthreads();
  // adjacent bins in pairs, one 64-bit atomic per non-empty pair (same-address
  // atomics from every die serialize; a bin never exceeds 2^24)
  for (int i = threadIdx.x; i < kBins1 / 2; i += kScanNT)
    if (h[2 * i] | h[2 * i + 1])
      atomicAdd(reinterpret_cast<unsigned long long*>(ws.hist + (size_t)r * kBins1 + 2 * i),
                (unsigned long long)h[2 * i] | ((unsigned long long)h[2 * i + 1] << 32));
}

// FCH tokens per workgroup: 4096, or 8192 on rows longer than 2^18 tokens so
// that at most 128 workgroups per row share the row's two output counters
// (same-address atomics from every die serialize).
template <int FCH>
__global__ __launch_bounds__(kScanNT) void topk_filter_kernel(const int32_t* __restrict__ ctx_len,
                                                              int P, int T_stride, int K,
                                                              const float* __restrict__ scores,
                                                              TopkWs ws) {
  __shared__ int s_b1;
  __shared__ uint32_t s_above;
  __shared__ int s_wsum[kScanNT / kWave];
  __shared__ uint32_t s_base_sel, s_base_cand;
  const int r = blockIdx.y;
  const int n = row_visible(ctx_len, P, r);
  constexpr int kFPer = FCH / kScanNT / 4;   // 16-byte loads per thread
  const int base = blockIdx.x * FCH;
  if (n <= K || base >= n) return;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wid = tid / kWave;
  const float* row = scores + (size_t)r * T_stride;
  // 16 consecutive-in-lane-order tokens per thread, as four 16-byte loads
  // (rows are 256-byte aligned and padded to a multiple of 64 tokens)
  float4 v[kFPer];
#pragma unroll
  for (int u = 0; u < kFPer; ++u) {
    const int t = base + (u * kScanNT + tid) * 4;
    if (t < n) v[u] = *reinterpret_cast<const float4*>(row + t);
  }
  if (wid == 0) {
    // defined values if the histogram holds fewer than K keys (it cannot, unless
    // the workspace was not zero on entry)
    if (lane == 0) {
      s_b1 = 0;
      s_above = 0;
    }
    wave_find_bin_top(ws.hist + (size_t)r * kBins1, (uint32_t)K, &s_b1, &s_above);
  }
  __syncthreads();
  const uint32_t b1 = (uint32_t)s_b1;
  if (blockIdx.x == 0 && tid == 0) {
    ws.cnt[r * kCnt + 2] = b1;
    ws.cnt[r * kCnt + 3] = s_above;
  }
  uint32_t key[kFPer * 4];
  int packed = 0;            // selections (low 16 bits), candidates (high 16 bits)
#pragma unroll
  for (int u = 0; u < kFPer; ++u) {
    const int t0 = base + (u * kScanNT + tid) * 4;
    const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = t0 + e < n ? score_key(f[e]) : 0u;   // key 0: never kept
      key[u * 4 + e] = k;
      const uint32_t bin = k >> 21;
      packed += (t0 + e < n) ? ((bin > b1) ? 1 : ((bin == b1) ? 0x10000 : 0)) : 0;
    }
  }
  // block exclusive prefix of the packed counts: DPP wave scan, then wave sums
  const int incl = wave_inclusive_scan_i32(packed);
  if (lane == kWave - 1) s_wsum[wid] = incl;
  __syncthreads();
  if (tid == 0) {
    int total = 0;
    for (int w = 0; w < kScanNT / kWave; ++w) {
      const int x = s_wsum[w];
      s_wsum[w] = total;
      total += x;
    }
    // both ranges with one 64-bit atomic on the adjacent counter pair (selections
    // in the low word, candidates in the high word; neither can carry into the
    // other): same-address atomics from every die serialize, so one per
    // workgroup instead of two
    const uint64_t inc = (uint64_t)(total & 0xFFFF) | ((uint64_t)((uint32_t)total >> 16) << 32);
    uint64_t old = 0;
    if (inc)
      old = atomicAdd(reinterpret_cast<unsigned long long*>(ws.cnt + r * kCnt),
                      (unsigned long long)inc);
    s_base_sel = (uint32_t)old;
    s_base_cand = (uint32_t)(old >> 32);
  }
  __syncthreads();
  if (!packed) return;
  const int ex = s_wsum[wid] + incl - packed;
  uint32_t ps = s_base_sel + (uint32_t)(ex & 0xFFFF);
  uint32_t pc = s_base_cand + (uint32_t)(ex >> 16);
  int32_t* sel = ws.sel + (size_t)r * K;
  uint32_t* ck = ws.ckey + (size_t)r * T_stride;
  int32_t* ct = ws.ctok + (size_t)r * T_stride;
#pragma unroll
  for (int u = 0; u < kFPer; ++u) {
    const int t0 = base + (u * kScanNT + tid) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = t0 + e;
      if (t >= n) continue;
      const uint32_t k = key[u * 4 + e];
      const uint32_t bin = k >> 21;
      // the bounds hold whenever the histogram is the row's (kept even if the
      // workspace was not zero on entry, so that no write leaves the row)
      if (bin > b1) {
        if (ps < (uint32_t)K) sel[ps] = t;
        ++ps;
      } else if (bin == b1) {
        if (pc < (uint32_t)T_stride) {
          ck[pc] = k;
          ct[pc] = t;
        }
        ++pc;
      }
    }
  }
}

// Finishes row blockIdx.x (see finalize_row).
__global__ __launch_bounds__(kFinNT) void topk_finalize_kernel(const int32_t* __restrict__ ctx_len,
                                                               int P, int T_stride, int K,
                                                               TopkWs ws, int32_t* __restrict__ topk) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kFinLdsBytes];
  finalize_row(blockIdx.x, ctx_len, P, T_stride, K, ws, topk, lds);
}

}  // namespace

size_t topk_workspace_bytes(int B, int P, int T_stride, int K) {
  const size_t R = (size_t)B * P;
  return align256(R * kBins1 * 4) + align256(R * kCnt * 4) + align256(R * K * 4) +
         align256(R * T_stride * 4) + align256(R * T_stride * 4);
}

hipError_t launch_topk(const BatchDims& d, int K, const float* scores, int32_t* topk, void* ws,
                       hipStream_t s) {
  const int R = d.B * d.P;
  TopkWs w = topk_ws(ws, R, d.T_stride, K);
  const int nchunk = (d.T_stride + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(topk_zero_kernel, dim3(R), dim3(kScanNT), 0, s, w);
  hipLaunchKernelGGL(topk_hist_kernel, dim3(nchunk, R), dim3(kScanNT), 0, s, d.ctx_len, d.P,
                     d.T_stride, K, scores, w);
  return launch_topk_select(d, K, scores, topk, ws, s);
}

hipError_t launch_topk_hist(const BatchDims& d, int K, const float* scores, void* ws,
                            hipStream_t s) {
  const int R = d.B * d.P;
  TopkWs w = topk_ws(ws, R, d.T_stride, K);
  const int nchunk = (d.T_stride + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(topk_hist_kernel, dim3(nchunk, R), dim3(kScanNT), 0, s, d.ctx_len, d.P,
                     d.T_stride, K, scores, w);
  return hipGetLastError();
}

uint32_t* topk_histograms(void* ws) { return static_cast<uint32_t*>(ws); }

hipError_t launch_topk_zero(const BatchDims& d, int K, void* ws, uint32_t** hist, hipStream_t s) {
  const int R = d.B * d.P;
  TopkWs w = topk_ws(ws, R, d.T_stride, K);
  *hist = w.hist;
  hipLaunchKernelGGL(topk_zero_kernel, dim3(R), dim3(kScanNT), 0, s, w);
  return hipGetLastError();
}

hipError_t launch_topk_select(const BatchDims& d, int K, const float* scores, int32_t* topk,
                              void* ws, hipStream_t s) {
  const int R = d.B * d.P;
  TopkWs w = topk_ws(ws, R, d.T_stride, K);
  hipError_t e = launch_topk_filter(d, K, scores, ws, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_finalize_kernel, dim3(R), dim3(kFinNT), 0, s, d.ctx_len, d.P,
                     d.T_stride, K, w, topk);
  return hipGetLastError();
}

hipError_t launch_topk_finalize(const BatchDims& d, int K, int32_t* topk, void* ws,
                                hipStream_t s) {
  const int R = d.B * d.P;
  TopkWs w = topk_ws(ws, R, d.T_stride, K);
  hipLaunchKernelGGL(topk_finalize_kernel, dim3(R), dim3(kFinNT), 0, s, d.ctx_len, d.P,
                     d.T_stride, K, w, topk);
  return hipGetLastError();
}

hipError_t launch_topk_filter(const BatchDims& d, int K, const float* scores, void* ws,
                              hipStream_t s) {
  const int R = d.B * d.P;
  TopkWs w = topk_ws(ws, R, d.T_stride, K);
  if (d.T_stride > 64 * kFChunk) {
    const int nchunk = (d.T_stride + kFChunkLong - 1) / kFChunkLong;
    hipLaunchKernelGGL(topk_filter_kernel<kFChunkLong>, dim3(nchunk, R), dim3(kScanNT), 0, s,
                       d.ctx_len, d.P, d.T_stride, K, scores, w);
  } else if ((size_t)R * ((d.T_stride + kFChunk - 1) / kFChunk) < 256) {
    const int nchunk = (d.T_stride + kFChunkShort - 1) / kFChunkShort;
    hipLaunchKernelGGL(topk_filter_kernel<kFChunkShort>, dim3(nchunk, R), dim3(kScanNT), 0, s,
                       d.ctx_len, d.P, d.T_stride, K, scores, w);
  } else {
    const int nchunk = (d.T_stride + kFChunk - 1) / kFChunk;
    hipLaunchKernelGGL(topk_filter_kernel<kFChunk>, dim3(nchunk, R), dim3(kScanNT), 0, s,
                       d.ctx_len, d.P, d.T_stride, K, scores, w);
  }
  return hipGetLastError();
}

}  // namespace hs
