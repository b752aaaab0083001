// Exact top-K per query position on gfx950 (K best tokens of the indexer,
// page "Un contexte d'un million sur huit H200", section "Ce qui se passe";
// K = 2048 on "vLLM sert GLM-5.3 en contexte 1M sur 16 H200", section
// "Comment s'y prendre").
//
// Scores map to order-preserving uint32 keys.  A row (one request position,
// up to 2^24 tokens) is spread over many workgroups so that a handful of very
// long rows still fills the chip:
//   1. zero       per-row histogram and counters
//   2. histogram  of the top 11 key bits, per 8192-token chunk: LDS counts,
//                 then one global atomic per non-empty bin (the fused path of
//                 hs_indexer_topk builds it in the indexer's epilogue instead)
//   3. filter     every chunk re-derives the bin b1 holding the K-th largest
//                 key; keys above b1 are selected outright, keys in b1 become
//                 candidates (one global append per workgroup)
//   4. finalize   one workgroup per row goes on with the radix select over
//                 the candidates (11 + 10 more bits), sends ties at the
//                 threshold to the lower token (radix select on the token
//                 index), and writes the K tokens in ascending order through
//                 an LDS bitmap per 64K-token segment.
// Passes 3 and 4 stay separate kernels: handing a row from many workgroups to
// one inside a kernel needs a device-scope release per workgroup, which on a
// multi-die GPU writes back L2 and costs far more than a kernel boundary.
// Rows of at most 2^18 tokens skip that hand-off: one 1024-thread workgroup per
// row streams the row once (keys above the threshold bin go straight into an
// LDS bitmap, keys in it into an LDS candidate list), finishes the radix select
// and emits from the bitmap -- one kernel after the histogram instead of two,
// and no candidate round trip through HBM.
// The selection is exact: the same tokens as a full sort by (score desc,
// token asc), written in ascending token order, -1 padded for short rows.
#include "hs_common.h"
#include "hs_launch.h"

namespace hs {
namespace {

constexpr int kBins1 = 2048;   // top 11 key bits
constexpr int kChunk = 8192;   // tokens per workgroup in passes 2 and 3
constexpr int kScanNT = 256;
constexpr int kMaxK = 8192;
constexpr int kCnt = 8;                   // counters per row
constexpr int kFinNT = 1024;
constexpr int kSegTok = 1 << 16;          // tokens per bitmap segment in finalize
constexpr int kSegWords = kSegTok / 32;
constexpr int kSelNT = 1024;
constexpr int kSelMaxN = 1 << 18;         // longest row of the one-workgroup select
constexpr int kSelWords = kSelMaxN / 32;
constexpr int kSelCand = 12288;           // candidates held in LDS (else in the workspace)
constexpr int kSelU = 8;                  // 16-byte score loads per thread per round

struct TopkWs {
  uint32_t* hist;   // [R][2048]
  uint32_t* cnt;    // [R][8]: selected-above count, candidate count, b1, count above b1,
                    //         finished-chunk ticket
  int32_t* sel;     // [R][K]
  uint32_t* ckey;   // [R][T_stride]
  int32_t* ctok;    // [R][T_stride]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline TopkWs topk_ws(void* base, int R, int T_stride, int K) {
  char* p = static_cast<char*>(base);
  TopkWs w;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)R * kBins1 * 4);
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)R * kCnt * 4);
  w.sel = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)R * K * 4);
  w.ckey = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)R * T_stride * 4);
  w.ctok = reinterpret_cast<int32_t*>(p);
  return w;
}

__device__ __forceinline__ int row_visible(const int32_t* ctx_len, int P, int r) {
  const int b = r / P, p = r % P;
  return max(ctx_len[b] - P + p + 1, 0);
}

// Finds the bin d with before(d) < k <= before(d) + h[d], where before(d) sums
// the bins preceding d in scan order (descending bins when from_top).  Bins in
// LDS; the result is written to *d_out / *before_out by the one thread that
// finds it.  Every thread of the block must call it.
template <int NT>
__device__ void find_bin(const uint32_t* h, int nbins, uint32_t k, bool from_top, int* scratch,
                         int* d_out, uint32_t* before_out) {
  const int bpt = nbins >= NT ? nbins / NT : 1;
  const int owners = nbins / bpt;
  const int tid = threadIdx.x;
  uint32_t local = 0;
  if (tid < owners)
    for (int j = 0; j < bpt; ++j) {
      const int pos = tid * bpt + j;
      local += h[from_top ? nbins - 1 - pos : pos];
    }
  int total;
  const uint32_t excl = (uint32_t)block_exclusive_scan<NT>((int)local, scratch, &total);
  if (tid < owners) {
    uint32_t before = excl;
    for (int j = 0; j < bpt; ++j) {
      const int pos = tid * bpt + j;
      const int bin = from_top ? nbins - 1 - pos : pos;
      const uint32_t c = h[bin];
      if (before < k && before + c >= k) {
        *d_out = bin;
        *before_out = before;
      }
      before += c;
    }
  }
  __syncthreads();
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
  for (int i = threadIdx.x; i < kBins1; i += kScanNT)
    if (h[i]) atomicAdd(&ws.hist[(size_t)r * kBins1 + i], h[i]);
}

// Exact threshold among the candidates ck/ct[0, nc) (every key has top bits
// b1): tau = the kk-th largest key (bits 20..10, then 9..0), and t_cut = the
// largest token kept among keys equal to tau (ties go to lower tokens;
// INT_MAX when all of them are kept).  Returned in every thread.
template <int NT>
__device__ void candidates_threshold(const uint32_t* ck, const int32_t* ct, int nc, uint32_t b1,
                                     uint32_t kk, uint32_t* h, int* scratch, int* s_d,
                                     uint32_t* s_before, uint32_t* tau_out, int* t_cut_out) {
  const int tid = threadIdx.x;
  // key bits 20..10
  for (int i = tid; i < kBins1; i += NT) h[i] = 0;
  __syncthreads();
  for (int i = tid; i < nc; i += NT) atomicAdd(&h[(ck[i] >> 10) & 0x7FFu], 1u);
  __syncthreads();
  find_bin<NT>(h, kBins1, kk, true, scratch, s_d, s_before);
  const uint32_t dA = (uint32_t)*s_d;
  kk -= *s_before;
  // key bits 9..0
  for (int i = tid; i < 1024; i += NT) h[i] = 0;
  __syncthreads();
  for (int i = tid; i < nc; i += NT) {
    const uint32_t key = ck[i];
    if (((key >> 10) & 0x7FFu) == dA) atomicAdd(&h[key & 0x3FFu], 1u);
  }
  __syncthreads();
  find_bin<NT>(h, 1024, kk, true, scratch, s_d, s_before);
  const uint32_t dB = (uint32_t)*s_d;
  kk -= *s_before;                       // ties at the threshold to take
  const uint32_t n_eq = h[dB];
  const uint32_t tau = (b1 << 21) | (dA << 10) | dB;
  __syncthreads();
  // ties: keep the kk lowest tokens among keys == tau
  int t_cut = 0x7FFFFFFF;
  if (n_eq > kk) {
    uint32_t prefix = 0, need = kk;
    for (int sh = 16; sh >= 0; sh -= 8) {
      for (int i = tid; i < 256; i += NT) h[i] = 0;
      __syncthreads();
      for (int i = tid; i < nc; i += NT) {
        if (ck[i] != tau) continue;
        const uint32_t t = (uint32_t)ct[i];
        if (sh == 16 || (t >> (sh + 8)) == prefix) atomicAdd(&h[(t >> sh) & 0xFFu], 1u);
      }
      __syncthreads();
      find_bin<NT>(h, 256, need, false, scratch, s_d, s_before);
      prefix = (prefix << 8) | (uint32_t)*s_d;
      need -= *s_before;
      __syncthreads();
    }
    t_cut = (int)prefix;
  }
  *tau_out = tau;
  *t_cut_out = t_cut;
}

// Writes the set bits of bm[0, nwords) as ascending tokens t_base + bit to
// out[written ...]; returns the number written.  Every thread must call it.
template <int NT, int WPT>
__device__ int emit_bitmap(const uint32_t* bm, int nwords, int t_base, int written,
                           int32_t* __restrict__ out, int* scratch) {
  const int tid = threadIdx.x;
  uint32_t wd[WPT];
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int w = tid * WPT + j;
    wd[j] = w < nwords ? bm[w] : 0u;
    cnt += __popc(wd[j]);
  }
  int tot;
  int pos = written + block_exclusive_scan<NT>(cnt, scratch, &tot);
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    uint32_t x = wd[j];
    const int t0 = t_base + (tid * WPT + j) * 32;
    while (x) {
      const int bit = __ffs(x) - 1;
      out[pos++] = t0 + bit;
      x &= x - 1;
    }
  }
  return tot;
}

// Finishes row r (n > K visible tokens) from the outright selections and the
// candidates written by every chunk of the row.
template <int NT>
__device__ void finalize_row(int r, int n, int T_stride, int K, const TopkWs& ws,
                             int32_t* __restrict__ out, uint32_t* h, int32_t* outl, uint32_t* bm,
                             int* scratch, int* s_d, uint32_t* s_before, int* s_pos) {
  const int tid = threadIdx.x;
  const uint32_t b1 = ws.cnt[r * kCnt + 2];
  const uint32_t above = ws.cnt[r * kCnt + 3];
  const int nc = (int)ws.cnt[r * kCnt + 1];
  const uint32_t* ck = ws.ckey + (size_t)r * T_stride;
  const int32_t* ct = ws.ctok + (size_t)r * T_stride;
  uint32_t tau;
  int t_cut;
  candidates_threshold<NT>(ck, ct, nc, b1, (uint32_t)K - above, h, scratch, s_d, s_before, &tau,
                           &t_cut);
  // collect: the tokens selected outright, then the chosen candidates
  const int32_t* sel = ws.sel + (size_t)r * K;
  for (int i = tid; i < (int)above; i += NT) outl[i] = sel[i];
  if (tid == 0) *s_pos = (int)above;
  __syncthreads();
  for (int i = tid; i < nc; i += NT) {
    const uint32_t key = ck[i];
    const int t = ct[i];
    if (key > tau || (key == tau && t <= t_cut)) {
      const int at = atomicAdd(s_pos, 1);
      if (at < kMaxK) outl[at] = t;
    }
  }
  __syncthreads();
  // emit the K selected tokens in ascending order: an LDS bitmap per 2^16-token
  // segment, then a popcount prefix sum over its words
  int written = 0;
  const int nseg = (n + kSegTok - 1) / kSegTok;
  for (int sg = 0; sg < nseg; ++sg) {
    for (int i = tid; i < kSegWords; i += NT) bm[i] = 0u;
    __syncthreads();
    for (int i = tid; i < K; i += NT) {
      const int t = outl[i];
      if (t / kSegTok == sg) atomicOr(&bm[(t % kSegTok) >> 5], 1u << (t & 31));
    }
    __syncthreads();
    written += emit_bitmap<NT, kSegWords / NT>(bm, kSegWords, sg * kSegTok, written, out, scratch);
  }
}

__global__ __launch_bounds__(kScanNT) void topk_filter_kernel(const int32_t* __restrict__ ctx_len,
                                                              int P, int T_stride, int K,
                                                              const float* __restrict__ scores,
                                                              TopkWs ws) {
  constexpr int kPer = kChunk / kScanNT;   // keys per thread, kept in registers
  __shared__ uint32_t h[kBins1];
  __shared__ int scratch[kScanNT / kWave + 1];
  __shared__ int s_b1;
  __shared__ uint32_t s_above;
  __shared__ uint32_t s_base_sel, s_base_cand;
  const int r = blockIdx.y;
  const int n = row_visible(ctx_len, P, r);
  const int base = blockIdx.x * kChunk;
  if (n <= K || base >= n) return;
  const float* row = scores + (size_t)r * T_stride;
  const int end = min(base + kChunk, n);
  uint32_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int t = base + i * kScanNT + threadIdx.x;
    key[i] = t < end ? score_key(row[t]) : 0u;
  }
  for (int i = threadIdx.x; i < kBins1; i += kScanNT) h[i] = ws.hist[(size_t)r * kBins1 + i];
  __syncthreads();
  find_bin<kScanNT>(h, kBins1, (uint32_t)K, true, scratch, &s_b1, &s_above);
  const uint32_t b1 = (uint32_t)s_b1;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws.cnt[r * kCnt + 2] = b1;
    ws.cnt[r * kCnt + 3] = s_above;
  }
  // count this thread's selections (low 16 bits) and candidates (high 16 bits)
  int packed = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int t = base + i * kScanNT + threadIdx.x;
    const uint32_t bin = key[i] >> 21;
    if (t < end) packed += (bin > b1) ? 1 : ((bin == b1) ? 0x10000 : 0);
  }
  int total;
  const int ex = block_exclusive_scan<kScanNT>(packed, scratch, &total);
  if (threadIdx.x == 0) {
    s_base_sel = (total & 0xFFFF) ? atomicAdd(&ws.cnt[r * kCnt + 0], (uint32_t)(total & 0xFFFF)) : 0u;
    s_base_cand = (total >> 16) ? atomicAdd(&ws.cnt[r * kCnt + 1], (uint32_t)(total >> 16)) : 0u;
  }
  __syncthreads();
  uint32_t ps = s_base_sel + (uint32_t)(ex & 0xFFFF);
  uint32_t pc = s_base_cand + (uint32_t)(ex >> 16);
  int32_t* sel = ws.sel + (size_t)r * K;
  uint32_t* ck = ws.ckey + (size_t)r * T_stride;
  int32_t* ct = ws.ctok + (size_t)r * T_stride;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int t = base + i * kScanNT + threadIdx.x;
    if (t >= end) continue;
    const uint32_t bin = key[i] >> 21;
    if (bin > b1) {
      sel[ps++] = t;
    } else if (bin == b1) {
      ck[pc] = key[i];
      ct[pc] = t;
      ++pc;
    }
  }
}

__global__ __launch_bounds__(kFinNT) void topk_finalize_kernel(const int32_t* __restrict__ ctx_len,
                                                               int P, int T_stride, int K,
                                                               TopkWs ws, int32_t* __restrict__ topk) {
  __shared__ uint32_t h[kBins1];
  __shared__ int32_t outl[kMaxK];
  __shared__ uint32_t bm[kSegWords];
  __shared__ int scratch[kFinNT / kWave + 1];
  __shared__ int s_d, s_pos;
  __shared__ uint32_t s_before;
  const int r = blockIdx.x;
  const int n = row_visible(ctx_len, P, r);
  int32_t* out = topk + (size_t)r * K;
  if (n <= K) {
    for (int k = threadIdx.x; k < K; k += kFinNT) out[k] = k < n ? k : -1;
    return;
  }
  finalize_row<kFinNT>(r, n, T_stride, K, ws, out, h, outl, bm, scratch, &s_d, &s_before, &s_pos);
}

// Filter and finalize of one row (n <= 2^18 visible tokens) in one workgroup,
// from the row's complete 11-bit histogram.
__global__ __launch_bounds__(kSelNT) void topk_select_row_kernel(
    const int32_t* __restrict__ ctx_len, int P, int T_stride, int K,
    const float* __restrict__ scores, TopkWs ws, int32_t* __restrict__ topk) {
  __shared__ uint32_t h[kBins1];
  __shared__ uint32_t bm[kSelWords];
  __shared__ uint32_t s_ck[kSelCand];
  __shared__ int32_t s_ct[kSelCand];
  __shared__ int scratch[kSelNT / kWave + 1];
  __shared__ int s_d, s_nc;
  __shared__ uint32_t s_before;
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const int n = row_visible(ctx_len, P, r);
  int32_t* out = topk + (size_t)r * K;
  if (n <= K) {
    for (int k = tid; k < K; k += kSelNT) out[k] = k < n ? k : -1;
    return;
  }
  const float* row = scores + (size_t)r * T_stride;
  // the first round's 16-byte loads go out before the histogram scan; every
  // round then issues the next round's loads before working on its own
  constexpr int kStep = kSelNT * 4 * kSelU;            // tokens per round
  float4 v[kSelU];
#pragma unroll
  for (int u = 0; u < kSelU; ++u) {
    const int t = (u * kSelNT + tid) * 4;
    if (t < n) v[u] = *reinterpret_cast<const float4*>(row + t);
  }
  for (int i = tid; i < kBins1; i += kSelNT) h[i] = ws.hist[(size_t)r * kBins1 + i];
  const int nwords = (n + 31) >> 5;
  for (int i = tid; i < nwords; i += kSelNT) bm[i] = 0u;
  if (tid == 0) s_nc = 0;
  __syncthreads();
  find_bin<kSelNT>(h, kBins1, (uint32_t)K, true, scratch, &s_d, &s_before);
  const uint32_t b1 = (uint32_t)s_d;
  const uint32_t above = s_before;
  // the histogram gives the candidate count up front: LDS when they fit
  const bool in_lds = h[b1] <= (uint32_t)kSelCand;
  const int cap = in_lds ? kSelCand : T_stride;
  uint32_t* ck = in_lds ? s_ck : ws.ckey + (size_t)r * T_stride;
  int32_t* ct = in_lds ? s_ct : ws.ctok + (size_t)r * T_stride;
  const int lane = lane_id();
  for (int base = 0; base < n; base += kStep) {
    float4 nx[kSelU];
#pragma unroll
    for (int u = 0; u < kSelU; ++u) {
      const int t = base + kStep + (u * kSelNT + tid) * 4;
      if (t < n) nx[u] = *reinterpret_cast<const float4*>(row + t);
    }
#pragma unroll
    for (int u = 0; u < kSelU; ++u) {
      const int t0 = base + (u * kSelNT + tid) * 4;
      const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + e;
        const uint32_t key = score_key(f[e]);
        const uint32_t bin = key >> 21;
        const bool ok = t < n;
        if (ok && bin > b1) atomicOr(&bm[t >> 5], 1u << (t & 31));
        const bool cand = ok && bin == b1;
        const uint64_t m = __ballot(cand);
        if (m) {
          const int leader = __ffsll((long long)m) - 1;
          int basepos = 0;
          if (lane == leader) basepos = atomicAdd(&s_nc, __popcll(m));
          basepos = __shfl(basepos, leader);
          const int at = basepos + lanes_below(m);
          if (cand && at < cap) {
            ck[at] = key;
            ct[at] = t;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kSelU; ++u) v[u] = nx[u];
  }
  __syncthreads();
  const int nc = min(s_nc, cap);
  uint32_t tau;
  int t_cut;
  candidates_threshold<kSelNT>(ck, ct, nc, b1, (uint32_t)K - above, h, scratch, &s_d, &s_before,
                               &tau, &t_cut);
  for (int i = tid; i < nc; i += kSelNT) {
    const uint32_t key = ck[i];
    const int t = ct[i];
    if (key > tau || (key == tau && t <= t_cut)) atomicOr(&bm[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  emit_bitmap<kSelNT, kSelWords / kSelNT>(bm, nwords, 0, 0, out, scratch);
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
  if (d.T_stride <= kSelMaxN) {
    hipLaunchKernelGGL(topk_select_row_kernel, dim3(R), dim3(kSelNT), 0, s, d.ctx_len, d.P,
                       d.T_stride, K, scores, w, topk);
    return hipGetLastError();
  }
  const int nchunk = (d.T_stride + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(topk_filter_kernel, dim3(nchunk, R), dim3(kScanNT), 0, s, d.ctx_len, d.P,
                     d.T_stride, K, scores, w);
  hipLaunchKernelGGL(topk_finalize_kernel, dim3(R), dim3(kFinNT), 0, s, d.ctx_len, d.P,
                     d.T_stride, K, w, topk);
  return hipGetLastError();
}

}  // namespace hs
