// Top-K selection pieces shared by the top-K kernels and the fused
// selection + resolve kernel: the workspace layout, the bin searches, the
// exact threshold among the candidates and the finalize of one row (see
// topk.hip for the whole selection).
#pragma once

#include "hs_common.h"

namespace hs {
namespace topk_sel {

constexpr int kBins1 = 2048;   // top 11 key bits
constexpr int kChunk = 8192;   // tokens per workgroup of the histogram pass
constexpr int kFChunk = 4096;  // tokens per workgroup of the filter pass (rows up to 2^18)
constexpr int kFChunkLong = 8192;    // the same for longer rows
constexpr int kFChunkShort = 1024;   // the same when few rows would leave the chip idle
constexpr int kScanNT = 256;
constexpr int kMaxK = 8192;
constexpr int kCnt = 8;                   // counters per row
constexpr int kFinNT = 1024;
constexpr int kFinCand = 12288;           // candidates staged in LDS by finalize

struct TopkWs {
  uint32_t* hist;   // [R][2048]
  uint32_t* cnt;    // [R][8]: selected-above count, candidate count, b1, count above b1
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

constexpr size_t kFinLdsBytes = 4 * ((size_t)kBins1 + kMaxK + 2 * (size_t)kFinCand);

// Finishes row r (n > K visible tokens) from the outright selections and the
// candidates written by every filter workgroup of the row, with kFinNT
// threads.  The caller provides the large LDS arrays (kFinLdsBytes bytes:
// h[kBins1], outl[kMaxK], s_cand[2 * kFinCand], in that order), so that a
// kernel that runs more work after the selection can reuse them.
__device__ __forceinline__ void finalize_row(int r, const int32_t* __restrict__ ctx_len, int P,
                                             int T_stride, int K, TopkWs ws,
                                             int32_t* __restrict__ topk, unsigned char* lds) {
  uint32_t* h = reinterpret_cast<uint32_t*>(lds);
  int32_t* outl = reinterpret_cast<int32_t*>(lds + 4 * kBins1);
  uint32_t* s_cand = reinterpret_cast<uint32_t*>(lds + 4 * (kBins1 + kMaxK));   // candidate keys, then tokens; later the bitmap
  uint32_t* s_ck = s_cand;
  int32_t* s_ct = reinterpret_cast<int32_t*>(s_cand + kFinCand);
  __shared__ int scratch[kFinNT / kWave + 1];
  __shared__ int s_d, s_pos, s_stage;
  __shared__ uint32_t s_before;
  const int tid = threadIdx.x;
  const int n = row_visible(ctx_len, P, r);
  int32_t* out = topk + (size_t)r * K;
  uint32_t* gk = ws.ckey + (size_t)r * T_stride;
  int32_t* gt = ws.ctok + (size_t)r * T_stride;
  int32_t* sel = ws.sel + (size_t)r * K;
  // Everything the call wrote into the row's part of the workspace is dead once
  // read, and is zeroed for the next call: the histogram and counters, the
  // outright selections and the candidates (every filter workgroup of the row
  // finished before this kernel began).  A workspace zeroed once therefore
  // comes back zero from every call, whatever the batch geometry of the next.
  auto clear_row = [&](int nc_written) {
    for (int i = tid; i < kBins1 / 4; i += kFinNT)
      reinterpret_cast<uint4*>(ws.hist + (size_t)r * kBins1)[i] = make_uint4(0, 0, 0, 0);
    if (tid < kCnt) ws.cnt[r * kCnt + tid] = 0;
    for (int i = tid; i < K; i += kFinNT) sel[i] = 0;
    for (int i = tid; i < nc_written; i += kFinNT) {
      gk[i] = 0u;
      gt[i] = 0;
    }
  };
  if (n <= K) {
    for (int k = tid; k < K; k += kFinNT) out[k] = k < n ? k : -1;
    clear_row(0);
    return;
  }
  // counts are clamped to the row's buffers (they hold whenever the workspace
  // was zero on entry; the clamps keep every access inside the row otherwise)
  const uint32_t b1 = ws.cnt[r * kCnt + 2];
  const uint32_t above = min(ws.cnt[r * kCnt + 3], (uint32_t)K);
  const int nc = (int)min(ws.cnt[r * kCnt + 1], (uint32_t)T_stride);
  // the outright selections and (when they fit) the candidates go to LDS with
  // one round of independent loads: every load is issued before the first one
  // is used (indices past the end are clamped and their values dropped)
  // loops over global memory issue kLd independent loads per thread before
  // using any of them (the candidates' order does not matter to the result)
  constexpr int kLd = 8;
  static_assert(kLd * kFinNT >= kMaxK, "one round of loads covers the outright selections");
  constexpr int kStage = kFinCand / kFinNT;
  static_assert(kStage * kFinNT == kFinCand, "one round of loads stages every candidate in LDS");
  const bool in_lds = nc <= kFinCand;
  {
    int32_t sx[kLd];
    uint32_t kx[kStage];
    int32_t tx[kStage];
#pragma unroll
    for (int u = 0; u < kLd; ++u) sx[u] = sel[min(tid + u * kFinNT, max((int)above - 1, 0))];
    if (in_lds) {
      const int last = max(nc - 1, 0);
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int i = min(tid + u * kFinNT, last);
        kx[u] = gk[i];
        tx[u] = gt[i];
      }
    }
#pragma unroll
    for (int u = 0; u < kLd; ++u)
      if (tid + u * kFinNT < (int)above) outl[tid + u * kFinNT] = sx[u];
    if (in_lds) {
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int i = tid + u * kFinNT;
        if (i < nc) {
          s_ck[i] = kx[u];
          s_ct[i] = tx[u];
        }
      }
    }
  }
  if (tid == 0) {
    s_pos = (int)above;
    s_stage = 0;                  // staging cursor of the two-pass path below
    s_d = 0;                      // bin searches leave these unchanged if they find
    s_before = 0;                 // nothing (only with a workspace not zero on entry)
  }
  __syncthreads();
  const int lane = lane_id();
  // chosen candidates join the outright selections: one ballot and one LDS
  // atomic per wave (same-address atomics from every thread serialize)
  auto push = [&](bool chosen, int t) {
    const uint64_t m = __ballot(chosen);
    if (m) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_pos, __popcll(m));
      base = __shfl(base, 0);
      const int at = base + lanes_below(m);
      if (chosen && at < kMaxK) outl[at] = t;
    }
  };
  const uint32_t* ck = in_lds ? s_ck : gk;
  const int32_t* ct = in_lds ? s_ct : gt;
  int nsel = nc;                  // candidates the threshold search runs over
  uint32_t kk = (uint32_t)K - above;
  if (!in_lds) {
    // Too many candidates for LDS: one pass over global memory bins them by
    // key bits 20..10 and finds the sub-bin dA holding the kk-th largest key;
    // a second pass selects the candidates above dA outright and stages those
    // in dA in LDS (their number is the bin's count), and the search goes on
    // over the staged set.  A sub-bin too large for LDS keeps every pass in
    // global memory.
    for (int i = tid; i < kBins1; i += kFinNT) h[i] = 0;
    __syncthreads();
    for (int i0 = tid; i0 < nc; i0 += kLd * kFinNT) {
      uint32_t kx[kLd];
#pragma unroll
      for (int u = 0; u < kLd; ++u) kx[u] = gk[min(i0 + u * kFinNT, nc - 1)];
#pragma unroll
      for (int u = 0; u < kLd; ++u)
        if (i0 + u * kFinNT < nc) atomicAdd(&h[(kx[u] >> 10) & 0x7FFu], 1u);
    }
    __syncthreads();
    find_bin<kFinNT>(h, kBins1, kk, true, scratch, &s_d, &s_before);
    const uint32_t dA = (uint32_t)s_d;
    const int n2 = (int)h[dA];
    if (n2 <= kFinCand) {
      kk -= s_before;
      // every thread runs the same number of batches (the ballots need whole waves)
      const int nc_up = (nc + kLd * kFinNT - 1) / (kLd * kFinNT) * (kLd * kFinNT);
      for (int i0 = tid; i0 < nc_up; i0 += kLd * kFinNT) {
        uint32_t kx[kLd];
        int32_t tx[kLd];
#pragma unroll
        for (int u = 0; u < kLd; ++u) {
          const int i = min(i0 + u * kFinNT, nc - 1);
          kx[u] = gk[i];
          tx[u] = gt[i];
        }
#pragma unroll
        for (int u = 0; u < kLd; ++u) {
          const bool valid = i0 + u * kFinNT < nc;
          const uint32_t key = kx[u];
          const int t = tx[u];
          const uint32_t sub = (key >> 10) & 0x7FFu;
          push(valid && sub > dA, t);
          const bool stage = valid && sub == dA;
          const uint64_t m = __ballot(stage);
          if (m) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&s_stage, __popcll(m));
            base = __shfl(base, 0);
            if (stage) {
              const int at = base + lanes_below(m);
              s_ck[at] = key;
              s_ct[at] = t;
            }
          }
        }
      }
      __syncthreads();
      ck = s_ck;
      ct = s_ct;
      nsel = n2;
    }
    __syncthreads();
  }
  uint32_t tau;
  int t_cut;
  candidates_threshold<kFinNT>(ck, ct, nsel, b1, kk, h, scratch, &s_d, &s_before, &tau, &t_cut);
  const int ns_up = (nsel + kFinNT - 1) / kFinNT * kFinNT;
  for (int i = tid; i < ns_up; i += kFinNT) {
    bool chosen = false;
    int t = 0;
    if (i < nsel) {
      const uint32_t key = ck[i];
      t = ct[i];
      chosen = key > tau || (key == tau && t <= t_cut);
    }
    push(chosen, t);
  }
  __syncthreads();
  // emit the K selected tokens in ascending order: an LDS bitmap laid over the
  // (now dead) candidate list, one pass per 786432 tokens of the row.  Thread j
  // owns a run of wpt bitmap words; a block scan of the runs' popcounts goes to
  // LDS, and each selected token finds its own output index as its run's
  // prefix plus the popcounts of the words before it in the run, so the work
  // per thread stays even however the selection clusters.
  // Runs are whole 16-byte groups of words (wpt a multiple of 4), so a run's
  // popcounts and a token's count of the set bits before it in its run come
  // from independent 16-byte LDS reads; the last group's words past the pass's
  // tokens are zero, and groups past it are never read.
  constexpr int kBmWords = 2 * kFinCand;
  constexpr int kBmTok = kBmWords * 32;
  constexpr int kMaxQ = kBmWords / kFinNT / 4;   // 16-byte groups per run, at most
  static_assert(kBmWords % (4 * kFinNT) == 0 && kFinNT <= kBins1, "runs fit the prefix array");
  uint32_t* bmw = s_cand;
  const uint4* bmq = reinterpret_cast<const uint4*>(s_cand);
  uint32_t* run_pre = h;                    // the radix histogram is dead by now
  auto popc4 = [](uint4 x) { return __popc(x.x) + __popc(x.y) + __popc(x.z) + __popc(x.w); };
  int written = 0;
  for (int seg0 = 0; seg0 < n; seg0 += kBmTok) {
    const int nwords = (min(kBmTok, n - seg0) + 31) / 32;
    const int qpt = (nwords + 4 * kFinNT - 1) / (4 * kFinNT);   // groups per run, <= kMaxQ
    const int ngroups = (nwords + 3) / 4;
    for (int i = tid; i < 4 * ngroups; i += kFinNT) bmw[i] = 0u;
    __syncthreads();
    for (int i = tid; i < K; i += kFinNT) {
      const int t = outl[i] - seg0;
      if (t >= 0 && t < kBmTok) atomicOr(&bmw[t >> 5], 1u << (t & 31));
    }
    __syncthreads();
    int c = 0;
#pragma unroll
    for (int q = 0; q < kMaxQ; ++q)
      if (q < qpt && tid * qpt + q < ngroups) c += popc4(bmq[tid * qpt + q]);
    int tot;
    run_pre[tid] = (uint32_t)block_exclusive_scan<kFinNT>(c, scratch, &tot);
    __syncthreads();
    for (int i = tid; i < K; i += kFinNT) {
      const int t = outl[i] - seg0;
      if (t < 0 || t >= kBmTok) continue;
      const int w = t >> 5;
      const int run = w / (4 * qpt);
      const int dw = w - run * 4 * qpt;                 // words of the run before w
      int rank = (int)run_pre[run] + __popc(bmw[w] & ((1u << (t & 31)) - 1u));
#pragma unroll
      for (int q = 0; q < kMaxQ; ++q) {
        if (4 * q >= dw) continue;
        const uint4 x = bmq[run * qpt + q];
        const int k = dw - 4 * q;                      // words of this group before w
        rank += __popc(x.x) + (k > 1 ? __popc(x.y) : 0) + (k > 2 ? __popc(x.z) : 0) +
                (k > 3 ? __popc(x.w) : 0);
      }
      out[written + rank] = outl[i];
    }
    written += tot;
    __syncthreads();   // the next pass rewrites the bitmap and the run prefixes
  }
  clear_row(nc);
}


}  // namespace topk_sel
}  // namespace hs
