// Fused resolve of the selected tokens on gfx950 (page "Un contexte d'un
// million sur huit H200", section "Les trois états de résidence": resident
// tokens are read in place, hot tokens refresh their LRU entry, a fault copies
// a single row from pinned host memory, and no CPU decision sits on the path).
//
// Two kernels, both decided entirely on the device:
//   resolve    one 1024-thread workgroup per request owns that request's
//              tables, so no state is shared between workgroups:
//              1. U = sorted distinct union of the P positions' selections
//                 (each list is sorted: ranks by binary search, then dedup);
//              2. classify U in ascending order: resident page / hot hit
//                 (stamp <- s) / fault, faults compacted in token order;
//              3. victims: the |F| smallest (stamp, slot) keys among slots
//                 with stamp < s, emitted one distinct stamp at a time in slot
//                 order (an MSD radix select plus an LDS sort when they span
//                 many stamps);
//              4. fault i takes victim i: evict, insert, stamp, record;
//              5. row ids of every (position, k) from the updated tables.
//   fault copy a persistent grid takes the faults in small batches, a few
//              requests at a time: each 576-value row is read straight from
//              pinned host memory (zero-copy) and written to its slot's pool
//              row in every layer, with its scale; it also advances the step
//              counter.
#include "hs_common.h"
#include "hs_launch.h"
#include "topk_select.h"

namespace hs {
namespace {

constexpr int kResNT = 1024;
constexpr int kMaxSel = 8192;   // P*K
constexpr int kCopyNT = 256;
constexpr int kCopyWGs = 256;
constexpr int kCopyInFlight = 4;
constexpr int kCopyBatch = 8;        // faults per workgroup batch
constexpr int kCopyMaxL = 16;
constexpr int kCopyCntLds = 4096;    // requests whose fault counts the copy stages in LDS
constexpr int kMaxSlotsPerThread = 16;   // C <= 16384
constexpr int kMaxStampRounds = 32;
constexpr int kMaxEntriesPerThread = kMaxSel / kResNT;   // 8
constexpr int kMaxHotBlocks = 16384 / 64;

__device__ __forceinline__ int lower_bound_lds(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int upper_bound_lds(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Finds the bin d of h[0..256) with before(d) < k <= before(d) + h[d],
// scanning from bin 0 upward (a tiny serial scan by one wave).
__device__ void find_bin256_lo(const uint32_t* h, uint32_t k, int* d_out, uint32_t* before_out) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    uint32_t c[4], loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = h[lane * 4 + j];
      loc += c[j];
    }
    uint32_t x = loc;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    uint32_t before = x - loc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (before < k && before + c[j] >= k) {
        *d_out = lane * 4 + j;
        *before_out = before;
      }
      before += c[j];
    }
  }
  __syncthreads();
}

// Block-wide exclusive prefix sums of NW words at once, each word holding two
// 16-bit counters (no counter's block total exceeds 65535, so no carry crosses
// a field): ex = the sums over earlier threads, tot = the block totals.  buf:
// [NT / 64][NW] words of LDS that nothing touches again before the next
// barrier.  One barrier.
template <int NT, int NW>
__device__ __forceinline__ void block_scan_packed16(const uint32_t (&v)[NW], uint32_t (*buf)[NW],
                                                    uint32_t (&ex)[NW], uint32_t (&tot)[NW]) {
  constexpr int NWV = NT / kWave;
  static_assert(NT % kWave == 0 && NWV >= 1 && NWV <= 16, "one to sixteen whole waves");
  const int lane = lane_id();
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  uint32_t x[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) x[k] = (uint32_t)wave_inclusive_scan_i32((int)v[k]);
  if (lane == kWave - 1)
#pragma unroll
    for (int k = 0; k < NW; ++k) buf[wid][k] = x[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    int ws = lane < NWV ? (int)buf[lane][k] : 0;
    ws += __builtin_amdgcn_update_dpp(0, ws, 0x111, 0xF, 0xF, false);   // row_shr:1
    ws += __builtin_amdgcn_update_dpp(0, ws, 0x112, 0xF, 0xF, false);   // row_shr:2
    ws += __builtin_amdgcn_update_dpp(0, ws, 0x114, 0xF, 0xF, false);   // row_shr:4
    ws += __builtin_amdgcn_update_dpp(0, ws, 0x118, 0xF, 0xF, false);   // row_shr:8
    const uint32_t before = wid ? (uint32_t)__builtin_amdgcn_readlane(ws, wid - 1) : 0u;
    tot[k] = (uint32_t)__builtin_amdgcn_readlane(ws, NWV - 1);
    ex[k] = before + x[k] - v[k];
  }
}

__device__ __forceinline__ int field16(const uint32_t* w, int j) {
  return (int)((w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
}

// NT threads per request (every instance uses 1024: with fewer waves per CU
// the table lookups, bound by how many misses one CU keeps in flight, take
// longer than the per-wave scans save).  MAXS: stamp registers per thread (slots of a
// thread's run, C <= MAXS * NT); MAXE: distinct selected tokens per thread
// (P * K <= MAXE * NT).  The launch
// takes the smallest instance that fits: every per-thread loop is unrolled to
// these bounds, and a latency-bound kernel that runs once per workgroup pays
// for its code size in instruction fetches.  ONE: one query position (P = 1),
// whose list is already U: entry i * 1024 + t stays with thread t from its load
// to its row id, so the table lookups go out as soon as the list arrives.
// FUSED (one position): the workgroup first finishes its row's top-K selection
// (topk_sel::finalize_row, after the filter pass; it writes topk_out and
// returns the selection's workspace row to zero) and then resolves that list,
// read back from topk_out, in the same LDS.  topk is unused then.
template <int NT, int MAXS, int MAXE, bool ONE, bool FUSED>
__global__ __launch_bounds__(NT) void resolve_kernel(
    int T_stride, int max_blocks, int P, int K, const int32_t* __restrict__ topk, int C,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ hot_blocks,
    int32_t* __restrict__ tok2slot, int32_t* __restrict__ slot2tok, int32_t* __restrict__ stamp,
    const int32_t* __restrict__ step, int32_t* __restrict__ err,
    const int64_t* __restrict__ host_bt, int32_t* __restrict__ row_ids,
    int32_t* __restrict__ faults, int32_t* __restrict__ counts,
    const int32_t* __restrict__ ctx_len, topk_sel::TopkWs tws, int32_t* topk_out) {
  static_assert(!FUSED || ONE, "the fused selection serves one query position");
  // R1: merge lists, then victims (slots, or sorted 64-bit keys on the general path).
  // Fused: these three arrays share their LDS with the selection's, which is
  // dead once the row's top-K is written.
  constexpr int kResLds = 16 * kMaxSel;
  constexpr int kFusedLds = kResLds > (int)topk_sel::kFinLdsBytes ? kResLds
                                                                  : (int)topk_sel::kFinLdsBytes;
  __shared__ __attribute__((aligned(16))) uint64_t sA64_[FUSED ? 1 : kMaxSel];
  __shared__ int32_t sU_[FUSED ? 1 : kMaxSel];   // U when P > 1
  __shared__ int32_t sF_[FUSED ? 1 : kMaxSel];   // faulting tokens, ascending
  __shared__ __attribute__((aligned(16))) unsigned char arena[FUSED ? kFusedLds : 16];
  uint64_t* const sA64 = FUSED ? reinterpret_cast<uint64_t*>(arena) : sA64_;
  int32_t* const sU = FUSED ? reinterpret_cast<int32_t*>(arena + 8 * kMaxSel) : sU_;
  int32_t* const sF = FUSED ? reinterpret_cast<int32_t*>(arena + 12 * kMaxSel) : sF_;
  __shared__ int32_t sHot[kMaxHotBlocks];  // this request's hot blocks
  __shared__ uint32_t sHitMask[kMaxHotBlocks * 2];   // slots hit at this step (C bits)
  __shared__ int scratch[NT / kWave + 1];
  __shared__ uint32_t h256[256];
  __shared__ int s_nlist[4];
  __shared__ int s_wl[NT / kWave][4];   // valid entries per (wave, list)
  __shared__ int s_res, s_hit, s_ev, s_vcnt, s_d;
  __shared__ int s_wa[2][NT / kWave], s_wb[2][NT / kWave];   // per-wave partials
  __shared__ uint32_t s_before;
  __shared__ unsigned long long s_kmin, s_kmax;
  __shared__ uint32_t s_fscan[NT / kWave][(MAXE + 1) / 2];   // fault counts (ONE)
  __shared__ uint32_t s_vscan[NT / kWave][8];                 // candidates per stamp
  __shared__ int s_wsig[NT / kWave];                          // oldest stamp below s, per wave
  int32_t* sA = reinterpret_cast<int32_t*>(sA64);

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int PK = P * K;
  const int32_t* tk = (FUSED ? topk_out : topk) + (size_t)b * PK;
  const int32_t* btb = bt + (size_t)b * max_blocks;
  const int64_t* hbt = host_bt ? host_bt + (size_t)b * max_blocks : nullptr;
  int32_t* t2s = tok2slot + (size_t)b * T_stride;
  int32_t* s2t = slot2tok + (size_t)b * C;
  int32_t* stp = stamp + (size_t)b * C;
  // this request's hot blocks (LDS), a cleared hit mask, and the stamps of this
  // thread's contiguous run of slots for the victim choice, read before the
  // hits of this step are known (they are masked in from sHitMask later
  // instead of read back).  ONE: the slots' owners too, so that an evicted
  // token is known without another round of loads.
  const int S = (C + NT - 1) / NT;
  int st_reg[MAXS], ow_reg[MAXS];
  auto load_slots = [&]() {
    for (int i = tid; i < (C >> 6); i += NT) sHot[i] = hot_blocks[(size_t)b * (C >> 6) + i];
    for (int i = tid; i < (C >> 5); i += NT) sHitMask[i] = 0u;
#pragma unroll
    for (int j = 0; j < MAXS; ++j) {
      const int v = tid * S + j;
      st_reg[j] = (j < S && v < C) ? stp[v] : 0x7FFFFFFF;
      if constexpr (ONE) ow_reg[j] = (j < S && v < C) ? s2t[v] : -1;
    }
  };
  if constexpr (FUSED) {
    // the slot state does not depend on the selection: its loads overlap it
    load_slots();
    topk_sel::finalize_row(b, ctx_len, 1, T_stride, K, tws, topk_out, arena);
    __syncthreads();   // the row's top-K (this workgroup's global writes) and the LDS handed over
  }
  const int s = step[0] + 1;

  if (tid == 0) {
    s_res = 0;
    s_hit = 0;
    s_ev = 0;
    s_vcnt = 0;
    s_kmin = ~0ull;
    s_kmax = 0ull;
  }
  int row[MAXE];
  int xs[MAXE];   // ONE: entry i * NT + tid; else entry i * NT + tid of the P lists
  // ONE: the list's tokens come first, and the page, host-page and hot-slot
  // lookups of every entry go out as soon as they arrive (one round), ahead of
  // the hot blocks, stamps and slot owners below
  int rb[MAXE], vs[MAXE];
  int64_t hrow[MAXE];
  if constexpr (ONE) {
#pragma unroll
    for (int i = 0; i < MAXE; ++i) {
      const int e = i * NT + tid;
      xs[i] = e < K ? tk[e] : -1;
    }
#pragma unroll
    for (int i = 0; i < MAXE; ++i) {
      const int t = xs[i];
      rb[i] = t >= 0 ? btb[t >> 6] : 0;
      hrow[i] = (t >= 0 && hbt) ? hbt[t >> 6] : -1;
      vs[i] = (t >= 0 && C > 0) ? t2s[t] : -1;
    }
  }
  if constexpr (!FUSED) load_slots();
  int32_t* sOld = sU;   // ONE: the previous owner of victim i (sU is not used)
  // the oldest stamp below s before this step's hits: no candidate victim is
  // older (published to LDS here, read after a later barrier)
  {
    int mn = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < MAXS; ++j)
      if (st_reg[j] < s) mn = min(mn, st_reg[j]);
    mn = wave_min_i32(mn);
    if (lane == 0) s_wsig[tid / kWave] = mn;
  }
  int nF;
  // several positions: U, its size, the run U[u0, u0 + E) this thread
  // classifies, and (bitmap path) the index in U of each of its list entries
  int nU = 0, E = 0, u0 = 0;
  const int32_t* U = nullptr;
  int urank[MAXE];
  bool have_rank = false;
  if constexpr (ONE) {
    // 1-2. the list is U; its lookups went out above
    __syncthreads();   // counters, hot blocks and hit mask initialized
    int my_res = 0, my_hit = 0;
    uint32_t fw[(MAXE + 1) / 2];
#pragma unroll
    for (int k = 0; k < (MAXE + 1) / 2; ++k) fw[k] = 0u;
#pragma unroll
    for (int i = 0; i < MAXE; ++i) {
      row[i] = -1;
      const int t = xs[i];
      if (t < 0) continue;
      if (rb[i] >= 0) {
        ++my_res;
        row[i] = rb[i] * kBlock + (t & 63);
      } else if (vs[i] >= 0) {
        ++my_hit;
        stp[vs[i]] = s;
        atomicOr(&sHitMask[vs[i] >> 5], 1u << (vs[i] & 31));
        row[i] = sHot[vs[i] >> 6] * kBlock + (vs[i] & 63);
      } else if (hrow[i] < 0) {
        atomicOr(err, 2);
      } else {
        row[i] = -2;          // fault; index assigned below
        fw[i >> 1] += 1u << (16 * (i & 1));
      }
    }
    // fault positions in entry (= token) order: entry i * 1024 + t comes after
    // every entry of rounds before i and of threads before t in round i
    uint32_t fex[(MAXE + 1) / 2], ftot[(MAXE + 1) / 2];
    block_scan_packed16<NT, (MAXE + 1) / 2>(fw, s_fscan, fex, ftot);
    int base = 0;
    nF = 0;
#pragma unroll
    for (int i = 0; i < MAXE; ++i) nF += field16(ftot, i);
#pragma unroll
    for (int i = 0; i < MAXE; ++i) {
      if (row[i] == -2) {
        const int pos = base + field16(fex, i);
        sF[pos] = xs[i];
        row[i] = -2 - pos;
      }
      base += field16(ftot, i);
    }
    my_res = wave_sum_i32(my_res);
    my_hit = wave_sum_i32(my_hit);
    if (lane == 0) {
      if (my_res) atomicAdd(&s_res, my_res);
      if (my_hit) atomicAdd(&s_hit, my_hit);
    }
    // no barrier: the hit mask is complete (the scan's barrier followed every
    // hit), and the fault list is read only after the victims' barriers
  } else {
    // 1. U = sorted distinct selected tokens.  Each list is sorted with a -1
    // tail; valid entries are counted with one ballot per wave and list.  The
    // lists are read in the same round of loads as the hot blocks and stamps.
    int32_t* Lin = sA;             // P lists of K
    int32_t* M = sA + kMaxSel;     // merged run with duplicates
    {
      const int wid = tid / kWave;
      int nl[4] = {0, 0, 0, 0};
      // unrolled to the instance's bound (P*K <= MAXE*1024) so that every load is
      // issued before the first one is used
#pragma unroll
      for (int i = 0; i < MAXE; ++i) {
        const int e = i * NT + tid;
        xs[i] = e < PK ? tk[e] : -1;
      }
#pragma unroll
      for (int i = 0; i < MAXE; ++i) {
        const int e = i * NT + tid;
        if (e < PK) Lin[e] = xs[i];
        // one list per run of K entries (K may not be a multiple of 64)
#pragma unroll
        for (int p = 0; p < 4; ++p)
          if (p < P) nl[p] += __popcll(__ballot(xs[i] >= 0 && e >= p * K && e < p * K + K));
      }
      if (lane == 0)
#pragma unroll
        for (int p = 0; p < 4; ++p) s_wl[wid][p] = nl[p];
    }
    __syncthreads();
    if (tid < P) {
      int c = 0;
      for (int w = 0; w < NT / kWave; ++w) c += s_wl[w][tid];
      s_nlist[tid] = c;
    }
    __syncthreads();
    if (P == 1) {
      nU = s_nlist[0];
      U = Lin;
    } else if (T_stride <= kMaxSel * 32) {
      // a bitmap of the selected tokens over the merge region: duplicates across
      // the positions collapse, and a token's index in U is the number of set
      // bits below it (thread j owns a run of 2^lw words; a block scan of the
      // runs' popcounts, then the popcounts before the token inside its run)
      uint32_t* bm = reinterpret_cast<uint32_t*>(M);
      int32_t* run_pre = sF;                 // the fault list is written later
      const int nwords = T_stride / 32;
      const int wpt = (nwords + NT - 1) / NT;
      const int lw = wpt <= 1 ? 0 : 32 - __clz(wpt - 1);   // runs of a power of two >= wpt words
      for (int w = tid; w < nwords; w += NT) bm[w] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MAXE; ++i)
        if (xs[i] >= 0) atomicOr(&bm[xs[i] >> 5], 1u << (xs[i] & 31));
      __syncthreads();
      int c = 0;
      for (int j = 0; j < (1 << lw); ++j) {
        const int w = (tid << lw) + j;
        if (w < nwords) c += __popc(bm[w]);
      }
      int tot;
      run_pre[tid] = block_exclusive_scan<NT>(c, scratch, &tot);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MAXE; ++i) {
        urank[i] = -1;
        const int x = xs[i];
        if (x < 0) continue;
        const int w = x >> 5, run = w >> lw;
        int r = run_pre[run] + __popc(bm[w] & ((1u << (x & 31)) - 1u));
        for (int w2 = run << lw; w2 < w; ++w2) r += __popc(bm[w2]);
        urank[i] = r;
        sU[r] = x;                            // equal tokens write the same entry
      }
      nU = tot;
      U = sU;
      have_rank = true;
      __syncthreads();
    } else {
      int total = 0;
      for (int p = 0; p < P; ++p) total += s_nlist[p];
      for (int e = tid; e < PK; e += NT) {
        const int p = e / K, i = e - p * K;
        if (i >= s_nlist[p]) continue;
        const int x = Lin[e];
        int pos = i;
        for (int q = 0; q < P; ++q) {
          if (q == p) continue;
          pos += (q < p) ? upper_bound_lds(Lin + q * K, s_nlist[q], x)
                         : lower_bound_lds(Lin + q * K, s_nlist[q], x);
        }
        M[pos] = x;
      }
      __syncthreads();
      int run = 0;
      for (int base = 0; base < total; base += NT) {
        const int idx = base + tid;
        const bool keep = idx < total && (idx == 0 || M[idx] != M[idx - 1]);
        const int x = idx < total ? M[idx] : 0;
        int tot;
        const int ex = block_exclusive_scan<NT>(keep ? 1 : 0, scratch, &tot);
        if (keep) sU[run + ex] = x;
        run += tot;
      }
      nU = run;
      U = sU;
      __syncthreads();
    }

    // 2. classify.  Thread t owns the contiguous run U[t*E, t*E + E); all of its
    // table reads are issued together.  Rows: >= 0 known, -1 none, <= -2 the
    // (-2 - i)-th fault, resolved once victims are known.
    E = (nU + NT - 1) / NT;   // <= MAXE
    u0 = tid * E;
    int tok[MAXE];
    // the hot-slot lookup is issued with the page lookups (every token has an
    // entry), so the classification waits for one round of loads, not two
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
      const bool ok = e < E && u0 + e < nU;
      tok[e] = ok ? U[u0 + e] : -1;
      rb[e] = ok ? btb[tok[e] >> 6] : 0;
      hrow[e] = (ok && hbt) ? hbt[tok[e] >> 6] : -1;
      vs[e] = (ok && C > 0) ? t2s[tok[e]] : -1;
    }
    int my_res = 0, my_hit = 0, my_f = 0;
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
      row[e] = -1;
      const int t = tok[e];
      if (t < 0) continue;
      if (rb[e] >= 0) {
        ++my_res;
        row[e] = rb[e] * kBlock + (t & 63);
      } else if (vs[e] >= 0) {
        ++my_hit;
        stp[vs[e]] = s;
        atomicOr(&sHitMask[vs[e] >> 5], 1u << (vs[e] & 31));
        row[e] = sHot[vs[e] >> 6] * kBlock + (vs[e] & 63);
      } else if (hrow[e] < 0) {
        atomicOr(err, 2);
      } else {
        row[e] = -2;          // fault; index assigned below
        ++my_f;
      }
    }
    {
      int pos = block_exclusive_scan<NT>(my_f, scratch, &nF);
#pragma unroll
      for (int e = 0; e < MAXE; ++e)
        if (row[e] == -2) {
          sF[pos] = tok[e];
          row[e] = -2 - pos;
          ++pos;
        }
    }
    // per-wave totals, one LDS atomic per wave (same-address atomics from every
    // thread serialize)
    my_res = wave_sum_i32(my_res);
    my_hit = wave_sum_i32(my_hit);
    if (lane == 0) {
      if (my_res) atomicAdd(&s_res, my_res);
      if (my_hit) atomicAdd(&s_hit, my_hit);
    }
    // The stamps written above are read back below only by this workgroup, and
    // no line of the table was read before: the barrier's workgroup-scope
    // release/acquire is enough (a device-scope fence would write back L2).
    __syncthreads();

  }

  // 3. victims: the n_serve smallest (stamp, slot) keys among slots with
  // stamp < s, in that order.  Slots are split into contiguous runs per thread
  // with their stamps in registers.  LRU victims usually span a few distinct
  // stamps: a packed count per stamp value places them all at once; else one
  // distinct stamp value at a time (oldest first), its slots emitted in slot
  // order by one block prefix sum; beyond kMaxStampRounds values the general
  // path (radix select + sort) takes over.
  int n_serve = 0;
  bool keys64 = false;            // victims as sorted 64-bit keys (general path)
  int32_t* V32 = sA;              // victim slots, fast path (R1: the merge lists are dead)
  if (nF > 0 && C > 0) {
    const int wid = tid / kWave;
    // this step's hits leave the candidates
#pragma unroll
    for (int j = 0; j < MAXS; ++j) {
      const int v = tid * S + j;
      if (j < S && v < C && (sHitMask[v >> 5] >> (v & 31)) & 1u) st_reg[j] = s;
    }
    // Candidates counted per stamp value from the oldest one sig on (a counter
    // for each of the 15 oldest values, a 16th for all later ones), with one
    // packed block scan: a slot's place in (stamp, slot) order is the count of
    // older values plus the slots of its value in earlier threads and earlier
    // in its own run.  Exact whenever every victim has one of the 15 oldest
    // values; otherwise the rounds below take over.
    int sig = 0x7FFFFFFF;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) sig = min(sig, s_wsig[w]);
    // this thread's counters: 16 values in 8 private LDS words (two 16-bit
    // fields each) in the upper half of sA, which holds nothing at this point
    // (victims fill its lower half); LDS atomics count without selects
    uint32_t* pc = reinterpret_cast<uint32_t*>(sA) + kMaxSel + tid * 8;
    int bk[MAXS];
    uint32_t vc[8];
    *reinterpret_cast<uint4*>(pc) = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(pc + 4) = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < MAXS; ++j) {
      bk[j] = st_reg[j] < s ? min(st_reg[j] - sig, 15) : -1;
      if (bk[j] >= 0) atomicAdd(&pc[bk[j] >> 1], 1u << (16 * (bk[j] & 1)));
    }
    {
      const uint4 a = *reinterpret_cast<const uint4*>(pc);
      const uint4 c = *reinterpret_cast<const uint4*>(pc + 4);
      vc[0] = a.x; vc[1] = a.y; vc[2] = a.z; vc[3] = a.w;
      vc[4] = c.x; vc[5] = c.y; vc[6] = c.z; vc[7] = c.w;
    }
    uint32_t vex[8], vtot[8];
    block_scan_packed16<NT, 8>(vc, s_vscan, vex, vtot);
    int n_cand = 0, older15 = 0;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (v == 15) older15 = n_cand;
      n_cand += field16(vtot, v);
    }
    n_serve = min(nF, n_cand);
    const bool packed = n_serve <= older15;
    if (packed) {
      // the counters become this thread's next place in each value's run
      // (below n_cand <= 16384: fields never carry); each slot takes its place
      // with one LDS atomic, in slot order
      int before = 0;
      uint32_t pl[8];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t at = (uint32_t)(before + field16(vex, v));
        if (v & 1) pl[v >> 1] |= at << 16; else pl[v >> 1] = at;
        before += field16(vtot, v);
      }
      *reinterpret_cast<uint4*>(pc) = make_uint4(pl[0], pl[1], pl[2], pl[3]);
      *reinterpret_cast<uint4*>(pc + 4) = make_uint4(pl[4], pl[5], pl[6], pl[7]);
#pragma unroll
      for (int j = 0; j < MAXS; ++j)
        if (bk[j] >= 0 && bk[j] < 15) {
          const int sh = 16 * (bk[j] & 1);
          const int pos = (int)((atomicAdd(&pc[bk[j] >> 1], 1u << sh) >> sh) & 0xFFFFu);
          if (pos < n_serve) {
            V32[pos] = tid * S + j;
            if constexpr (ONE) sOld[pos] = ow_reg[j];
          }
        }
    } else {
      int my_c = 0, my_min = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < MAXS; ++j) {
        if (st_reg[j] < s) {
          ++my_c;
          my_min = min(my_min, st_reg[j]);
        }
      }
      // the oldest candidate stamp: wave reductions, one barrier
      my_c = wave_sum_i32(my_c);
      my_min = wave_min_i32(my_min);
      if (lane == 0) {
        s_wa[0][wid] = my_c;
        s_wb[0][wid] = my_min;
      }
      __syncthreads();
      int sigma = 0x7FFFFFFF;
#pragma unroll
      for (int w = 0; w < NT / kWave; ++w) sigma = min(sigma, s_wb[0][w]);
      int got = 0;
      bool fast = true;
      // one distinct stamp per round, slots in slot order: a slot's rank within
      // the round is the number of equal stamps in earlier slots, counted with
      // one ballot per slot of a thread's run (slot = tid*S + j) plus the
      // earlier waves' totals; one barrier per round (partials double-buffered)
      for (int round = 0; got < n_serve; ++round) {
        if (round == kMaxStampRounds) {
          fast = false;
          break;
        }
        const int buf = (round + 1) & 1;
        int below = 0, wtot = 0, my_next = 0x7FFFFFFF;
        uint64_t m[MAXS];
#pragma unroll
        for (int j = 0; j < MAXS; ++j) {
          m[j] = __ballot(st_reg[j] == sigma);
          below += lanes_below(m[j]);
          wtot += __popcll(m[j]);
          if (st_reg[j] > sigma && st_reg[j] < s) my_next = min(my_next, st_reg[j]);
        }
        my_next = wave_min_i32(my_next);
        if (lane == 0) {
          s_wa[buf][wid] = wtot;
          s_wb[buf][wid] = my_next;
        }
        __syncthreads();
        int off = 0, tot = 0, nxt = 0x7FFFFFFF;
#pragma unroll
        for (int w = 0; w < NT / kWave; ++w) {
          const int x = s_wa[buf][w];
          off += w < wid ? x : 0;
          tot += x;
          nxt = min(nxt, s_wb[buf][w]);
        }
        // equal stamps in this thread's earlier slots
        int pos = got + off + below;
#pragma unroll
        for (int j = 0; j < MAXS; ++j)
          if (st_reg[j] == sigma) {
            if (pos < n_serve) {
              V32[pos] = tid * S + j;
              if constexpr (ONE) sOld[pos] = ow_reg[j];
            }
            ++pos;
          }
        got += tot;
        sigma = nxt;
      }
      if (!fast) {
        keys64 = true;
        unsigned long long kmin = ~0ull, kmax = 0ull;
        for (int v = tid; v < C; v += NT) {
          const int st = stp[v];
          if (st < s) {
            const unsigned long long key = ((unsigned long long)(uint32_t)st << 32) | (uint32_t)v;
            kmin = min(kmin, key);
            kmax = max(kmax, key);
          }
        }
        atomicMin(&s_kmin, kmin);
        atomicMax(&s_kmax, kmax);
        __syncthreads();
        unsigned long long thr = s_kmax;
        if (n_serve < n_cand) {
          // MSD radix select of the n_serve-th smallest key, from the highest
          // byte in which candidate keys differ
          const unsigned long long diff = s_kmin ^ s_kmax;
          const int top_byte = (63 - __builtin_clzll(diff)) >> 3;
          unsigned long long prefix = (top_byte == 7) ? 0ull : (s_kmin >> (8 * (top_byte + 1)));
          uint32_t need = (uint32_t)n_serve;
          for (int pos = top_byte; pos >= 0; --pos) {
            if (tid < 256) h256[tid] = 0;
            __syncthreads();
            for (int v = tid; v < C; v += NT) {
              const int st = stp[v];
              if (st >= s) continue;
              const unsigned long long key = ((unsigned long long)(uint32_t)st << 32) | (uint32_t)v;
              if (pos == 7 || (key >> (8 * (pos + 1))) == prefix)
                atomicAdd(&h256[(key >> (8 * pos)) & 0xFFu], 1u);
            }
            __syncthreads();
            find_bin256_lo(h256, need, &s_d, &s_before);
            prefix = (prefix << 8) | (unsigned long long)s_d;
            need -= s_before;
            __syncthreads();
          }
          thr = prefix;
        }
        // gather the victims (exactly n_serve keys <= thr) and sort them
        uint64_t* V = sA64;
        for (int v = tid; v < C; v += NT) {
          const int st = stp[v];
          if (st >= s) continue;
          const unsigned long long key = ((unsigned long long)(uint32_t)st << 32) | (uint32_t)v;
          if (key <= thr) {
            const int at = atomicAdd(&s_vcnt, 1);
            if (at < kMaxSel) V[at] = key;
          }
        }
        int np = 1;
        while (np < n_serve) np <<= 1;
        __syncthreads();
        for (int i = n_serve + tid; i < np; i += NT) V[i] = ~0ull;
        __syncthreads();
        for (int size = 2; size <= np; size <<= 1) {
          for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < np / 2; i += NT) {
              const int lo = 2 * i - (i & (stride - 1));
              const int hi = lo + stride;
              const bool asc = (lo & size) == 0;
              const uint64_t a = V[lo], c = V[hi];
              if ((a > c) == asc) {
                V[lo] = c;
                V[hi] = a;
              }
            }
            __syncthreads();
          }
        }
      }
    }
    __syncthreads();
    // 4. fault i -> victim i.  Victims are distinct slots and an evicted token
    // is hot, so never one of the faults: every old slot owner is read first
    // (one round of loads, n_serve <= P*K <= MAXE * NT), then written.
    int my_ev = 0;
    int32_t* fb = faults + (size_t)b * PK * 2;
    int vv[MAXE], tt[MAXE], oo[MAXE];
#pragma unroll
    for (int u = 0; u < MAXE; ++u) {
      const int i = tid + u * NT;
      vv[u] = -1;
      tt[u] = 0;
      if (i < n_serve) {
        vv[u] = keys64 ? (int)(uint32_t)sA64[i] : V32[i];
        tt[u] = sF[i];
      }
    }
    // previous owners: recorded with the victims (ONE, packed and round paths)
    // or read from the table
    const bool old_known = ONE && !keys64;
#pragma unroll
    for (int u = 0; u < MAXE; ++u)
      oo[u] = vv[u] < 0 ? -1 : old_known ? sOld[tid + u * NT] : s2t[vv[u]];
#pragma unroll
    for (int u = 0; u < MAXE; ++u) {
      const int v = vv[u], t = tt[u], i = tid + u * NT;
      if (v < 0) continue;
      if (oo[u] >= 0) {
        t2s[oo[u]] = -1;
        ++my_ev;
      }
      s2t[v] = t;
      t2s[t] = v;
      stp[v] = s;
      fb[2 * i] = t;
      fb[2 * i + 1] = v;
    }
    my_ev = wave_sum_i32(my_ev);
    if (lane == 0 && my_ev) atomicAdd(&s_ev, my_ev);
  }
  if (tid == 0 && n_serve < nF) atomicOr(err, 1);
  // fault rows from their victims (faults past n_serve keep row -1)
#pragma unroll
  for (int e = 0; e < MAXE; ++e)
    if (row[e] <= -2) {
      const int i = -2 - row[e];
      if (i < n_serve) {
        const int v = keys64 ? (int)(uint32_t)sA64[i] : V32[i];
        row[e] = sHot[v >> 6] * kBlock + (v & 63);
      } else {
        row[e] = -1;
      }
    }

  // 5. row ids of every (position, k)
  int32_t* rid = row_ids + (size_t)b * PK;
  if constexpr (ONE) {
#pragma unroll
    for (int i = 0; i < MAXE; ++i) {
      const int e = i * NT + tid;
      if (e < K) rid[e] = row[i];
    }
  } else if (P == 1) {
#pragma unroll
    for (int e = 0; e < MAXE; ++e)
      if (e < E && u0 + e < nU) rid[u0 + e] = row[e];
    for (int k = nU + tid; k < K; k += NT) rid[k] = -1;
  } else {
    __syncthreads();                       // every read of the victims is done
    int32_t* rowU = sA;
#pragma unroll
    for (int e = 0; e < MAXE; ++e)
      if (e < E && u0 + e < nU) rowU[u0 + e] = row[e];
    __syncthreads();
    if (have_rank) {
#pragma unroll
      for (int i = 0; i < MAXE; ++i) {
        const int e = i * NT + tid;
        if (e < PK) rid[e] = xs[i] < 0 ? -1 : rowU[urank[i]];
      }
    } else {
      for (int e = tid; e < PK; e += NT) {
        const int t = tk[e];
        rid[e] = t < 0 ? -1 : rowU[lower_bound_lds(sU, nU, t)];
      }
    }
  }
  __syncthreads();                         // every eviction is counted
  if (tid == 0) {
    counts[b * 4 + 0] = s_res;
    counts[b * 4 + 1] = s_hit;
    counts[b * 4 + 2] = n_serve;
    counts[b * 4 + 3] = s_ev;
  }
}

// Fault copies.  Zero-copy reads of pinned host memory are bound by the host
// link and, for rows scattered over gigabytes of 4-KiB host pages, by the
// GPU's address translation: random rows inside a 75 MB window stream at the
// link rate, the same rows spread over 2.4 GB lose about 12 %.  So the grid
// keeps few requests in flight: each request's faults are cut into small
// batches (BATCH faults) dealt to the persistent workgroups round-robin in
// request order, so that the batches in flight at any time come from about
// grid x BATCH / faults-per-request requests.  A workgroup pipelines its
// batches: while the host reads of one batch are in flight, the source and
// destination rows of its next batch are looked up into the other LDS buffer.
template <int BATCH>
struct CopyCursor {
  int b, j, gbb;   // request, batch within it, batches of earlier requests

  // Advances to this workgroup's next batch; false when there is none.
  // nfault(b): the fault count of request b.
  template <typename F>
  __device__ bool next(int B, F nfault, int grid, int me) {
    j += grid;
    while (b < B) {
      const int nb = (nfault(b) + BATCH - 1) / BATCH;
      if (j < nb) return true;
      gbb += nb;
      ++b;
      j = me - gbb % grid;
      if (j < 0) j += grid;
    }
    return false;
  }
};

template <int NT, int U, int BATCH>
__global__ __launch_bounds__(NT) void fault_copy_kernel(
    int B, int PK, int C, int L, int row_bytes, int max_blocks, const int32_t* __restrict__ faults,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ hot_blocks,
    const int64_t* __restrict__ host_bt, const uint8_t* __restrict__ host_rows,
    const float* __restrict__ host_scale, int64_t host_layer_rows, int64_t host_pitch,
    uint8_t* __restrict__ pool, float* __restrict__ row_scale, int64_t pool_layer_rows,
    int32_t* __restrict__ step, int l0, int nl) {
  __shared__ int64_t s_src[2][BATCH * kCopyMaxL];
  __shared__ int64_t s_dst[2][BATCH * kCopyMaxL];
  __shared__ int s_n[2];
  // every request's fault count, read once into LDS (up to kCopyCntLds requests):
  // a workgroup walks the requests to find its batches, and a walk of dependent
  // global loads would cost a memory round trip per request
  __shared__ int s_cnt[kCopyCntLds];
  // layers l0 .. l0 + nl - 1 of the L layers; the call that copies the last
  // layer ends the step
  if (l0 + nl == L && blockIdx.x == 0 && threadIdx.x == 0) step[0] = step[0] + 1;
  const bool cnt_lds = B <= kCopyCntLds;
  if (cnt_lds)
    for (int i = threadIdx.x; i < B; i += NT) s_cnt[i] = counts[i * 4 + 2];
  __syncthreads();
  auto nfault = [&](int r) { return cnt_lds ? s_cnt[r] : counts[r * 4 + 2]; };
  const int cpr = row_bytes / 16;           // 16-byte chunks per row
  const int grid = gridDim.x, me = blockIdx.x;
  // source and destination byte offsets of one batch, one (fault, layer) per thread
  auto lookup = [&](const CopyCursor<BATCH>& cu, int buf) {
    const int n = nfault(cu.b);
    const int f0 = cu.j * BATCH;
    const int nloc = min(BATCH, n - f0);
    if (threadIdx.x == 0) s_n[buf] = nloc;
    for (int i = threadIdx.x; i < nloc * nl; i += NT) {
      const int fi = f0 + i / nl, l = l0 + i % nl;
      const int32_t* fb = faults + ((size_t)cu.b * PK + fi) * 2;
      const int t = fb[0], sl = fb[1];
      const int64_t hr = host_bt[(size_t)cu.b * max_blocks + (t >> 6)] + (t & 63);
      const int64_t pr =
          (int64_t)hot_blocks[(size_t)cu.b * (C >> 6) + (sl >> 6)] * kBlock + (sl & 63);
      const int64_t hrow = (int64_t)l * host_layer_rows + hr * host_pitch;
      s_src[buf][i] = hrow * row_bytes;
      s_dst[buf][i] = ((int64_t)l * pool_layer_rows + pr) * row_bytes;
      if (host_scale) row_scale[(size_t)l * pool_layer_rows + pr] = host_scale[hrow];
    }
  };
  CopyCursor<BATCH> cur{0, me - grid, 0};
  bool have = cur.next(B, nfault, grid, me);
  if (have) lookup(cur, 0);
  __syncthreads();
  int buf = 0;
  while (have) {
    CopyCursor<BATCH> nxt = cur;
    const bool have_next = nxt.next(B, nfault, grid, me);
    const int nchunk = s_n[buf] * nl * cpr;
    for (int c0 = 0; c0 < nchunk; c0 += NT * U) {
      uint4 v[U];
      int64_t d[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = c0 + u * NT + (int)threadIdx.x;
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        int64_t dd = -1;
        if (idx < nchunk) {
          const int row = idx / cpr, c = idx - row * cpr;
          x = *reinterpret_cast<const uint4*>(host_rows + s_src[buf][row] + (int64_t)c * 16);
          dd = s_dst[buf][row] + (int64_t)c * 16;
        }
        v[u] = x;
        d[u] = dd;
      }
      // the next batch's lookups go out while these host reads are in flight
      if (c0 == 0 && have_next) lookup(nxt, buf ^ 1);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (d[u] >= 0) *reinterpret_cast<uint4*>(pool + d[u]) = v[u];
    }
    if (nchunk == 0 && have_next) lookup(nxt, buf ^ 1);
    __syncthreads();
    cur = nxt;
    have = have_next;
    buf ^= 1;
  }
}

}  // namespace

hipError_t launch_resolve_tables(const BatchDims& d, int K, const int32_t* topk,
                                 const ResidencyArgs& r, int32_t* row_ids, int32_t* faults,
                                 int32_t* counts, hipStream_t s) {
#define HS_RESOLVE(NT_, S_, E_, ONE_)                                                         \
  hipLaunchKernelGGL((resolve_kernel<NT_, S_, E_, ONE_, false>), dim3(d.B), dim3(NT_), 0, s,     \
                     d.T_stride, d.max_blocks, d.P, K, topk, r.C, r.bt, r.hot_blocks, r.tok2slot,  \
                     r.slot2tok, r.stamp, r.step, r.err, r.host_bt, row_ids, faults, counts,       \
                     nullptr, topk_sel::TopkWs{}, nullptr)
  const int slots = (r.C + kResNT - 1) / kResNT, entries = (d.P * K + kResNT - 1) / kResNT;
  static_assert(kMaxSlotsPerThread == 16 && kMaxEntriesPerThread == 8, "instances below");
  if (d.P == 1) {
    if (slots <= 4 && entries <= 2) HS_RESOLVE(kResNT, 4, 2, true);
    else if (slots <= 16 && entries <= 2) HS_RESOLVE(kResNT, 16, 2, true);
    else HS_RESOLVE(kResNT, 16, 8, true);
  } else {
    if (slots <= 4 && entries <= 2) HS_RESOLVE(kResNT, 4, 2, false);
    else if (slots <= 4 && entries <= 4) HS_RESOLVE(kResNT, 4, 4, false);
    else if (slots <= 8 && entries <= 4) HS_RESOLVE(kResNT, 8, 4, false);
    else if (slots <= 8 && entries <= 8) HS_RESOLVE(kResNT, 8, 8, false);
    else if (slots <= 10 && entries <= 8) HS_RESOLVE(kResNT, 10, 8, false);   // (3+2)K hot rows at K = 2048
    else HS_RESOLVE(kResNT, 16, 8, false);
  }
#undef HS_RESOLVE
  return hipGetLastError();
}

hipError_t launch_finalize_resolve(const BatchDims& d, int K, int32_t* topk, void* ws,
                                   const ResidencyArgs& r, int32_t* row_ids, int32_t* faults,
                                   int32_t* counts, hipStream_t s) {
  if (d.P != 1) {
    hipError_t e = launch_topk_finalize(d, K, topk, ws, s);
    if (e != hipSuccess) return e;
    return launch_resolve_tables(d, K, topk, r, row_ids, faults, counts, s);
  }
  const topk_sel::TopkWs w = topk_sel::topk_ws(ws, d.B, d.T_stride, K);
#define HS_FUSED(S_, E_)                                                                     \
  hipLaunchKernelGGL((resolve_kernel<kResNT, S_, E_, true, true>), dim3(d.B), dim3(kResNT), 0, s, \
                     d.T_stride, d.max_blocks, 1, K, nullptr, r.C, r.bt, r.hot_blocks,            \
                     r.tok2slot, r.slot2tok, r.stamp, r.step, r.err, r.host_bt, row_ids, faults,  \
                     counts, d.ctx_len, w, topk)
  const int slots = (r.C + kResNT - 1) / kResNT, entries = (K + kResNT - 1) / kResNT;
  if (slots <= 4 && entries <= 2) HS_FUSED(4, 2);
  else if (slots <= 16 && entries <= 2) HS_FUSED(16, 2);
  else HS_FUSED(16, 8);
#undef HS_FUSED
  return hipGetLastError();
}

hipError_t launch_fault_copy(const BatchDims& d, int K, const ResidencyArgs& r,
                             const int32_t* faults, const int32_t* counts, int l0, int nl,
                             int workgroups, hipStream_t s) {
  const int PK = d.P * K;
  const int row_bytes = kDLat * r.kv_bytes;
  const int grid = workgroups > 0 ? workgroups : kCopyWGs;
  hipLaunchKernelGGL((fault_copy_kernel<kCopyNT, kCopyInFlight, kCopyBatch>), dim3(grid), dim3(kCopyNT), 0, s, d.B, PK, r.C, r.L,
                     row_bytes, d.max_blocks, faults, counts, r.hot_blocks, r.host_bt,
                     static_cast<const uint8_t*>(r.host_rows), r.host_scale, r.host_layer_rows,
                     r.host_row_pitch,
                     static_cast<uint8_t*>(r.pool), r.row_scale, r.pool_layer_rows, r.step, l0,
                     nl);
  return hipGetLastError();
}

}  // namespace hs
