// Sparse MLA decode attention on gfx950, absorbed (MQA) form: every head
// attends over the same selected 576-value latent rows, which serve as keys,
// and over their first 512 values, which serve as values (page "vLLM sert
// GLM-5.3 en contexte 1M sur 16 H200", section "Comment s'y prendre", option
// sparse_mla_force_mqa; the selected rows come from the indexer's top-K, page
// "Un contexte d'un million sur huit H200", section "Ce qui se passe").
//
// bf16 x E4M3 path, one workgroup = 4 waves on one (request, position, group
// of 16 heads) and a slice of its K selected rows; each wave works alone on
// its quarter of the slice, in 16-row tiles, and the four waves merge at the
// end:
//   gather   a ring of 4 tiles of row loads in registers, every load issued
//            unconditionally (a slot past the last tile reads one line of a
//            valid row) so that the compiler waits for the oldest tile only.
//            Lane (n, g) reads bytes 16g .. 16g+15 of every 64-byte chunk of
//            row n, so one wave load covers whole 64-byte chunks of 16 rows;
//            the contraction index is permuted the same way in the query
//            fragments, which a sum allows.
//   QK       two tiles at a time, two independent product chains: S^T[16 rows
//            x 16 heads] over the 576 values (18 steps of
//            v_mfma_f32_16x16x32_bf16), E4M3 converted to bf16 in registers;
//            the queries sit once per workgroup in LDS (rows padded so that
//            the 16 heads' fragment reads fall on distinct banks).  The value
//            parts go row-major into the wave's own LDS stash.
//   softmax  online per head over the two tiles' 32 rows, in the log2 domain,
//            the row scale folded into logit and probability; the running
//            output is rescaled only when some maximum moved.
//   PV       O^T[512 dims x 16 heads] += V^T . P^T with the 32 rows as the
//            contraction: laid out as rows 4g..4g+3 of each tile in lane group
//            g, the probabilities already are this lane's B operand; the V^T
//            fragments come out of the row-major stash through gfx950's
//            transposing LDS read (ds_read_b64_tr_b16).  The 512 x 16 outputs
//            live in the accumulation registers.
//   merge    the four waves' (O, max, sum) through LDS in wave order.
// A workgroup covers rows [split*R, split*R + R) in ascending k (or one chunk
// of a chunk list: the token-sharded path).  With one slice it writes out/lse
// directly; otherwise the combine kernel merges the slices' (O, max, sum) in
// slice order, so the reduction order depends only on the order of row_ids,
// never on where a row is stored.
#include "hs_common.h"
#include "hs_launch.h"

namespace hs {
namespace {

constexpr int kMlaNT = 256;
constexpr int kMlaTargetWGs = 256;   // splits of the selected rows fill about this many workgroups
constexpr int kMlaMaxSplitRows = 1024;   // and no slice walks more than 16 tiles
constexpr int kMlaRing = 4;              // tiles of row gathers in flight per workgroup
constexpr int kMaxShards = 64;           // token shards of the sharded attention
constexpr int kTile = 64;
constexpr int kPtStride = 72;   // bf16 per head of the probability tile (mla_tile_kernel)
constexpr int kHq = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kVrStride = 520;  // bf16 per row of the value tile: 512 + 8 pad (1040 bytes)

typedef short lds_v4i16 __attribute__((ext_vector_type(4)));

// Four consecutive value rows r0..r0+3 of one dim, for the MFMA A operand
// (V^T: dims as M, rows as K), read from the row-major value tile with
// gfx950's transposing LDS read: within each 16-lane group, source lane c
// names 4 dims of row r0 + c/4 (dims d0 + 4*(c%4)), and lane i receives dim
// d0 + i of rows r0 .. r0+3.
__device__ __forceinline__ lds_v4i16 vr_read_tr(const uint16_t* Vr, int r0, int d0, int c) {
  const uint16_t* src = Vr + (r0 + (c >> 2)) * kVrStride + d0 + 4 * (c & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) lds_v4i16*)(
          (__attribute__((address_space(3))) uint16_t*)(src)));
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

template <bool SPLIT>
__global__ __launch_bounds__(kMlaNT, 1) void mla_bf16_e4m3_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ pool,
    const float* __restrict__ row_scale, const int32_t* __restrict__ row_ids, int K,
    int rows_per_split, int nsplit, float qk_scale_log2, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml,
    int64_t pool_layer_rows, int hgroups, const int32_t* __restrict__ chunk_lo,
    const int32_t* __restrict__ chunk_hi) {
  // per wave: the value parts of its current two 16-row tiles (bf16, row-major);
  // once every wave is done with its rows, the same memory holds the four
  // waves' output partials for the in-workgroup merge
  __shared__ __attribute__((aligned(16))) uint16_t stash[4][2][16 * kVrStride];
  __shared__ int s_rid[4][kMlaMaxSplitRows / 4];   // each wave's row ids, -1 past its rows
  __shared__ float s_m[4][kHq], s_l[4][kHq];
  // the queries, loaded once per workgroup: rows of 72 16-byte words padded to
  // 73, so that the 16 heads' fragment reads fall on distinct banks
  constexpr int kQRow = kDLat * 2 / 16;
  __shared__ uint4 s_q[kHq * (kQRow + 1)];
  static_assert(sizeof(stash) >= 4 * kHq * kDVal * sizeof(float), "the merge reuses the stash");

  // blockIdx.y = (request position) * hgroups + (group of 16 heads): the
  // queries, outputs and partials of that head group; the row ids are the
  // request position's, shared by its head groups
  const int bp = blockIdx.y, split = blockIdx.x;
  const int rbp = bp / hgroups;
  // layer blockIdx.z of a multi-layer call: its queries, pool rows, scales,
  // outputs and partials sit one layer stride further (same row ids)
  {
    const size_t layer = blockIdx.z, BPn = gridDim.y;
    q += layer * BPn * kHq * kDLat;
    pool += layer * (size_t)pool_layer_rows * kDLat;
    if (row_scale) row_scale += layer * (size_t)pool_layer_rows;
    out += layer * BPn * kHq * kDVal;
    if (lse) lse += layer * BPn * kHq;
    if (SPLIT) {
      part_o += layer * BPn * nsplit * kHq * kDVal;
      part_ml += layer * BPn * nsplit * kHq * 2;
    }
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  // the slice [kb, kb + nrows) of the selection: split * rows_per_split on,
  // or the chunk of a chunk list (at most rows_per_split rows); wave w takes
  // its quarter [w0, w1), in 16-row tiles (rows_per_split is a multiple of 64)
  int kb, nrows;
  if (chunk_lo) {
    kb = min(max(chunk_lo[(size_t)rbp * nsplit + split], 0), K);
    nrows = min(max(chunk_hi[(size_t)rbp * nsplit + split] - kb, 0), min(rows_per_split, K - kb));
  } else {
    kb = split * rows_per_split;
    nrows = max(min(K, kb + rows_per_split) - kb, 0);
  }
  const int per_wave = rows_per_split / 4;
  const int w0 = min(wave * per_wave, nrows), w1 = min(w0 + per_wave, nrows);
  const int ntiles = (w1 - w0 + 15) / 16;

  // contraction step s takes dims dim0(s) .. +8 of head n (Q) and of row n (X)
  auto dim0 = [&](int s) { return 64 * (s >> 1) + 16 * g + 8 * (s & 1); };
  // the row ids first (the gathers wait for them), then the queries, which
  // stay in flight while the row ids go to this wave's own LDS row (the wave
  // alone reads them back, in program order after these writes)
  int* wrid = s_rid[wave];
  int first = -1;
  constexpr int kPer = kMlaMaxSplitRows / 4 / kWave;
  int r[kPer];
  constexpr int kQPer = (kHq * kQRow + kMlaNT - 1) / kMlaNT;
  const uint4* qg = reinterpret_cast<const uint4*>(q + (size_t)bp * kHq * kDLat);
  uint4 qv[kQPer];
  {
    const int32_t* rp = row_ids + (size_t)rbp * K + kb + w0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = lane + u * kWave;
      r[u] = i < w1 - w0 ? rp[i] : -1;
    }
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
      const int i = tid + kMlaNT * k;
      qv[k] = i < kHq * kQRow ? qg[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      wrid[lane + u * kWave] = r[u];
      if (first < 0 && r[u] >= 0) first = r[u];
    }
  }
  // a valid row of this wave: the target of reads that fill rows with id -1
  // and ring slots past the last tile (their probabilities are zero).  A wave
  // with no valid row reads the workgroup's queries instead (any readable 16
  // bytes) and skips the work.
  const uint64_t have = __ballot(first >= 0);
  const int fallback = have ? __shfl(first, __ffsll((long long)have) - 1) : 0;
  const uint8_t* const no_row = reinterpret_cast<const uint8_t*>(qg);
  // the scale of this wave's row `lane` (rows of tiles 0..3), one load per wave
  const float sc_lane = have ? row_scale[r[0] >= 0 ? r[0] : fallback]
                             : *reinterpret_cast<const float*>(no_row);
  const bool few = ntiles <= kMlaRing;   // every tile in flight from the start

  f32x4_t o[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  // Row gathers: a ring of kMlaRing tiles in registers, every gather issued
  // unconditionally so that the compiler waits for the oldest tile only.
  // Lane (n, g) gathers row n of the tile, bytes 64v + 16g .. +16 for v =
  // 0..8 (a wave load covers whole 64-byte chunks of 16 rows).  A slot past
  // the last tile reads one 16-byte line of the fallback row instead.  Beyond
  // the first kMlaRing tiles a slot also loads its rows' scales.
  uint4 raw[kMlaRing][9];
  float rs[kMlaRing];
  auto issue = [&](int t, uint4* rw, float& sc, bool with_scale) {
    const bool live = have && t < ntiles;
    const int rid = wrid[min(t, max(ntiles - 1, 0)) * 16 + n];
    const int row = (live && rid >= 0) ? rid : fallback;
    // the scale first: waiting for it never waits for the row loads behind it
    if (with_scale) sc = row_scale[row];
    const uint8_t* src = have ? pool + (size_t)row * kDLat + (live ? 16 * g : 0) : no_row;
    const int step = live ? 64 : 0;
#pragma unroll
    for (int v = 0; v < 9; ++v) rw[v] = *reinterpret_cast<const uint4*>(src + step * v);
  };
#pragma unroll
  for (int j = 0; j < kMlaRing; ++j) issue(j, raw[j], rs[j], false);
  // the queries to LDS once they arrive (the gathers stay in flight), then
  // every wave reads its fragments: head n, dims dim0(s) .. +8
#pragma unroll
  for (int k = 0; k < kQPer; ++k) {
    const int i = tid + kMlaNT * k;
    if (i < kHq * kQRow) s_q[(i / kQRow) * (kQRow + 1) + i % kQRow] = qv[k];
  }
  __syncthreads();
  // query fragment of contraction step s, read from LDS where it is used
  const uint4* qrow = s_q + n * (kQRow + 1);
  auto qfrag = [&](int s) { return as_bf16x8(qrow[dim0(s) / 8]); };

  if (have) {

    uint16_t* stA = stash[wave][0];
    uint16_t* stB = stash[wave][1];
    // Tiles t and t + 1 (slots a, b): S^T = X . Q^T for both (two independent
    // product chains), the value parts stashed in this wave's LDS, online
    // softmax over the 32 rows, then O^T += V^T . P^T with K = 32 rows laid
    // out as [rows 4g..4g+3 of tile t, rows 4g..4g+3 of tile t + 1] in lane
    // group g: the probabilities are then already the B operand of this lane.
    auto pair = [&](int t, const uint4* ra, float rsa, const uint4* rb, float rsb) {
      // scales of the tiles' rows: lane 16t + r holds row r of tile t (< 4),
      // a refilled slot's lane r holds its row r
      const bool lane_sc = t < kMlaRing;
      f32x4_t aA = f32x4_t{0.f, 0.f, 0.f, 0.f}, aB = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 18; ++s) {
        const uint4 ca = ra[s >> 1], cb = rb[s >> 1];
        u32x4_t xa, xb;
        const uint32_t la = (s & 1) ? ca.z : ca.x, ha = (s & 1) ? ca.w : ca.y;
        const uint32_t lb = (s & 1) ? cb.z : cb.x, hb = (s & 1) ? cb.w : cb.y;
        xa[0] = e4m3x2_to_bf16x2(la, false);
        xa[1] = e4m3x2_to_bf16x2(la, true);
        xa[2] = e4m3x2_to_bf16x2(ha, false);
        xa[3] = e4m3x2_to_bf16x2(ha, true);
        xb[0] = e4m3x2_to_bf16x2(lb, false);
        xb[1] = e4m3x2_to_bf16x2(lb, true);
        xb[2] = e4m3x2_to_bf16x2(hb, false);
        xb[3] = e4m3x2_to_bf16x2(hb, true);
        const bf16x8_t qs = qfrag(s);
        aA = mfma16x16x32(as_bf16x8(xa), qs, aA);
        aB = mfma16x16x32(as_bf16x8(xb), qs, aB);
        if (dim0(s) < kDVal) {
          *reinterpret_cast<uint4*>(stA + n * kVrStride + dim0(s)) = make_uint4(xa[0], xa[1], xa[2], xa[3]);
          *reinterpret_cast<uint4*>(stB + n * kVrStride + dim0(s)) = make_uint4(xb[0], xb[1], xb[2], xb[3]);
        }
      }
      // logits of rows 4g+i of both tiles (head n), log2 domain; a row id of -1
      // (or a row past the wave's rows) gets -inf
      float z[8], sc[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        sc[i] = lane_sc ? __shfl(sc_lane, 16 * t + r) : __shfl(rsa, r);
        sc[4 + i] = lane_sc ? __shfl(sc_lane, 16 * (t + 1) + r) : __shfl(rsb, r);
        const int ida = wrid[t * 16 + r];
        const int idb_any = wrid[min(t + 1, ntiles - 1) * 16 + r];
        const int idb = (t + 1 < ntiles) ? idb_any : -1;
        z[i] = ida >= 0 ? aA[i] * qk_scale_log2 * sc[i] : -INFINITY;
        z[4 + i] = idb >= 0 ? aB[i] * qk_scale_log2 * sc[4 + i] : -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])),
                       fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
      mx = max_rows16(mx);
      const float m_new = fmaxf(m_run, mx);
      float alpha = 1.f, p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run - m_new);
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = exp2f(z[i] - m_new);
      }
      l_part = l_part * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
      m_run = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) o[dt] *= alpha;
      }
      // probabilities times the row scale (which multiplies the value codes)
      u32x4_t pw;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pw[i] = f32_to_bf16_rne(p[2 * i] * sc[2 * i]) | (f32_to_bf16_rne(p[2 * i + 1] * sc[2 * i + 1]) << 16);
      const bf16x8_t pb = as_bf16x8(pw);
      // the stash writes above come first in this wave's LDS order
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const lds_v4i16 lo = vr_read_tr(stA, 4 * g, 16 * dt, n);
        const lds_v4i16 hi = vr_read_tr(stB, 4 * g, 16 * dt, n);
        u32x4_t w;
        w[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
        w[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
        w[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
        w[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
        o[dt] = mfma16x16x32(as_bf16x8(w), pb, o[dt]);
      }
      __builtin_amdgcn_wave_barrier();
    };

    // tile t sits in slot t % kMlaRing.  A wave with at most kMlaRing tiles
    // (every slice of up to 256 rows) has all of them in flight from the start
    // and runs straight through; longer ones refill a processed pair's slots
    // with the tiles kMlaRing further on.  The branches are uniform per wave
    // and hold no global load.
    static_assert(kMlaRing == 4, "two pairs of slots");
    if (few) {
      pair(0, raw[0], rs[0], raw[1], rs[1]);
      if (ntiles > 2) pair(2, raw[2], rs[2], raw[3], rs[3]);
    } else {
      for (int t0 = 0; t0 < ntiles; t0 += 4) {
        pair(t0, raw[0], rs[0], raw[1], rs[1]);
        issue(t0 + 4, raw[0], rs[0], true);
        issue(t0 + 5, raw[1], rs[1], true);
        if (t0 + 2 < ntiles) pair(t0 + 2, raw[2], rs[2], raw[3], rs[3]);
        issue(t0 + 6, raw[2], rs[2], true);
        issue(t0 + 7, raw[3], rs[3], true);
      }
    }
  }

  // merge the four waves in wave order: per head, M = max of the waves'
  // maxima, each wave weighted by 2^(m_w - M).  Each wave's accumulators go
  // to LDS as they sit in its registers ([tile dt][lane] float4s, lane
  // (n, g) holding head n, dims 16dt + 4g .. +3), so writes and reads are
  // lane-contiguous 16-byte accesses.
  const float l_w = sum_rows16(l_part);
  __syncthreads();                               // every wave is done with its stash
  float4* s_o = reinterpret_cast<float4*>(&stash[0][0][0]);   // [4 waves][32 tiles][64 lanes]
#pragma unroll
  for (int dt = 0; dt < 32; ++dt)
    s_o[(wave * 32 + dt) * kWave + lane] = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
  if (g == 0) {
    s_m[wave][n] = m_run;
    s_l[wave][n] = l_w;
  }
  __syncthreads();
  // thread j merges slots j + 256k (k = 0..7) of the [32 tiles][64 lanes]
  // grid: all of head h = j % 16
  const int h = tid & 15;
  float mw[4], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = s_m[w][h];
    M = fmaxf(M, mw[w]);
  }
  float e[4], L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    e[w] = (M != -INFINITY && mw[w] != -INFINITY) ? exp2f(mw[w] - M) : 0.f;
    L = fmaf(s_l[w][h], e[w], L);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* dst = SPLIT ? part_o + (((size_t)bp * nsplit + split) * kHq + h) * kDVal
                     : out + ((size_t)bp * kHq + h) * kDVal;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int slot = tid + 256 * k;                  // tile dt = slot / 64, lane = slot % 64
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 v = s_o[w * 32 * kWave + slot];
      acc.x = fmaf(v.x, e[w], acc.x);
      acc.y = fmaf(v.y, e[w], acc.y);
      acc.z = fmaf(v.z, e[w], acc.z);
      acc.w = fmaf(v.w, e[w], acc.w);
    }
    const int d = 16 * (slot >> 6) + 4 * ((slot & 63) >> 4);
    if (!SPLIT) acc = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    *reinterpret_cast<float4*>(dst + d) = acc;
  }
  if (tid < kHq) {
    if (!SPLIT) {
      if (lse) lse[(size_t)bp * kHq + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    } else {
      const size_t base = ((size_t)bp * nsplit + split) * kHq + h;
      part_ml[base * 2] = M;
      part_ml[base * 2 + 1] = L;
    }
  }
}

// Long slices (more than kMlaRing tiles per wave): the four waves share each
// 64-row tile (wave w gathers rows 16w..16w+15 and owns output dims
// 128w..128w+127), one tile of gathers in flight, the tile maximum combined
// through LDS, two workgroups per CU.  Its 32 accumulator registers leave room
// for the next tile's loads, where the per-wave kernel's 128 do not.
template <bool SPLIT>
__global__ __launch_bounds__(kMlaNT, 2) void mla_tile_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ pool,
    const float* __restrict__ row_scale, const int32_t* __restrict__ row_ids, int K,
    int rows_per_split, int nsplit, float qk_scale_log2, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml,
    int64_t pool_layer_rows, int hgroups) {
  __shared__ __attribute__((aligned(16))) uint16_t Vr[kTile * kVrStride];   // value tile, row-major
  __shared__ __attribute__((aligned(16))) uint16_t Pt[kHq * kPtStride];
  __shared__ float red[4][kHq];

  // blockIdx.y = (request position) * hgroups + (group of 16 heads)
  const int bp = blockIdx.y, split = blockIdx.x;
  const int rbp = bp / hgroups;
  // layer blockIdx.z of a multi-layer call: its queries, pool rows, scales,
  // outputs and partials sit one layer stride further (same row ids)
  {
    const size_t layer = blockIdx.z, BPn = gridDim.y;
    q += layer * BPn * kHq * kDLat;
    pool += layer * (size_t)pool_layer_rows * kDLat;
    if (row_scale) row_scale += layer * (size_t)pool_layer_rows;
    out += layer * BPn * kHq * kDVal;
    if (lse) lse += layer * BPn * kHq;
    if (SPLIT) {
      part_o += layer * BPn * nsplit * kHq * kDVal;
      part_ml += layer * BPn * nsplit * kHq * 2;
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int kb = split * rows_per_split;
  const int ke = min(K, kb + rows_per_split);

  // contraction step s takes dims dim0(s) .. +8 of head n (Q) and of row n (X)
  auto dim0 = [&](int s) { return 64 * (s >> 1) + 16 * g + 8 * (s & 1); };
  const int32_t* rid_p = row_ids + (size_t)rbp * K;
  const int r_local = 16 * wave + n;
  // row ids run one tile ahead of the row loads, so a tile's rows wait for one
  // round of loads, not two; this lane gathers row r_local, bytes 64v + 16g .. +16
  auto load_rid = [&](int kt) {
    const int kk = kt + r_local;
    return (kk < ke) ? rid_p[kk] : -1;
  };
  // the first row ids go out before the queries: loads complete in order, so
  // the first gather then waits for its row ids only
  int rid = load_rid(kb), rid_n = load_rid(kb + kTile);
  bf16x8_t qf[18];
  {
    const uint16_t* qp = q + ((size_t)bp * kHq + n) * kDLat;
#pragma unroll
    for (int s = 0; s < 18; ++s)
      qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + dim0(s)));
  }
  f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
  auto gather = [&](int rid, float& rs, uint4* raw) {
    rs = 0.f;
    if (rid >= 0) {
      const uint8_t* src = pool + (size_t)rid * kDLat + 16 * g;
#pragma unroll
      for (int v = 0; v < 9; ++v) raw[v] = *reinterpret_cast<const uint4*>(src + 64 * v);
      rs = row_scale ? row_scale[rid] : 1.f;
    } else {
#pragma unroll
      for (int v = 0; v < 9; ++v) raw[v] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  float rs, rs_n = 0.f;
  uint4 raw[9], raw_n[9];
  gather(rid, rs, raw);
  for (int kt = kb; kt < ke; kt += kTile) {
    int rid_nn = -1;
    if (kt + kTile < ke) {
      gather(rid_n, rs_n, raw_n);
      rid_nn = load_rid(kt + 2 * kTile);
    }
    // S^T = X . Q^T over 576 values; stash the value part (row-major) in LDS
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      const uint4 c = raw[s >> 1];
      const uint32_t lo = (s & 1) ? c.z : c.x;
      const uint32_t hi = (s & 1) ? c.w : c.y;
      u32x4_t xb;
      xb[0] = e4m3x2_to_bf16x2(lo, false);
      xb[1] = e4m3x2_to_bf16x2(lo, true);
      xb[2] = e4m3x2_to_bf16x2(hi, false);
      xb[3] = e4m3x2_to_bf16x2(hi, true);
      acc = mfma16x16x32(as_bf16x8(xb), qf[s], acc);
      if (dim0(s) < kDVal)
        *reinterpret_cast<uint4*>(Vr + r_local * kVrStride + dim0(s)) =
            make_uint4(xb[0], xb[1], xb[2], xb[3]);
    }
    // logits of this lane's rows 4g+i (head n), log2 domain
    float z[4];
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int src_lane = 4 * g + i;
      const int r_i = __shfl(rid, src_lane);
      sc[i] = __shfl(rs, src_lane);
      z[i] = (r_i >= 0) ? acc[i] * qk_scale_log2 * sc[i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mx = max_rows16(mx);
    if (g == 0) red[wave][n] = mx;
    __syncthreads();
    const float mt = fmaxf(fmaxf(red[0][n], red[1][n]), fmaxf(red[2][n], red[3][n]));
    const float m_new = fmaxf(m_run, mt);
    float alpha = 1.f, p[4] = {0.f, 0.f, 0.f, 0.f};
    if (m_new != -INFINITY) {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = exp2f(z[i] - m_new);
    }
    l_part = l_part * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    {
      const uint32_t w0 = f32_to_bf16_rne(p[0] * sc[0]) | (f32_to_bf16_rne(p[1] * sc[1]) << 16);
      const uint32_t w1 = f32_to_bf16_rne(p[2] * sc[2]) | (f32_to_bf16_rne(p[3] * sc[3]) << 16);
      *reinterpret_cast<uint2*>(Pt + n * kPtStride + 16 * wave + 4 * g) = make_uint2(w0, w1);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    m_run = m_new;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8_t pb = as_bf16x8(*reinterpret_cast<const uint4*>(Pt + n * kPtStride + 32 * c + 8 * g));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int d0 = 128 * wave + 16 * dt;
        const lds_v4i16 lo = vr_read_tr(Vr, 32 * c + 8 * g, d0, n);
        const lds_v4i16 hi = vr_read_tr(Vr, 32 * c + 8 * g + 4, d0, n);
        u32x4_t w;
        w[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
        w[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
        w[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
        w[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
        o[dt] = mfma16x16x32(as_bf16x8(w), pb, o[dt]);
      }
    }
    __syncthreads();
    rid = rid_n;
    rs = rs_n;
    rid_n = rid_nn;
#pragma unroll
    for (int v = 0; v < 9; ++v) raw[v] = raw_n[v];
  }

  float lp = l_part;
  lp = sum_rows16(lp);
  if (g == 0) red[wave][n] = lp;
  __syncthreads();
  const float l_tot = (red[0][n] + red[1][n]) + (red[2][n] + red[3][n]);
  if (!SPLIT) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* op = out + ((size_t)bp * kHq + n) * kDVal + 128 * wave + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(op + 16 * dt) =
          make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    if (lse && wave == 0 && g == 0)
      lse[(size_t)bp * kHq + n] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const size_t base = ((size_t)bp * nsplit + split) * kHq + n;
    float* op = part_o + base * kDVal + 128 * wave + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<float4*>(op + 16 * dt) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (wave == 0 && g == 0) {
      part_ml[base * 2] = m_run;
      part_ml[base * 2 + 1] = l_tot;
    }
  }
}

// fp32 path (vector ALUs), 16-row tiles; same online softmax in log2 domain.
__global__ __launch_bounds__(kMlaNT) void mla_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ pool, const int32_t* __restrict__ row_ids,
    int K, int rows_per_split, int nsplit, float qk_scale_log2, int split_mode,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, int hgroups, const int32_t* __restrict__ chunk_lo,
    const int32_t* __restrict__ chunk_hi) {
  __shared__ float Qs[kHq][kDLat];
  __shared__ float Xs[16][kDLat];
  __shared__ float Ps[kHq][16];
  __shared__ int Rs[16];
  const int bp = blockIdx.y, split = blockIdx.x;   // as in the bf16 kernel
  const int rbp = bp / hgroups;
  const int tid = threadIdx.x;
  const int h = tid >> 4, r = tid & 15;       // logits: (head, row); PV: (head, dim group)
  int kb, ke;
  if (chunk_lo) {
    kb = min(max(chunk_lo[(size_t)rbp * nsplit + split], 0), K);
    ke = min(max(chunk_hi[(size_t)rbp * nsplit + split], kb), min(kb + rows_per_split, K));
  } else {
    kb = split * rows_per_split;
    ke = min(K, kb + rows_per_split);
  }
  for (int i = tid; i < kHq * kDLat; i += kMlaNT) Qs[i / kDLat][i % kDLat] = q[(size_t)bp * kHq * kDLat + i];
  float acc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) acc[j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int32_t* rid_p = row_ids + (size_t)rbp * K;
  for (int kt = kb; kt < ke; kt += 16) {
    __syncthreads();
    if (tid < 16) Rs[tid] = (kt + tid < ke) ? rid_p[kt + tid] : -1;
    __syncthreads();
    for (int i = tid; i < 16 * kDLat; i += kMlaNT) {
      const int rr = i / kDLat, d = i % kDLat;
      const int rid = Rs[rr];
      Xs[rr][d] = rid >= 0 ? pool[(size_t)rid * kDLat + d] : 0.f;
    }
    __syncthreads();
    float z = -INFINITY;
    if (Rs[r] >= 0) {
      float dot = 0.f;
      for (int d = 0; d < kDLat; ++d) dot = fmaf(Qs[h][d], Xs[r][d], dot);
      z = dot * qk_scale_log2;
    }
    float mt = z;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mt = fmaxf(mt, __shfl_xor(mt, o));
    const float m_new = fmaxf(m_run, mt);
    float alpha = 1.f, p = 0.f;
    if (m_new != -INFINITY) {
      alpha = exp2f(m_run - m_new);
      p = exp2f(z - m_new);
    }
    float ps = p;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    Ps[h][r] = p;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float a = acc[j] * alpha;
      const int d = r + 16 * j;
      for (int rr = 0; rr < 16; ++rr) a = fmaf(Ps[h][rr], Xs[rr][d], a);
      acc[j] = a;
    }
  }
  if (!split_mode) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) out[((size_t)bp * kHq + h) * kDVal + r + 16 * j] = acc[j] * inv;
    if (lse && r == 0) lse[(size_t)bp * kHq + h] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const size_t base = ((size_t)bp * nsplit + split) * kHq + h;
#pragma unroll
    for (int j = 0; j < 32; ++j) part_o[base * kDVal + r + 16 * j] = acc[j];
    if (r == 0) {
      part_ml[base * 2] = m_run;
      part_ml[base * 2 + 1] = l_run;
    }
  }
}

// Merges the slices of each (request, position, head) in slice order: two
// waves per (request, position, head), each for 256 of the 512 output dims
// (one float4 per lane).  Every slice's maximum and sum are read at once, a
// lane per slice, and combined with wave reductions; each slice's weight is
// then broadcast from its lane while the partial outputs stream in eight
// slices at a time with no load waiting on another.
constexpr int kCombineMaxSplit = 128;   // K <= 8192 rows in tiles of 64
__global__ __launch_bounds__(kWave) void mla_combine_kernel(int nsplit, const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            float* __restrict__ out,
                                                            float* __restrict__ lse) {
  // grid (B*P, heads, 2 * layers): a wave per (request-position, head, half of the dims, layer)
  const int bp = blockIdx.x, h = blockIdx.y, half = blockIdx.z & 1;
  {
    const size_t layer = blockIdx.z >> 1, BPn = gridDim.x;   // z = 2 * layer + half
    part_o += layer * BPn * nsplit * kHq * kDVal;
    part_ml += layer * BPn * nsplit * kHq * 2;
    out += layer * BPn * kHq * kDVal;
    if (lse) lse += layer * BPn * kHq;
  }
  const int lane = threadIdx.x;
  auto ml_index = [&](int sidx) { return (((size_t)bp * nsplit + sidx) * kHq + h) * 2; };
  // the first eight slices' partial outputs go out before the maxima and sums,
  // so that up to eight slices cost one round trip: this wave's 256 of the 512
  // dims, one float4 per lane per slice
  const float4* src = reinterpret_cast<const float4*>(
                          part_o + (((size_t)bp * nsplit) * kHq + h) * kDVal + 256 * half) + lane;
  const size_t split_stride = (size_t)kHq * kDVal / 4;      // float4s from one split to the next
  float4 v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    v[u] = (u < nsplit) ? src[(size_t)u * split_stride] : make_float4(0.f, 0.f, 0.f, 0.f);
  // every split's (m, l) at once: lane s holds splits s and 64 + s
  float ms[kCombineMaxSplit / kWave], ls[kCombineMaxSplit / kWave];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kCombineMaxSplit / kWave; ++k) {
    const int sidx = kWave * k + lane;
    ms[k] = sidx < nsplit ? part_ml[ml_index(sidx)] : -INFINITY;
    ls[k] = sidx < nsplit ? part_ml[ml_index(sidx) + 1] : 0.f;
    M = fmaxf(M, ms[k]);
  }
  M = max_rows16(M);
  M = fmaxf(M, __shfl_xor(M, 1));
  M = fmaxf(M, __shfl_xor(M, 2));
  M = fmaxf(M, __shfl_xor(M, 4));
  M = fmaxf(M, __shfl_xor(M, 8));
  float wl[kCombineMaxSplit / kWave];
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < kCombineMaxSplit / kWave; ++k) {
    wl[k] = (M != -INFINITY && ms[k] != -INFINITY) ? exp2f(ms[k] - M) : 0.f;
    L = fmaf(ls[k], wl[k], L);
  }
  L = sum_rows16(L);
  L += __shfl_xor(L, 1);
  L += __shfl_xor(L, 2);
  L += __shfl_xor(L, 4);
  L += __shfl_xor(L, 8);
  // values in split order; a split's partial output is finite (zero when it saw
  // no row), and weight 0 drops it
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = (s0 + u < nsplit) ? src[(size_t)(s0 + u) * split_stride] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sidx = s0 + u;
      const float wsel = sidx < kWave ? wl[0] : wl[1];
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsel), sidx & (kWave - 1)));
      acc.x = fmaf(v[u].x, w, acc.x);
      acc.y = fmaf(v[u].y, w, acc.y);
      acc.z = fmaf(v[u].z, w, acc.z);
      acc.w = fmaf(v[u].w, w, acc.w);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  reinterpret_cast<float4*>(out + ((size_t)bp * kHq + h) * kDVal + 256 * half)[lane] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (lse && half == 0 && lane == 0)
    lse[(size_t)bp * kHq + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

__host__ inline int rows_per_split_for(int K, int nsplit) {
  int r = (K + nsplit - 1) / nsplit;
  return (r + kTile - 1) / kTile * kTile;
}

// ---- token-sharded attention (several GPUs splitting the cache by tokens,
// emulated on one): the selected rows each shard owns are a contiguous range
// of the ascending top-K, attended in chunks of at most kShardChunk rows

constexpr int kShardChunk = 256;   // rows per workgroup: each wave's 64 rows fit its ring

// One workgroup per request position: the boundaries of its shards' ranges in
// the top-K list (entry k is in shard topk[k] / shard_len; -1 entries end the
// list), then the chunk list: the chunks of shard 0, then shard 1, ...,
// chunk_first[s] the first chunk of shard s, empty chunks up to cmax.
__global__ __launch_bounds__(256) void shard_chunks_kernel(const int32_t* __restrict__ topk, int K,
                                                           int S, int shard_len, int cmax,
                                                           int32_t* __restrict__ chunk_lo,
                                                           int32_t* __restrict__ chunk_hi,
                                                           int32_t* __restrict__ chunk_first) {
  __shared__ int s_bounds[kMaxShards + 1];
  __shared__ int s_total;
  const int bp = blockIdx.x, tid = threadIdx.x;
  const int32_t* t = topk + (size_t)bp * K;
  for (int i = tid; i <= S; i += 256) s_bounds[i] = 0;
  __syncthreads();
  auto shard_of = [&](int k) {
    const int tok = t[k];
    return tok >= 0 ? min(tok / shard_len, S) : S;
  };
  // entry k starts shards prev+1 .. cur (each shard's start is written once
  // when the list is ascending)
  for (int k = tid; k <= K; k += 256) {
    const int cur = k < K ? shard_of(k) : S;
    const int prev = k > 0 ? shard_of(k - 1) : -1;
    for (int sh = prev + 1; sh <= min(cur, S); ++sh) s_bounds[sh] = k;
  }
  __syncthreads();
  if (tid < kWave) {
    int lo = 0, hi = 0, nch = 0;
    if (tid < S) {
      lo = min(max(s_bounds[tid], 0), K);
      hi = max(min(max(s_bounds[tid + 1], 0), K), lo);
      nch = (hi - lo + kShardChunk - 1) / kShardChunk;
    }
    // an ascending list needs at most K / kShardChunk + S chunks (cmax); the
    // clamps keep any other list's chunks inside the arrays
    const int incl = wave_inclusive_scan_i32(nch);
    const int first = min(incl - nch, cmax);
    const int last = min(incl, cmax);
    if (tid < S) {
      chunk_first[(size_t)bp * (S + 1) + tid] = first;
      for (int j = 0; j < last - first; ++j) {
        chunk_lo[(size_t)bp * cmax + first + j] = lo + j * kShardChunk;
        chunk_hi[(size_t)bp * cmax + first + j] = min(hi, lo + (j + 1) * kShardChunk);
      }
    }
    const int total = min(__builtin_amdgcn_readlane(incl, kWave - 1), cmax);
    if (tid == 0) {
      chunk_first[(size_t)bp * (S + 1) + S] = total;
      s_total = total;
    }
  }
  __syncthreads();
  for (int c = s_total + tid; c < cmax; c += 256) {
    chunk_lo[(size_t)bp * cmax + c] = 0;
    chunk_hi[(size_t)bp * cmax + c] = 0;
  }
}

// Per (request position, shard, head, half of the dims), one wave: the shard's
// chunks merged in chunk order into the shard's normalised output and its
// log-sum-exp (natural log), as one GPU of a token-sharded cache hands them
// over; a shard with no selected row gives 0 and -inf.
__global__ __launch_bounds__(kWave) void shard_merge_kernel(int S, int Hq, int cmax,
                                                            const int32_t* __restrict__ chunk_first,
                                                            const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            float* __restrict__ shard_out,
                                                            float* __restrict__ shard_lse) {
  const int bp = blockIdx.x / S, sh = blockIdx.x % S, h = blockIdx.y, half = blockIdx.z;
  const int lane = threadIdx.x;
  const int pbp = bp * (Hq / kHq) + h / kHq, hl = h % kHq;
  const int c0 = chunk_first[(size_t)bp * (S + 1) + sh];
  // at most K / kShardChunk <= 32 chunks for an ascending list; a lane each
  const int nc = min(chunk_first[(size_t)bp * (S + 1) + sh + 1] - c0, kWave);
  auto ml = [&](int c) { return part_ml + (((size_t)pbp * cmax + c0 + c) * kHq + hl) * 2; };
  const float m = lane < nc ? ml(lane)[0] : -INFINITY;
  const float l = lane < nc ? ml(lane)[1] : 0.f;
  float M = max_rows16(m);
  M = fmaxf(M, __shfl_xor(M, 1));
  M = fmaxf(M, __shfl_xor(M, 2));
  M = fmaxf(M, __shfl_xor(M, 4));
  M = fmaxf(M, __shfl_xor(M, 8));
  const float w = (M != -INFINITY && m != -INFINITY) ? exp2f(m - M) : 0.f;
  float L = sum_rows16(l * w);
  L += __shfl_xor(L, 1);
  L += __shfl_xor(L, 2);
  L += __shfl_xor(L, 4);
  L += __shfl_xor(L, 8);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = 0; c < nc; ++c) {
    const float wc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), c));
    const float4 v = reinterpret_cast<const float4*>(
        part_o + (((size_t)pbp * cmax + c0 + c) * kHq + hl) * kDVal + 256 * half)[lane];
    acc.x = fmaf(v.x, wc, acc.x);
    acc.y = fmaf(v.y, wc, acc.y);
    acc.z = fmaf(v.z, wc, acc.z);
    acc.w = fmaf(v.w, wc, acc.w);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  reinterpret_cast<float4*>(shard_out + (((size_t)bp * S + sh) * Hq + h) * kDVal + 256 * half)[lane] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (half == 0 && lane == 0)
    shard_lse[((size_t)bp * S + sh) * Hq + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// Per (request position, head, half of the dims), one wave: the S shards'
// outputs merged in shard order by their log-sum-exp weights,
// out = sum_s e^(lse_s - LSE) out_s with LSE = ln sum_s e^(lse_s).
__global__ __launch_bounds__(kWave) void shard_lse_combine_kernel(int S, int Hq,
                                                                  const float* __restrict__ shard_out,
                                                                  const float* __restrict__ shard_lse,
                                                                  float* __restrict__ out,
                                                                  float* __restrict__ lse) {
  const int bp = blockIdx.x, h = blockIdx.y, half = blockIdx.z, lane = threadIdx.x;
  const float ls = lane < S ? shard_lse[((size_t)bp * S + lane) * Hq + h] : -INFINITY;
  float M = max_rows16(ls);
  M = fmaxf(M, __shfl_xor(M, 1));
  M = fmaxf(M, __shfl_xor(M, 2));
  M = fmaxf(M, __shfl_xor(M, 4));
  M = fmaxf(M, __shfl_xor(M, 8));
  const float w = (M != -INFINITY && ls != -INFINITY) ? expf(ls - M) : 0.f;
  float L = sum_rows16(w);
  L += __shfl_xor(L, 1);
  L += __shfl_xor(L, 2);
  L += __shfl_xor(L, 4);
  L += __shfl_xor(L, 8);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sh = 0; sh < S; ++sh) {
    const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), sh));
    const float4 v = reinterpret_cast<const float4*>(
        shard_out + (((size_t)bp * S + sh) * Hq + h) * kDVal + 256 * half)[lane];
    acc.x = fmaf(v.x, ws, acc.x);
    acc.y = fmaf(v.y, ws, acc.y);
    acc.z = fmaf(v.z, ws, acc.z);
    acc.w = fmaf(v.w, ws, acc.w);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  reinterpret_cast<float4*>(out + ((size_t)bp * Hq + h) * kDVal + 256 * half)[lane] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (lse && half == 0 && lane == 0)
    lse[(size_t)bp * Hq + h] = L > 0.f ? M + logf(L) : -INFINITY;
}

}  // namespace

// Splits of the K rows so that one launch of L layers and G head groups fills
// about kMlaTargetWGs workgroups, with at most kMlaMaxSplitRows rows per slice
// (a slice's tiles run one after another: at 256 request-positions one slice
// each would walk 32 tiles).
int mla_num_splits(int B, int P, int K, int L, int G) {
  const int BPL = B * P * L * G;
  const int max_split = (K + kTile - 1) / kTile;
  static_assert(8192 / kTile <= kCombineMaxSplit, "one lane per slice in the combine");
  int ns = (kMlaTargetWGs + BPL - 1) / BPL;
  ns = max(ns, (K + kMlaMaxSplitRows - 1) / kMlaMaxSplitRows);
  if (ns > max_split) ns = max_split;
  if (ns < 1) ns = 1;
  const int rps = rows_per_split_for(K, ns);
  return (K + rps - 1) / rps;
}

size_t mla_workspace_bytes(int B, int P, int K, int Hq, int L) {
  const int G = Hq / kHq;
  const int ns = mla_num_splits(B, P, K, L, G);
  if (ns <= 1) return 0;
  const size_t parts = (size_t)L * B * P * ns * Hq;
  return parts * kDVal * 4 + parts * 2 * 4;
}

hipError_t launch_mla_bf16_e4m3(const BatchDims& d, int K, int L, int Hq, int64_t pool_layer_rows,
                                const uint16_t* q, const uint8_t* pool, const float* row_scale,
                                const int32_t* row_ids, float sm_scale, float* out, float* lse,
                                void* ws, hipStream_t s) {
  const int G = Hq / kHq;
  const int BPG = d.B * d.P * G;
  const int ns = mla_num_splits(d.B, d.P, K, L, G);
  const int rps = rows_per_split_for(K, ns);
  const float qk = sm_scale * kLog2e;
  // slices of three or four tiles per wave go to the per-wave kernel, whose
  // whole slice is in flight at once; longer ones, and short ones (whose waves
  // would not repay the per-wave kernel's query staging and four-way merge),
  // to the shared-tile kernel
  const bool tiles = rps > kMlaRing * 16 * 4 || rps <= 2 * 16 * 4;
  if (ns == 1) {
    if (tiles)
      hipLaunchKernelGGL((mla_tile_kernel<false>), dim3(1, BPG, L), dim3(kMlaNT), 0, s, q, pool,
                         row_scale, row_ids, K, rps, 1, qk, out, lse, nullptr, nullptr,
                         pool_layer_rows, G);
    else
      hipLaunchKernelGGL((mla_bf16_e4m3_kernel<false>), dim3(1, BPG, L), dim3(kMlaNT), 0, s, q,
                         pool, row_scale, row_ids, K, rps, 1, qk, out, lse, nullptr, nullptr,
                         pool_layer_rows, G, nullptr, nullptr);
    return hipGetLastError();
  }
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + (size_t)L * BPG * ns * kHq * kDVal;
  if (tiles)
    hipLaunchKernelGGL((mla_tile_kernel<true>), dim3(ns, BPG, L), dim3(kMlaNT), 0, s, q, pool,
                       row_scale, row_ids, K, rps, ns, qk, out, lse, part_o, part_ml,
                       pool_layer_rows, G);
  else
    hipLaunchKernelGGL((mla_bf16_e4m3_kernel<true>), dim3(ns, BPG, L), dim3(kMlaNT), 0, s, q,
                       pool, row_scale, row_ids, K, rps, ns, qk, out, lse, part_o, part_ml,
                       pool_layer_rows, G, nullptr, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(BPG, kHq, 2 * L), dim3(kWave), 0, s, ns, part_o,
                     part_ml, out, lse);
  return hipGetLastError();
}

hipError_t launch_mla_f32(const BatchDims& d, int K, int L, int Hq, int64_t pool_layer_rows,
                          const float* q, const float* pool, const int32_t* row_ids,
                          float sm_scale, float* out, float* lse, void* ws, hipStream_t s) {
  const int G = Hq / kHq;
  const int BPG = d.B * d.P * G;
  const int ns = mla_num_splits(d.B, d.P, K, L, G);
  const int rps = rows_per_split_for(K, ns);
  const float qk = sm_scale * kLog2e;
  // one launch per layer; the layers reuse the first layer's partials (same stream)
  float* part_o = static_cast<float*>(ws);
  float* part_ml = ns > 1 ? part_o + (size_t)BPG * ns * kHq * kDVal : nullptr;
  for (int l = 0; l < L; ++l) {
    const float* ql = q + (size_t)l * BPG * kHq * kDLat;
    const float* pl = pool + (size_t)l * pool_layer_rows * kDLat;
    float* ol = out + (size_t)l * BPG * kHq * kDVal;
    float* ll = lse ? lse + (size_t)l * BPG * kHq : nullptr;
    hipLaunchKernelGGL(mla_f32_kernel, dim3(ns, BPG), dim3(kMlaNT), 0, s, ql, pl, row_ids, K, rps,
                       ns, qk, ns > 1 ? 1 : 0, ol, ll, part_o, part_ml, G, nullptr, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ns > 1) {
      hipLaunchKernelGGL(mla_combine_kernel, dim3(BPG, kHq, 2), dim3(kWave), 0, s, ns, part_o,
                         part_ml, ol, ll);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

namespace {
struct ShardWs {
  int cmax;
  int32_t *chunk_lo, *chunk_hi, *chunk_first;
  float *part_o, *part_ml;
};
__host__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
__host__ inline ShardWs shard_ws(void* base, int BP, int K, int S, int Hq) {
  ShardWs w;
  w.cmax = (K + kShardChunk - 1) / kShardChunk + S;
  char* p = static_cast<char*>(base);
  const size_t nc = (size_t)BP * w.cmax;
  w.chunk_lo = reinterpret_cast<int32_t*>(p);
  p += align256(nc * 4);
  w.chunk_hi = reinterpret_cast<int32_t*>(p);
  p += align256(nc * 4);
  w.chunk_first = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)BP * (S + 1) * 4);
  w.part_o = reinterpret_cast<float*>(p);
  p += align256(nc * Hq * kDVal * 4);
  w.part_ml = reinterpret_cast<float*>(p);
  p += align256(nc * Hq * 2 * 4);
  return w;
}
}  // namespace

size_t mla_sharded_workspace_bytes(int B, int P, int K, int S, int Hq) {
  ShardWs w = shard_ws(nullptr, B * P, K, S, Hq);
  return reinterpret_cast<size_t>(w.part_ml) +
         align256((size_t)B * P * w.cmax * Hq * 2 * 4);
}

hipError_t launch_mla_sharded(const BatchDims& d, int K, int S, int Hq, bool f32, const void* q,
                              const void* pool, const float* row_scale, const int32_t* topk,
                              const int32_t* row_ids, float sm_scale, float* shard_out,
                              float* shard_lse, float* out, float* lse, void* ws, hipStream_t s) {
  const int BP = d.B * d.P, G = Hq / kHq;
  ShardWs w = shard_ws(ws, BP, K, S, Hq);
  const float qk = sm_scale * kLog2e;
  hipLaunchKernelGGL(shard_chunks_kernel, dim3(BP), dim3(256), 0, s, topk, K, S, d.T_stride / S,
                     w.cmax, w.chunk_lo, w.chunk_hi, w.chunk_first);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (f32)
    hipLaunchKernelGGL(mla_f32_kernel, dim3(w.cmax, BP * G), dim3(kMlaNT), 0, s,
                       static_cast<const float*>(q), static_cast<const float*>(pool), row_ids, K,
                       kShardChunk, w.cmax, qk, 1, nullptr, nullptr, w.part_o, w.part_ml, G,
                       w.chunk_lo, w.chunk_hi);
  else
    hipLaunchKernelGGL((mla_bf16_e4m3_kernel<true>), dim3(w.cmax, BP * G, 1), dim3(kMlaNT), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(pool),
                       row_scale, row_ids, K, kShardChunk, w.cmax, qk, nullptr, nullptr, w.part_o,
                       w.part_ml, (int64_t)0, G, w.chunk_lo, w.chunk_hi);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shard_merge_kernel, dim3(BP * S, Hq, 2), dim3(kWave), 0, s, S, Hq, w.cmax,
                     w.chunk_first, w.part_o, w.part_ml, shard_out, shard_lse);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shard_lse_combine_kernel, dim3(BP, Hq, 2), dim3(kWave), 0, s, S, Hq,
                     shard_out, shard_lse, out, lse);
  return hipGetLastError();
}

}  // namespace hs
