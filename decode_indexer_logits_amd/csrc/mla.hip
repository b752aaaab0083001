// Sparse MLA decode attention on gfx950, absorbed (MQA) form: every head
// attends over the same selected 576-value latent rows, which serve as keys,
// and over their first 512 values, which serve as values (page "vLLM sert
// GLM-5.3 en contexte 1M sur 16 H200", section "Comment s'y prendre", option
// sparse_mla_force_mqa; the selected rows come from the indexer's top-K, page
// "Un contexte d'un million sur huit H200", section "Ce qui se passe").
//
// bf16 x E4M3 path, one workgroup = 4 waves on one (request, position) and a
// contiguous slice of its K selected rows, in 64-row tiles:
//   QK   wave w takes rows 16w..16w+15 of the tile: S^T[rows x 16 heads] on
//        the matrix cores (18 steps of v_mfma_f32_16x16x32_bf16 over the 576
//        values).  Lane (n, g) reads bytes 16g .. 16g+15 of every 64-byte
//        chunk of its row straight from HBM (the gather by row id; row ids
//        are read one tile ahead), so one wave load covers whole 64-byte
//        chunks of 16 rows; the contraction index is permuted the same way in
//        the query fragments, which a sum allows.  It converts E4M3 -> bf16 in
//        registers and also stores its value entries row-major into LDS at
//        their own dims (16-byte writes).
//   softmax  online, per head; the tile maximum is combined across the four
//        waves through LDS; the row's scale is folded into the logit and
//        into the probability that multiplies its value codes.
//   PV   wave w owns output dims 128w..128w+127: O^T[dims x heads] +=
//        V^T[dims x 64 rows] . P^T[64 rows x heads], operands read from LDS;
//        the V^T fragments come out of the row-major tile through gfx950's
//        transposing LDS read (ds_read_b64_tr_b16), so no transposed stores.
// A workgroup covers rows [split*R, split*R + R) in ascending k.  With one
// slice it writes out/lse directly; otherwise the combine kernel merges the
// slices' (O, max, sum) in slice order, so the reduction order depends only on
// the order of row_ids, never on where a row is stored.
#include "hs_common.h"
#include "hs_launch.h"

namespace hs {
namespace {

constexpr int kMlaNT = 256;
constexpr int kMlaTargetWGs = 256;   // splits of the selected rows fill about this many workgroups
constexpr int kMlaMaxSplitRows = 1024;   // and no slice walks more than 16 tiles
constexpr int kTile = 64;
constexpr int kPtStride = 72;
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
__global__ __launch_bounds__(kMlaNT, 2) void mla_bf16_e4m3_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ pool,
    const float* __restrict__ row_scale, const int32_t* __restrict__ row_ids, int K,
    int rows_per_split, int nsplit, float qk_scale_log2, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml,
    int64_t pool_layer_rows) {
  __shared__ __attribute__((aligned(16))) uint16_t Vr[kTile * kVrStride];   // value tile, row-major
  __shared__ __attribute__((aligned(16))) uint16_t Pt[kHq * kPtStride];
  __shared__ float red[4][kHq];

  const int bp = blockIdx.y, split = blockIdx.x;
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
  const int32_t* rid_p = row_ids + (size_t)bp * K;
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
    float* __restrict__ part_ml) {
  __shared__ float Qs[kHq][kDLat];
  __shared__ float Xs[16][kDLat];
  __shared__ float Ps[kHq][16];
  __shared__ int Rs[16];
  const int bp = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x;
  const int h = tid >> 4, r = tid & 15;       // logits: (head, row); PV: (head, dim group)
  const int kb = split * rows_per_split;
  const int ke = min(K, kb + rows_per_split);
  for (int i = tid; i < kHq * kDLat; i += kMlaNT) Qs[i / kDLat][i % kDLat] = q[(size_t)bp * kHq * kDLat + i];
  float acc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) acc[j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int32_t* rid_p = row_ids + (size_t)bp * K;
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
  // values: this wave's 256 of the 512 dims, one float4 per lane per split, in
  // split order; a split's partial output is finite (zero when it saw no row),
  // so every load is unconditional and weight 0 drops it
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4* src = reinterpret_cast<const float4*>(
                          part_o + (((size_t)bp * nsplit) * kHq + h) * kDVal + 256 * half) + lane;
  const size_t split_stride = (size_t)kHq * kDVal / 4;      // float4s from one split to the next
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = (s0 + u < nsplit) ? src[(size_t)(s0 + u) * split_stride] : make_float4(0.f, 0.f, 0.f, 0.f);
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

}  // namespace

// Splits of the K rows so that one launch of L layers fills about
// kMlaTargetWGs workgroups, with at most kMlaMaxSplitRows rows per slice (a
// slice's tiles run one after another: at 256 request-positions one slice
// each would walk 32 tiles).
int mla_num_splits(int B, int P, int K, int L) {
  const int BPL = B * P * L;
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
  const int ns = mla_num_splits(B, P, K, L);
  if (ns <= 1) return 0;
  const size_t parts = (size_t)L * B * P * ns * Hq;
  return parts * kDVal * 4 + parts * 2 * 4;
}

hipError_t launch_mla_bf16_e4m3(const BatchDims& d, int K, int L, int64_t pool_layer_rows,
                                const uint16_t* q, const uint8_t* pool, const float* row_scale,
                                const int32_t* row_ids, float sm_scale, float* out, float* lse,
                                void* ws, hipStream_t s) {
  const int BP = d.B * d.P;
  const int ns = mla_num_splits(d.B, d.P, K, L);
  const int rps = rows_per_split_for(K, ns);
  const float qk = sm_scale * kLog2e;
  if (ns == 1) {
    hipLaunchKernelGGL((mla_bf16_e4m3_kernel<false>), dim3(1, BP, L), dim3(kMlaNT), 0, s, q, pool,
                       row_scale, row_ids, K, rps, 1, qk, out, lse, nullptr, nullptr,
                       pool_layer_rows);
    return hipGetLastError();
  }
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + (size_t)L * BP * ns * kHq * kDVal;
  hipLaunchKernelGGL((mla_bf16_e4m3_kernel<true>), dim3(ns, BP, L), dim3(kMlaNT), 0, s, q, pool,
                     row_scale, row_ids, K, rps, ns, qk, out, lse, part_o, part_ml,
                     pool_layer_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(BP, kHq, 2 * L), dim3(kWave), 0, s, ns, part_o,
                     part_ml, out, lse);
  return hipGetLastError();
}

hipError_t launch_mla_f32(const BatchDims& d, int K, int L, int64_t pool_layer_rows,
                          const float* q, const float* pool, const int32_t* row_ids,
                          float sm_scale, float* out, float* lse, void* ws, hipStream_t s) {
  const int BP = d.B * d.P;
  const int ns = mla_num_splits(d.B, d.P, K, L);
  const int rps = rows_per_split_for(K, ns);
  const float qk = sm_scale * kLog2e;
  // one launch per layer; the layers reuse the first layer's partials (same stream)
  float* part_o = static_cast<float*>(ws);
  float* part_ml = ns > 1 ? part_o + (size_t)BP * ns * kHq * kDVal : nullptr;
  for (int l = 0; l < L; ++l) {
    const float* ql = q + (size_t)l * BP * kHq * kDLat;
    const float* pl = pool + (size_t)l * pool_layer_rows * kDLat;
    float* ol = out + (size_t)l * BP * kHq * kDVal;
    float* ll = lse ? lse + (size_t)l * BP * kHq : nullptr;
    hipLaunchKernelGGL(mla_f32_kernel, dim3(ns, BP), dim3(kMlaNT), 0, s, ql, pl, row_ids, K, rps,
                       ns, qk, ns > 1 ? 1 : 0, ol, ll, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ns > 1) {
      hipLaunchKernelGGL(mla_combine_kernel, dim3(BP, kHq, 2), dim3(kWave), 0, s, ns, part_o,
                         part_ml, ol, ll);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace hs
