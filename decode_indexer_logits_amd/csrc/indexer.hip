// Indexer scores on gfx950.
//
// scores[b,p,t] = sum_h w[b,p,h] * max(0, q[b,p,h,:] . k[b,t,:]) + bias[b,t]
// for the visible tokens t <= T_b - P + p (indexer of page "Un contexte d'un
// million sur huit H200", section "Ce qui se passe"; the formula itself is the
// reading this library implements, as the page gives none).
//
// bf16 x E4M3 path.  For each (request, position) the contraction
// [H heads x D] . [D x T tokens] runs on the matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation) with heads as the M dimension
// and tokens as N, so that after the product each lane holds four heads of
// one token and the ReLU / weighted head sum is lane-local but for one sum
// over the wave's four 16-lane rows (three row-swap permutes per page cover
// its four 16-token groups).
// Keys are streamed once from HBM a 64-token page (64 x D bytes) at a time: for
// each 16-token group every lane loads 16 bytes of its token from each 64-byte
// half of the key row, so that a wave's load covers whole 64-byte halves of 16
// rows (the contraction index is permuted consistently in both operands, which
// a sum allows), converts E4M3 -> bf16 in registers (exact) and issues the
// products.
// Two pages are in flight per wave (a page is requested two pages before it
// is consumed; head weights sit in LDS so that the queries and the ring fit
// in registers), and a page's 64 scores leave in one coalesced store.  A
// page's dequant scale factors out of ReLU (positive scale), so it multiplies
// the head sum.
//
// Waves of a workgroup: with P positions, P groups of 4/P waves; each group
// keeps its position's queries in registers (H x D bf16 spread over the wave)
// and splits the tile's tokens.  Keys shared by the positions are re-read
// from the vector cache, not from HBM.
#include "hs_common.h"
#include "hs_launch.h"

#include <algorithm>
#include <mutex>

namespace hs {
namespace {

template <int P>
struct IdxCfg {
  static constexpr int WPP = (P == 1) ? 4 : (P == 2 ? 2 : 1);   // waves per position
  static constexpr int NW = P * WPP;
  static constexpr int NT = NW * kWave;
  static constexpr int TILE = 4096;                              // tokens per workgroup
};

// The multi-position kernels take a tile size at run time: up to this many
// pages per workgroup (block ids of pages l and 64 + l in lane l).
constexpr int kMpMaxPages = 2 * kWave;

// Adds two adjacent bins of a row's top-K histogram (the even one first) with
// one 64-bit atomic: same-address atomics from every die serialize, so one per
// non-empty pair instead of one per bin.  A bin counts at most 2^24 tokens, so
// the low word never carries into the high one.
__device__ __forceinline__ void hist_add_pair(uint32_t* even_bin, uint32_t lo, uint32_t hi) {
  if (lo | hi)
    atomicAdd(reinterpret_cast<unsigned long long*>(even_bin),
              (unsigned long long)lo | ((unsigned long long)hi << 32));
}

template <int P, int DK, int HT, bool HIST, int TILE>
__global__ __launch_bounds__(IdxCfg<P>::NT) void indexer_bf16_e4m3_kernel(
    const int32_t* __restrict__ ctx_len, int T_stride, int max_blocks,
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint8_t* __restrict__ pool, const float* __restrict__ scale,
    const int32_t* __restrict__ bt, const float* __restrict__ bias,
    float* __restrict__ scores, uint32_t* __restrict__ hist) {
  using Cfg = IdxCfg<P>;
  constexpr int H = 16 * HT;
  constexpr int KS = DK / 32;    // k-steps of 32
  constexpr int NV = DK / 64;    // 16-byte loads per lane per 16-token group
  constexpr int LPB = 4 * NV;    // 16-byte loads per lane per 64-token page
  const int b = blockIdx.y;
  const int T = ctx_len[b];
  const int tile0 = blockIdx.x * TILE;
  if (tile0 >= T) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int p = wave / Cfg::WPP, sub = wave % Cfg::WPP;
  const int lim = T - P + p;
  // Optional epilogue: the 2048-bin histogram of the top 11 bits of every
  // stored score's order-preserving key, per (request, position), counted in
  // LDS and added to `hist` (the first pass of the top-K radix select).
  __shared__ uint32_t sh_hist[HIST ? P * 2048 : 1];
  // The tile's scores are gathered in LDS and leave in one contiguous burst
  // at the end: 256-byte score stores interleaved with the key stream cost
  // far more HBM time than their bytes.
  __shared__ __attribute__((aligned(16))) float s_out[TILE];
  if (HIST) {
    for (int i = threadIdx.x; i < P * 2048; i += Cfg::NT) sh_hist[i] = 0;
    __syncthreads();
  }
  if (lim >= tile0) {

  // Contraction order: lane group g owns key bytes 16g .. 16g+15 of each
  // 64-byte half of a token's key, so that one 16-byte load per lane covers
  // whole 64-byte halves of 16 key rows (half the memory requests of a
  // 16-byte-strided layout).  k-step s takes dims dim0(s) .. +8 of head n in A
  // and of token n in B.
  auto dim0 = [&](int s) { return 16 * g + 64 * (s >> 1) + 8 * (s & 1); };
  // query fragments: head 16*mt + n, dims dim0(s) .. +8
  bf16x8_t qa[HT][KS];
  const uint16_t* qp = q + (size_t)(b * P + p) * H * DK;
#pragma unroll
  for (int mt = 0; mt < HT; ++mt)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qa[mt][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + (16 * mt + n) * DK + dim0(s)));
  // head weights stay in LDS (read as float4 per 16-token group) to keep
  // registers for the key ring
  __shared__ float4 sw4[P][H / 4];
  const float* wp = w + (size_t)(b * P + p) * H;
  if (sub == 0)
    for (int i = lane; i < H / 4; i += kWave) sw4[p][i] = reinterpret_cast<const float4*>(wp)[i];
  __syncthreads();

  const int npages = min(TILE / kBlock, (lim - tile0) / kBlock + 1);
  const int32_t* btb = bt + (size_t)b * max_blocks + tile0 / kBlock;
  const float* biasb = bias ? bias + (size_t)b * T_stride + tile0 : nullptr;
  const int lim_t = lim - tile0;

  // Page metadata of the whole tile is read once: lane l holds the physical
  // block and scale of pages l and 64 + l (a tile has at most 128 pages),
  // fetched later with readlane.  No load inside the page loop depends on
  // another load, so the in-order memory counter never forces a wait on pages
  // still in flight.
  static_assert(TILE == 512 || TILE == 4096 || TILE == 8192, "tile of 8, 64 or 128 pages");
  constexpr bool kTwo = TILE > 4096;
  const int blk_l = lane < npages ? btb[lane] : 0;
  const float sc_l = (scale && lane < npages) ? scale[blk_l] : 1.f;
  const int blk_h = (kTwo && kWave + lane < npages) ? btb[kWave + lane] : 0;
  const float sc_h = (kTwo && scale && kWave + lane < npages) ? scale[blk_h] : 1.f;
  auto page_blk = [&](int pi) {
    return (kTwo && pi >= kWave) ? __builtin_amdgcn_readlane(blk_h, pi - kWave)
                                 : __builtin_amdgcn_readlane(blk_l, pi);
  };
  auto page_scale = [&](int pi) {
    return __int_as_float((kTwo && pi >= kWave)
                              ? __builtin_amdgcn_readlane(__float_as_int(sc_h), pi - kWave)
                              : __builtin_amdgcn_readlane(__float_as_int(sc_l), pi));
  };
  // lane (n, g) loads, for token 16j + n of a page, bytes 16g + 64v .. +16, and
  // the bias of token 64*pi + lane.  Two pages are in flight per wave: page
  // i+2W is requested as soon as page i has been consumed (W = waves sharing
  // the position).
  auto load_page = [&](int pi, uint4* buf, float& bs) {
    const uint8_t* kp = pool + (size_t)page_blk(pi) * kBlock * DK + n * DK + 16 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < NV; ++v)
        buf[j * NV + v] = *reinterpret_cast<const uint4*>(kp + 16 * j * DK + 64 * v);
    const int tl = pi * kBlock + lane;
    bs = (biasb && tl <= lim_t) ? biasb[tl] : 0.f;
  };
  auto consume_page = [&](int pi, const uint4* buf, float bs) {
    float vj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4_t acc[HT];
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // each k-step's key fragment is converted right before its products
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint4 c = buf[j * NV + (s >> 1)];
        const uint32_t lo = (s & 1) ? c.z : c.x;
        const uint32_t hi = (s & 1) ? c.w : c.y;
        const bf16x8_t kb = e4m3x8_to_bf16x8(lo, hi);
#pragma unroll
        for (int mt = 0; mt < HT; ++mt) acc[mt] = mfma16x16x32(qa[mt][s], kb, acc[mt]);
      }
      float v = 0.f;
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) {
        const float4 wq = sw4[p][4 * mt + g];
        v = fmaf(wq.x, relu_bits(acc[mt][0]), v);
        v = fmaf(wq.y, relu_bits(acc[mt][1]), v);
        v = fmaf(wq.z, relu_bits(acc[mt][2]), v);
        v = fmaf(wq.w, relu_bits(acc[mt][3]), v);
      }
      vj[j] = v;                  // this lane's part of token 16j + n
    }
    // lane 16g + n stores token 16g + n of the page: one coalesced 256-byte store
    const float mine = sum_rows16_x4(vj[0], vj[1], vj[2], vj[3]);
    const int tl = pi * kBlock + lane;
    if (tl <= lim_t) {
      const float val = (scale ? mine * page_scale(pi) : mine) + bs;
      s_out[tl] = val;
      if (HIST) atomicAdd(&sh_hist[p * 2048 + (score_key(val) >> 21)], 1u);
    }
  };
  // Pages of this wave: pi = sub + k*W, k < npw.  Loads are unconditional
  // (past the end they re-read the last page, a cache hit) so that every
  // iteration issues the same memory operations and the compiler can wait for
  // exactly the oldest page instead of draining the queue.
  constexpr int W = Cfg::WPP;
  const int npw = (npages - sub + W - 1) / W;
  auto page_of = [&](int k) { return min(sub + k * W, npages - 1); };
  uint4 bufA[LPB], bufB[LPB];
  float bsA, bsB;
  load_page(page_of(0), bufA, bsA);
  load_page(page_of(1), bufB, bsB);
  for (int k = 0; k < npw; k += 2) {
    consume_page(sub + k * W, bufA, bsA);
    load_page(page_of(k + 2), bufA, bsA);
    if (k + 1 < npw) consume_page(sub + (k + 1) * W, bufB, bsB);
    load_page(page_of(k + 3), bufB, bsB);
  }
  }  // lim >= tile0
  __syncthreads();
  if (lim >= tile0) {
    // whole pages: entries past the visible limit are unspecified
    const int nt = min(TILE, ((lim - tile0) / kBlock + 1) * kBlock);
    float* o = scores + (size_t)(b * P + p) * T_stride + tile0;
    for (int i = 4 * threadIdx.x; i < nt; i += 4 * Cfg::NT)
      *reinterpret_cast<float4*>(o + i) = *reinterpret_cast<const float4*>(s_out + i);
  }
  if (HIST) {
    for (int i = threadIdx.x; i < P * 1024; i += Cfg::NT) {
      const int pos = i / 1024, bin = 2 * (i % 1024);
      hist_add_pair(&hist[(size_t)(b * P + pos) * 2048 + bin], sh_hist[pos * 2048 + bin],
                    sh_hist[pos * 2048 + bin + 1]);
    }
  }
}

// Several query positions (P = 2..4, speculative tokens): every position reads
// the same keys, so a workgroup loads and converts each key page once and
// shares it through LDS.  Wave w converts 16-token group w of the page
// (E4M3 -> bf16 MFMA B fragments, 16 KB per page) into one of two LDS page
// buffers while the page before is multiplied; the waves of position p
// (WPP = 4/P of them, groups split between them) read the fragments back and
// run the products against their position's queries.  One barrier per page.
// Raw key loads run three pages ahead in registers (8 bytes per token-row per
// lane, a quarter page per wave).  The tile (tokens per workgroup, up to
// kMpMaxPages pages) is chosen at launch.  The histogram epilogue packs two
// 16-bit bins per LDS word (a position sees at most 8192 tokens of a tile).
template <int P, int DK, int HT, bool HIST>
__global__ __launch_bounds__(256) void indexer_mp_kernel(
    const int32_t* __restrict__ ctx_len, int T_stride, int max_blocks,
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint8_t* __restrict__ pool, const float* __restrict__ scale,
    const int32_t* __restrict__ bt, const float* __restrict__ bias,
    float* __restrict__ scores, uint32_t* __restrict__ hist, int tile) {
  static_assert(P >= 2 && P <= 4, "multi-position kernel");
  constexpr int WPP = (P == 2) ? 2 : 1;      // waves per position (P = 3: wave 3 only converts)
  constexpr int H = 16 * HT;
  constexpr int KS = DK / 32;
  constexpr int NV = DK / 64;
  constexpr int FR = 4 * KS;                 // B fragments per page (4 groups x KS k-steps)
  __shared__ bf16x8_t sk[2][FR][kWave];      // two converted pages
  __shared__ float sbias[2][4][kWave];       // the two pages' token biases, per wave
  __shared__ uint32_t sh_hist[HIST ? P * 1024 : 1];
  __shared__ float s_scale[kMpMaxPages];     // the tile's page scales
  const int b = blockIdx.y;
  const int T = ctx_len[b];
  const int tile0 = blockIdx.x * tile;
  if (tile0 >= T) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int p = wave / WPP, sub = wave % WPP;
  const bool active = p < P;
  const int lim = T - P + (active ? p : P - 1);
  const int lim_any = T - 1;                 // last token any position sees
  if (HIST)
    for (int i = threadIdx.x; i < P * 1024; i += 256) sh_hist[i] = 0;
  const int npages = min(tile / kBlock, (lim_any - tile0) / kBlock + 1);
  const int32_t* btb = bt + (size_t)b * max_blocks + tile0 / kBlock;
  // block ids of pages l and 64 + l in lane l (read back with readlane); the
  // scales go to LDS, read once per page by the epilogue (visible after the
  // barrier that precedes the first page)
  const int blk_l = lane < npages ? btb[lane] : 0;
  const int blk_h = kWave + lane < npages ? btb[kWave + lane] : 0;
  if (wave == 0) {
    s_scale[lane] = (scale && lane < npages) ? scale[blk_l] : 1.f;
    s_scale[kWave + lane] = (scale && kWave + lane < npages) ? scale[blk_h] : 1.f;
  }
  auto page_blk = [&](int pi) {
    return pi >= kWave ? __builtin_amdgcn_readlane(blk_h, pi - kWave)
                       : __builtin_amdgcn_readlane(blk_l, pi);
  };
  auto page_scale = [&](int pi) { return s_scale[pi]; };
  // query fragments of this wave's position (same contraction order as the
  // one-position kernel)
  auto dim0 = [&](int s) { return 16 * g + 64 * (s >> 1) + 8 * (s & 1); };
  bf16x8_t qa[HT][KS];
  float wv[HT][4];
  const int pq = active ? p : 0;
  const uint16_t* qp = q + (size_t)(b * P + pq) * H * DK;
#pragma unroll
  for (int mt = 0; mt < HT; ++mt)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qa[mt][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + (16 * mt + n) * DK + dim0(s)));
  const float* wp = w + (size_t)(b * P + pq) * H;
#pragma unroll
  for (int mt = 0; mt < HT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = wp[16 * mt + 4 * g + i];
  float* out = scores + (size_t)(b * P + pq) * T_stride + tile0;
  const float* biasb = bias ? bias + (size_t)b * T_stride + tile0 : nullptr;
  const int lim_t = lim - tile0;
  // Raw keys of group `wave` of page pi (token 16*wave + n, bytes 16g + 64v)
  // and the bias of token 64*pi + lane, loaded together and without per-lane
  // conditions: pages past the tile's end re-read the last page and the bias
  // index is clamped to the request's last token (without a bias the load
  // reads ctx_len[0] and the value is dropped), so that every wait in the
  // loop is for the oldest page only.
  const int lim_any_t = lim_any - tile0;
  struct Raw { uint4 r[NV]; float bias; };
  auto load_raw = [&](int pi) {
    Raw x;
    const uint8_t* kp = pool + (size_t)page_blk(min(pi, npages - 1)) * kBlock * DK +
                        (16 * wave + n) * DK + 16 * g;
#pragma unroll
    for (int v = 0; v < NV; ++v) x.r[v] = *reinterpret_cast<const uint4*>(kp + 64 * v);
    const float* bp = biasb ? biasb + min(pi * kBlock + lane, lim_any_t)
                            : reinterpret_cast<const float*>(ctx_len);
    x.bias = *bp;
    return x;
  };
  auto convert = [&](const Raw& x, int buf) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 c = x.r[s >> 1];
      const uint32_t lo = (s & 1) ? c.z : c.x;
      const uint32_t hi = (s & 1) ? c.w : c.y;
      sk[buf][wave * KS + s][lane] = e4m3x8_to_bf16x8(lo, hi);
    }
    sbias[buf][wave][lane] = x.bias;
  };
  auto compute = [&](int pi, int buf) {
    if (!active) return;
    const int tl = pi * kBlock + lane;
    const float bs = biasb ? sbias[buf][wave][lane] : 0.f;
    float vj[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j % WPP != sub) continue;
      bf16x8_t kb[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) kb[s] = sk[buf][j * KS + s][lane];
      f32x4_t acc[HT];
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // keep issuing this wave's products back to back once they start
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int mt = 0; mt < HT; ++mt) acc[mt] = mfma16x16x32(qa[mt][s], kb[s], acc[mt]);
      __builtin_amdgcn_s_setprio(0);
      float v = 0.f;
#pragma unroll
      for (int mt = 0; mt < HT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wv[mt][i], relu_bits(acc[mt][i]), v);
      vj[j] = v;
    }
    // lane 16g + n stores token 16g + n when group g is one of this wave's
    // (the other groups' parts are zero)
    const float mine = sum_rows16_x4(vj[0], vj[1], vj[2], vj[3]);
    if (g % WPP == sub && tl <= lim_t) {
      const float val = (scale ? mine * page_scale(pi) : mine) + bs;
      out[tl] = val;
      if (HIST) {
        const uint32_t bin = score_key(val) >> 21;
        atomicAdd(&sh_hist[p * 1024 + (bin >> 1)], 1u << (16 * (bin & 1)));
      }
    }
  };
  // Software pipeline: raw loads three pages ahead, conversion one page
  // ahead.  Conversions and loads are unconditional (a page past the end is
  // converted into the idle buffer and never read), so the loop has no
  // per-page branch around memory operations.
  Raw rA = load_raw(0), rB = load_raw(1), rC = load_raw(2);
  convert(rA, 0);
  rA = load_raw(3);
  __syncthreads();
  for (int k = 0; k < npages; k += 3) {
    // page k+1 from rB, k+2 from rC, k+3 from rA
    convert(rB, (k + 1) & 1);
    rB = load_raw(k + 4);
    compute(k, k & 1);
    __syncthreads();
    convert(rC, (k + 2) & 1);
    rC = load_raw(k + 5);
    if (k + 1 < npages) compute(k + 1, (k + 1) & 1);
    __syncthreads();
    convert(rA, (k + 3) & 1);
    rA = load_raw(k + 6);
    if (k + 2 < npages) compute(k + 2, (k + 2) & 1);
    __syncthreads();
  }
  if (HIST) {
    for (int i = threadIdx.x; i < P * 1024; i += 256) {
      const uint32_t x = sh_hist[i];
      const int pos = i / 1024, bin = 2 * (i % 1024);
      hist_add_pair(hist + (size_t)(b * P + pos) * 2048 + bin, x & 0xFFFFu, x >> 16);
    }
  }
}

// E4M3 queries x E4M3 keys (D = 128; queries quantized per head by
// quantize_queries_kernel, the per-head scale already folded into w).  One
// 16x16x128 fp8 product covers 16 heads x 16 tokens over the whole key, and
// the key bytes are the B operand as loaded: no conversion at all.  Lane
// (n, g) holds contraction bytes 16g .. 16g+15 and 64+16g .. 64+16g+15 of
// head n's query and of token n's key (the same permutation of the
// contraction index in both operands), so each of its two 16-byte key loads
// covers whole 64-byte halves of 16 key rows.
// One position (P = 1): four waves split the tile's pages (8, 64 or 128 pages
// per workgroup, as in the bf16 kernel), each keeping the queries in registers
// (HT x 8 dwords) with two pages in flight.  Several positions use
// indexer_e4m3_mp_kernel below.
template <int P, int HT, bool HIST, int TILE>
__global__ __launch_bounds__(IdxCfg<P>::NT) void indexer_e4m3_kernel(
    const int32_t* __restrict__ ctx_len, int T_stride, int max_blocks,
    const uint8_t* __restrict__ q8, const float* __restrict__ w,
    const uint8_t* __restrict__ pool, const float* __restrict__ scale,
    const int32_t* __restrict__ bt, const float* __restrict__ bias,
    float* __restrict__ scores, uint32_t* __restrict__ hist) {
  using Cfg = IdxCfg<P>;
  constexpr int DK = 128;
  constexpr int H = 16 * HT;
  const int b = blockIdx.y;
  const int T = ctx_len[b];
  const int tile0 = blockIdx.x * TILE;
  if (tile0 >= T) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int p = wave / Cfg::WPP, sub = wave % Cfg::WPP;
  const int lim = T - P + p;
  __shared__ uint32_t sh_hist[HIST ? P * 2048 : 1];
  // The tile's scores are gathered in LDS and leave in one contiguous burst
  // at the end: 256-byte score stores interleaved with the key stream cost
  // far more HBM time than their bytes.
  __shared__ __attribute__((aligned(16))) float s_out[TILE];
  __shared__ float4 sw4[P][H / 4];
  if (HIST)
    for (int i = threadIdx.x; i < P * 2048; i += Cfg::NT) sh_hist[i] = 0;
  const float* wp = w + (size_t)(b * P + p) * H;
  if (sub == 0)
    for (int i = lane; i < H / 4; i += kWave) sw4[p][i] = reinterpret_cast<const float4*>(wp)[i];
  __syncthreads();

  if (lim >= tile0) {
  i32x8_t qa[HT];
  const uint8_t* qp = q8 + (size_t)(b * P + p) * H * DK + 16 * g;
#pragma unroll
  for (int mt = 0; mt < HT; ++mt) {
    const uint8_t* r = qp + (16 * mt + n) * DK;
    qa[mt] = as_i32x8(*reinterpret_cast<const uint4*>(r), *reinterpret_cast<const uint4*>(r + 64));
  }
  const int npages = min(TILE / kBlock, (lim - tile0) / kBlock + 1);
  const int32_t* btb = bt + (size_t)b * max_blocks + tile0 / kBlock;
  const float* biasb = bias ? bias + (size_t)b * T_stride + tile0 : nullptr;
  const int lim_t = lim - tile0;
  // block and scale of pages l and 64 + l in lane l (read back with readlane)
  static_assert(TILE == 512 || TILE == 4096 || TILE == 8192, "tile of 8, 64 or 128 pages");
  constexpr bool kTwo = TILE > 4096;
  const int blk_l = lane < npages ? btb[lane] : 0;
  const float sc_l = (scale && lane < npages) ? scale[blk_l] : 1.f;
  const int blk_h = (kTwo && kWave + lane < npages) ? btb[kWave + lane] : 0;
  const float sc_h = (kTwo && scale && kWave + lane < npages) ? scale[blk_h] : 1.f;
  auto page_blk = [&](int pi) {
    return (kTwo && pi >= kWave) ? __builtin_amdgcn_readlane(blk_h, pi - kWave)
                                 : __builtin_amdgcn_readlane(blk_l, pi);
  };
  auto page_scale = [&](int pi) {
    return __int_as_float((kTwo && pi >= kWave)
                              ? __builtin_amdgcn_readlane(__float_as_int(sc_h), pi - kWave)
                              : __builtin_amdgcn_readlane(__float_as_int(sc_l), pi));
  };
  // token 16j + n of the page: bytes 16g .. +16 and 64 + 16g .. +16
  auto load_page = [&](int pi, uint4* buf, float& bs) {
    const uint8_t* kp = pool + (size_t)page_blk(pi) * kBlock * DK + n * DK + 16 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      buf[2 * j] = *reinterpret_cast<const uint4*>(kp + 16 * j * DK);
      buf[2 * j + 1] = *reinterpret_cast<const uint4*>(kp + 16 * j * DK + 64);
    }
    const int tl = pi * kBlock + lane;
    bs = (biasb && tl <= lim_t) ? biasb[tl] : 0.f;
  };
  auto consume_page = [&](int pi, const uint4* buf, float bs) {
    f32x4_t acc[4][HT];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const i32x8_t kb = as_i32x8(buf[2 * j], buf[2 * j + 1]);
#pragma unroll
      for (int mt = 0; mt < HT; ++mt)
        acc[j][mt] = mfma16x16x128_e4m3(qa[mt], kb, f32x4_t{0.f, 0.f, 0.f, 0.f});
    }
    float vj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = 0.f;
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) {
        const float4 wq = sw4[p][4 * mt + g];
        v = fmaf(wq.x, relu_bits(acc[j][mt][0]), v);
        v = fmaf(wq.y, relu_bits(acc[j][mt][1]), v);
        v = fmaf(wq.z, relu_bits(acc[j][mt][2]), v);
        v = fmaf(wq.w, relu_bits(acc[j][mt][3]), v);
      }
      vj[j] = v;                  // this lane's part of token 16j + n
    }
    const float mine = sum_rows16_x4(vj[0], vj[1], vj[2], vj[3]);
    const int tl = pi * kBlock + lane;
    if (tl <= lim_t) {
      const float val = (scale ? mine * page_scale(pi) : mine) + bs;
      s_out[tl] = val;
      if (HIST) atomicAdd(&sh_hist[p * 2048 + (score_key(val) >> 21)], 1u);
    }
  };
  constexpr int W = Cfg::WPP;
  const int npw = (npages - sub + W - 1) / W;
  auto page_of = [&](int k) { return min(sub + k * W, npages - 1); };
  uint4 bufA[8], bufB[8];
  float bsA, bsB;
  load_page(page_of(0), bufA, bsA);
  load_page(page_of(1), bufB, bsB);
  for (int k = 0; k < npw; k += 2) {
    consume_page(sub + k * W, bufA, bsA);
    load_page(page_of(k + 2), bufA, bsA);
    if (k + 1 < npw) consume_page(sub + (k + 1) * W, bufB, bsB);
    load_page(page_of(k + 3), bufB, bsB);
  }
  }  // lim >= tile0
  __syncthreads();
  if (lim >= tile0) {
    // whole pages: entries past the visible limit are unspecified
    const int nt = min(TILE, ((lim - tile0) / kBlock + 1) * kBlock);
    float* o = scores + (size_t)(b * P + p) * T_stride + tile0;
    for (int i = 4 * threadIdx.x; i < nt; i += 4 * Cfg::NT)
      *reinterpret_cast<float4*>(o + i) = *reinterpret_cast<const float4*>(s_out + i);
  }
  if (HIST) {
    for (int i = threadIdx.x; i < P * 1024; i += Cfg::NT) {
      const int pos = i / 1024, bin = 2 * (i % 1024);
      hist_add_pair(&hist[(size_t)(b * P + pos) * 2048 + bin], sh_hist[pos * 2048 + bin],
                    sh_hist[pos * 2048 + bin + 1]);
    }
  }
}

// E4M3 x E4M3 with several query positions (P = 2..4): every position reads
// the same keys, so the workgroup loads each page once and shares the raw
// bytes through LDS.  Wave w loads 16-token group w of a page (each lane the
// 32 bytes that are its B operand) into one of two LDS page buffers while
// the page before is multiplied; the waves of position p (4/P of them at
// P = 2, one otherwise; at P = 3 wave 3 only loads) read every group back
// and run their products.  One barrier per page; raw loads run three pages
// ahead in registers.  The tile (up to kMpMaxPages pages) is chosen at
// launch.  The histogram epilogue packs two 16-bit bins per LDS word (a
// position sees at most 8192 tokens of a tile).
template <int P, int HT, bool HIST>
__global__ __launch_bounds__(256) void indexer_e4m3_mp_kernel(
    const int32_t* __restrict__ ctx_len, int T_stride, int max_blocks,
    const uint8_t* __restrict__ q8, const float* __restrict__ w,
    const uint8_t* __restrict__ pool, const float* __restrict__ scale,
    const int32_t* __restrict__ bt, const float* __restrict__ bias,
    float* __restrict__ scores, uint32_t* __restrict__ hist, int tile) {
  static_assert(P >= 2 && P <= 4, "multi-position kernel");
  constexpr int DK = 128;
  constexpr int WPP = (P == 2) ? 2 : 1;
  constexpr int H = 16 * HT;
  __shared__ uint4 sk[2][4][2][kWave];       // two pages: [group][half][lane]
  __shared__ float sbias[2][4][kWave];       // the two pages' token biases, per wave
  __shared__ uint32_t sh_hist[HIST ? P * 1024 : 1];
  __shared__ float s_scale[kMpMaxPages];     // the tile's page scales
  const int b = blockIdx.y;
  const int T = ctx_len[b];
  const int tile0 = blockIdx.x * tile;
  if (tile0 >= T) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int p = wave / WPP, sub = wave % WPP;
  const bool active = p < P;
  const int lim = T - P + (active ? p : P - 1);
  const int lim_any = T - 1;
  if (HIST)
    for (int i = threadIdx.x; i < P * 1024; i += 256) sh_hist[i] = 0;
  const int npages = min(tile / kBlock, (lim_any - tile0) / kBlock + 1);
  const int32_t* btb = bt + (size_t)b * max_blocks + tile0 / kBlock;
  // block ids of pages l and 64 + l in lane l (read back with readlane); the
  // scales go to LDS, read once per page by the epilogue (visible after the
  // barrier that precedes the first page)
  const int blk_l = lane < npages ? btb[lane] : 0;
  const int blk_h = kWave + lane < npages ? btb[kWave + lane] : 0;
  if (wave == 0) {
    s_scale[lane] = (scale && lane < npages) ? scale[blk_l] : 1.f;
    s_scale[kWave + lane] = (scale && kWave + lane < npages) ? scale[blk_h] : 1.f;
  }
  auto page_blk = [&](int pi) {
    return pi >= kWave ? __builtin_amdgcn_readlane(blk_h, pi - kWave)
                       : __builtin_amdgcn_readlane(blk_l, pi);
  };
  auto page_scale = [&](int pi) { return s_scale[pi]; };
  const int pq = active ? p : 0;
  i32x8_t qa[HT];
  float wv[HT][4];
  {
    const uint8_t* qp = q8 + (size_t)(b * P + pq) * H * DK + 16 * g;
    const float* wp = w + (size_t)(b * P + pq) * H;
#pragma unroll
    for (int mt = 0; mt < HT; ++mt) {
      const uint8_t* r = qp + (16 * mt + n) * DK;
      qa[mt] = as_i32x8(*reinterpret_cast<const uint4*>(r), *reinterpret_cast<const uint4*>(r + 64));
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[mt][i] = wp[16 * mt + 4 * g + i];
    }
  }
  float* out = scores + (size_t)(b * P + pq) * T_stride + tile0;
  const float* biasb = bias ? bias + (size_t)b * T_stride + tile0 : nullptr;
  const int lim_t = lim - tile0;
  // token 16*wave + n of page pi: key bytes 16g .. +16 and 64 + 16g .. +16,
  // with the bias of token 64*pi + lane; no per-lane condition on any load
  // (clamped page and bias index; without a bias the load reads ctx_len[0]
  // and the value is dropped), so every wait in the loop is for the oldest
  // page only.
  const int lim_any_t = lim_any - tile0;
  struct Raw { uint4 lo, hi; float bias; };
  auto load_raw = [&](int pi) {
    const uint8_t* kp = pool + (size_t)page_blk(min(pi, npages - 1)) * kBlock * DK +
                        (16 * wave + n) * DK + 16 * g;
    const float* bp = biasb ? biasb + min(pi * kBlock + lane, lim_any_t)
                            : reinterpret_cast<const float*>(ctx_len);
    return Raw{*reinterpret_cast<const uint4*>(kp), *reinterpret_cast<const uint4*>(kp + 64), *bp};
  };
  auto stash = [&](const Raw& r, int buf) {
    sk[buf][wave][0][lane] = r.lo;
    sk[buf][wave][1][lane] = r.hi;
    sbias[buf][wave][lane] = r.bias;
  };
  auto compute = [&](int pi, int buf) {
    if (!active) return;
    const int tl = pi * kBlock + lane;
    const float bs = biasb ? sbias[buf][wave][lane] : 0.f;
    float vj[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j % WPP != sub) continue;
      const i32x8_t kb = as_i32x8(sk[buf][j][0][lane], sk[buf][j][1][lane]);
      f32x4_t acc[HT];
#pragma unroll
      for (int mt = 0; mt < HT; ++mt)
        acc[mt] = mfma16x16x128_e4m3(qa[mt], kb, f32x4_t{0.f, 0.f, 0.f, 0.f});
      float v = 0.f;
#pragma unroll
      for (int mt = 0; mt < HT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wv[mt][i], relu_bits(acc[mt][i]), v);
      vj[j] = v;
    }
    const float mine = sum_rows16_x4(vj[0], vj[1], vj[2], vj[3]);
    if (g % WPP == sub && tl <= lim_t) {
      const float val = (scale ? mine * page_scale(pi) : mine) + bs;
      out[tl] = val;
      if (HIST) {
        const uint32_t bin = score_key(val) >> 21;
        atomicAdd(&sh_hist[p * 1024 + (bin >> 1)], 1u << (16 * (bin & 1)));
      }
    }
  };
  // loads and stashes are unconditional (a page past the end lands in the
  // idle buffer and is never read)
  Raw rA = load_raw(0), rB = load_raw(1), rC = load_raw(2);
  stash(rA, 0);
  rA = load_raw(3);
  __syncthreads();
  for (int k = 0; k < npages; k += 3) {
    stash(rB, (k + 1) & 1);
    rB = load_raw(k + 4);
    compute(k, k & 1);
    __syncthreads();
    stash(rC, (k + 2) & 1);
    rC = load_raw(k + 5);
    if (k + 1 < npages) compute(k + 1, (k + 1) & 1);
    __syncthreads();
    stash(rA, (k + 3) & 1);
    rA = load_raw(k + 6);
    if (k + 2 < npages) compute(k + 2, (k + 2) & 1);
    __syncthreads();
  }
  if (HIST) {
    for (int i = threadIdx.x; i < P * 1024; i += 256) {
      const uint32_t x = sh_hist[i];
      const int pos = i / 1024, bin = 2 * (i % 1024);
      hist_add_pair(hist + (size_t)(b * P + pos) * 2048 + bin, x & 0xFFFFu, x >> 16);
    }
  }
}

// Per-head E4M3 quantization of bf16 indexer queries, one wave per
// (request, position, head) row of DK values: amax by an integer max over the
// magnitudes' bits, then binary32 inv = 448 / amax, x = q * inv, and the
// hardware's round-to-nearest-even conversion to E4M3; rows with
// amax < 2^-64 become zero.  w_scaled = w * (amax / 448).
template <int DK>
__global__ __launch_bounds__(256) void quantize_queries_kernel(
    int rows, const uint16_t* __restrict__ q, const float* __restrict__ w,
    uint8_t* __restrict__ q8, float* __restrict__ w_scaled) {
  constexpr int PER = DK / kWave;   // 1 or 2 values per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  float x[PER];
  if (PER == 2) {
    const uint32_t u = reinterpret_cast<const uint32_t*>(q + (size_t)row * DK)[lane];
    x[0] = __uint_as_float(u << 16);
    x[PER - 1] = __uint_as_float(u & 0xFFFF0000u);
  } else {
    x[0] = __uint_as_float((uint32_t)q[(size_t)row * DK + lane] << 16);
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  m = wave_allreduce_u32(m, [](uint32_t a, uint32_t c) { return max(a, c); });
  const float amax = __uint_as_float(m);
  const bool live = amax >= 0x1p-64f;
  const float inv = live ? 448.f / amax : 0.f;
  if (PER == 2) {
    const uint32_t c = live ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[0] * inv, x[PER - 1] * inv, 0, false) & 0xFFFFu : 0u;
    reinterpret_cast<uint16_t*>(q8 + (size_t)row * DK)[lane] = (uint16_t)c;
  } else {
    const uint32_t c = live ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[0] * inv, 0.f, 0, false) & 0xFFu : 0u;
    q8[(size_t)row * DK + lane] = (uint8_t)c;
  }
  if (lane == 0) w_scaled[row] = w[row] * (live ? amax / 448.f : 0.f);
}

// fp32 path (vector ALUs): one thread per (position, token).
__global__ __launch_bounds__(256) void indexer_f32_kernel(
    const int32_t* __restrict__ ctx_len, int T_stride, int max_blocks, int P, int H, int DK,
    const float* __restrict__ q, const float* __restrict__ w, const float* __restrict__ pool,
    const int32_t* __restrict__ bt, const float* __restrict__ bias, float* __restrict__ scores) {
  extern __shared__ float sq[];   // H*DK queries then H weights
  const int bp = blockIdx.y;
  const int b = bp / P, p = bp % P;
  const int T = ctx_len[b];
  const int lim = T - P + p;
  const int t0 = blockIdx.x * 256;
  if (t0 > lim) return;
  for (int i = threadIdx.x; i < H * DK; i += 256) sq[i] = q[(size_t)bp * H * DK + i];
  for (int i = threadIdx.x; i < H; i += 256) sq[H * DK + i] = w[(size_t)bp * H + i];
  __syncthreads();
  const int t = t0 + threadIdx.x;
  if (t > lim) return;
  const int blk = bt[(size_t)b * max_blocks + (t >> 6)];
  const float4* kp = reinterpret_cast<const float4*>(pool + ((size_t)blk * kBlock + (t & 63)) * DK);
  float acc = 0.f;
  for (int h = 0; h < H; ++h) {
    const float* qh = sq + h * DK;
    float dot = 0.f;
    for (int d4 = 0; d4 < DK / 4; ++d4) {
      const float4 k = kp[d4];
      dot = fmaf(qh[4 * d4 + 0], k.x, dot);
      dot = fmaf(qh[4 * d4 + 1], k.y, dot);
      dot = fmaf(qh[4 * d4 + 2], k.z, dot);
      dot = fmaf(qh[4 * d4 + 3], k.w, dot);
    }
    acc = fmaf(sq[H * DK + h], fmaxf(dot, 0.f), acc);
  }
  if (bias) acc += bias[(size_t)b * T_stride + t];
  scores[(size_t)bp * T_stride + t] = acc;
}

// Workgroups of `kernel` (256 threads) resident on the current device at
// once: its occupancy per CU times the CUs, cached per kernel and device.
int resident_workgroups(const void* kernel) {
  struct Entry { const void* k; int dev, n; };
  static Entry cache[64];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].k == kernel && cache[i].dev == dev) return cache[i].n;
  int cus = 0, per_cu = 0;
  const bool ok =
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) == hipSuccess &&
      cus > 0 && per_cu > 0;
  if (!ok) {
    // not cached; the error it left is cleared so that the launch reports its own.
    // Fallback: four workgroups on each of 256 CUs.
    (void)hipGetLastError();
    return 1024;
  }
  const int n = cus * per_cu;
  if (used < 64) cache[used++] = Entry{kernel, dev, n};
  return n;
}

// Tokens per workgroup of the multi-position kernels: every request gets an
// equal share of one round of resident workgroups (one start-up and one tail
// per CU slot instead of a partly filled second round: MTP3, 64 requests of
// up to 86K tokens at four workgroups per CU, went from 22 tiles of 4096 tokens
// per request to 16 of 5440), in whole pages, at most kMpMaxPages pages.  Small
// batches take small tiles: four positions of 3 requests of 7K tokens run in
// 12.5 us with one-page tiles against 27.6 us with 16-page and 84 us with
// 64-page ones (bf16 queries), so there is no lower bound beyond one page.
int mp_tile(const BatchDims& d, const void* kernel) {
  const int per_req = std::max(1, resident_workgroups(kernel) / std::max(d.B, 1));
  int tile = (d.T_stride + per_req - 1) / per_req;
  tile = (tile + kBlock - 1) / kBlock * kBlock;
  return std::min(std::max(tile, kBlock), kMpMaxPages * kBlock);
}

template <int P, int DK, int HT>
hipError_t launch_mfma(const BatchDims& d, const uint16_t* q, const float* w, const uint8_t* pool,
                       const float* scale, const int32_t* bt, const float* bias, float* scores,
                       uint32_t* hist, hipStream_t s) {
  using Cfg = IdxCfg<P>;
  dim3 grid((d.T_stride + Cfg::TILE - 1) / Cfg::TILE, d.B);
  if (P > 1) {
    constexpr int PM = P > 1 ? P : 2;
    const void* k = hist ? reinterpret_cast<const void*>(&indexer_mp_kernel<PM, DK, HT, true>)
                         : reinterpret_cast<const void*>(&indexer_mp_kernel<PM, DK, HT, false>);
    const int tile = mp_tile(d, k);
    const dim3 gm((d.T_stride + tile - 1) / tile, d.B);
    if (hist)
      hipLaunchKernelGGL((indexer_mp_kernel<PM, DK, HT, true>), gm, dim3(256), 0, s, d.ctx_len,
                         d.T_stride, d.max_blocks, q, w, pool, scale, bt, bias, scores, hist, tile);
    else
      hipLaunchKernelGGL((indexer_mp_kernel<PM, DK, HT, false>), gm, dim3(256), 0, s, d.ctx_len,
                         d.T_stride, d.max_blocks, q, w, pool, scale, bt, bias, scores, hist, tile);
    return hipGetLastError();
  }
  // 128-page tiles when they still give every CU two workgroups (one round of
  // workgroups instead of two: fewer start-ups with no keys in flight); 8-page
  // tiles when 64-page ones would leave most of the chip idle (few short
  // requests: 8 requests of 32K tokens make 64 workgroups of 4096 tokens)
  if ((size_t)d.B * ((d.T_stride + 4095) / 4096) < 256) {
    const dim3 g8((d.T_stride + 511) / 512, d.B);
    if (hist)
      hipLaunchKernelGGL((indexer_bf16_e4m3_kernel<P, DK, HT, true, 512>), g8, dim3(Cfg::NT), 0,
                         s, d.ctx_len, d.T_stride, d.max_blocks, q, w, pool, scale, bt, bias,
                         scores, hist);
    else
      hipLaunchKernelGGL((indexer_bf16_e4m3_kernel<P, DK, HT, false, 512>), g8, dim3(Cfg::NT), 0,
                         s, d.ctx_len, d.T_stride, d.max_blocks, q, w, pool, scale, bt, bias,
                         scores, hist);
    return hipGetLastError();
  }
  if ((size_t)d.B * ((d.T_stride + 8191) / 8192) >= 512) {
    const dim3 g2((d.T_stride + 8191) / 8192, d.B);
    if (hist)
      hipLaunchKernelGGL((indexer_bf16_e4m3_kernel<P, DK, HT, true, 8192>), g2, dim3(Cfg::NT), 0,
                         s, d.ctx_len, d.T_stride, d.max_blocks, q, w, pool, scale, bt, bias,
                         scores, hist);
    else
      hipLaunchKernelGGL((indexer_bf16_e4m3_kernel<P, DK, HT, false, 8192>), g2, dim3(Cfg::NT), 0,
                         s, d.ctx_len, d.T_stride, d.max_blocks, q, w, pool, scale, bt, bias,
                         scores, hist);
    return hipGetLastError();
  }
  if (hist)
    hipLaunchKernelGGL((indexer_bf16_e4m3_kernel<P, DK, HT, true, 4096>), grid, dim3(Cfg::NT), 0,
                       s, d.ctx_len, d.T_stride, d.max_blocks, q, w, pool, scale, bt, bias,
                       scores, hist);
  else
    hipLaunchKernelGGL((indexer_bf16_e4m3_kernel<P, DK, HT, false, 4096>), grid, dim3(Cfg::NT), 0,
                       s, d.ctx_len, d.T_stride, d.max_blocks, q, w, pool, scale, bt, bias,
                       scores, hist);
  return hipGetLastError();
}

template <int P, int DK>
hipError_t dispatch_ht(int HT, const BatchDims& d, const uint16_t* q, const float* w,
                       const uint8_t* pool, const float* scale, const int32_t* bt,
                       const float* bias, float* scores, uint32_t* hist, hipStream_t s) {
  switch (HT) {
    case 1: return launch_mfma<P, DK, 1>(d, q, w, pool, scale, bt, bias, scores, hist, s);
    case 2: return launch_mfma<P, DK, 2>(d, q, w, pool, scale, bt, bias, scores, hist, s);
    case 3: return launch_mfma<P, DK, 3>(d, q, w, pool, scale, bt, bias, scores, hist, s);
    case 4: return launch_mfma<P, DK, 4>(d, q, w, pool, scale, bt, bias, scores, hist, s);
  }
  return hipErrorInvalidValue;
}

template <int P>
hipError_t dispatch_dk(int DK, int HT, const BatchDims& d, const uint16_t* q, const float* w,
                       const uint8_t* pool, const float* scale, const int32_t* bt,
                       const float* bias, float* scores, uint32_t* hist, hipStream_t s) {
  if (DK == 64) return dispatch_ht<P, 64>(HT, d, q, w, pool, scale, bt, bias, scores, hist, s);
  if (DK == 128) return dispatch_ht<P, 128>(HT, d, q, w, pool, scale, bt, bias, scores, hist, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_indexer_bf16_e4m3(const BatchDims& d, int H, int DK, const uint16_t* q,
                                   const float* w, const uint8_t* pool, const float* scale,
                                   const int32_t* bt, const float* bias, float* scores,
                                   uint32_t* hist, hipStream_t s) {
  const int HT = H / 16;
  switch (d.P) {
    case 1: return dispatch_dk<1>(DK, HT, d, q, w, pool, scale, bt, bias, scores, hist, s);
    case 2: return dispatch_dk<2>(DK, HT, d, q, w, pool, scale, bt, bias, scores, hist, s);
    case 3: return dispatch_dk<3>(DK, HT, d, q, w, pool, scale, bt, bias, scores, hist, s);
    case 4: return dispatch_dk<4>(DK, HT, d, q, w, pool, scale, bt, bias, scores, hist, s);
  }
  return hipErrorInvalidValue;
}

namespace {

template <int P, int HT, int TILE>
hipError_t launch_e4m3_one(const BatchDims& d, const uint8_t* q8, const float* w,
                           const uint8_t* pool, const float* scale, const int32_t* bt,
                           const float* bias, float* scores, uint32_t* hist, hipStream_t s) {
  using Cfg = IdxCfg<P>;
  const dim3 grid((d.T_stride + TILE - 1) / TILE, d.B);
  if (hist)
    hipLaunchKernelGGL((indexer_e4m3_kernel<P, HT, true, TILE>), grid, dim3(Cfg::NT), 0, s,
                       d.ctx_len, d.T_stride, d.max_blocks, q8, w, pool, scale, bt, bias, scores,
                       hist);
  else
    hipLaunchKernelGGL((indexer_e4m3_kernel<P, HT, false, TILE>), grid, dim3(Cfg::NT), 0, s,
                       d.ctx_len, d.T_stride, d.max_blocks, q8, w, pool, scale, bt, bias, scores,
                       hist);
  return hipGetLastError();
}

template <int P, int HT>
hipError_t launch_e4m3_ht(const BatchDims& d, const uint8_t* q8, const float* w,
                          const uint8_t* pool, const float* scale, const int32_t* bt,
                          const float* bias, float* scores, uint32_t* hist, hipStream_t s) {
  if constexpr (P > 1) {
    constexpr int PM = P > 1 ? P : 2;
    const void* k = hist ? reinterpret_cast<const void*>(&indexer_e4m3_mp_kernel<PM, HT, true>)
                         : reinterpret_cast<const void*>(&indexer_e4m3_mp_kernel<PM, HT, false>);
    const int tile = mp_tile(d, k);
    const dim3 gm((d.T_stride + tile - 1) / tile, d.B);
    if (hist)
      hipLaunchKernelGGL((indexer_e4m3_mp_kernel<PM, HT, true>), gm, dim3(256), 0, s, d.ctx_len,
                         d.T_stride, d.max_blocks, q8, w, pool, scale, bt, bias, scores, hist,
                         tile);
    else
      hipLaunchKernelGGL((indexer_e4m3_mp_kernel<PM, HT, false>), gm, dim3(256), 0, s, d.ctx_len,
                         d.T_stride, d.max_blocks, q8, w, pool, scale, bt, bias, scores, hist,
                         tile);
    return hipGetLastError();
  } else {
    // the one-position kernel takes the bf16 kernel's tiles: 128 pages when that
    // still gives two workgroups per CU, 8 when 64 would leave most CUs idle
    // (128K: 106.6 against 108.7 us with 64-page tiles)
    const size_t B = d.B;
    if (B * ((d.T_stride + 4095) / 4096) < 256)
      return launch_e4m3_one<P, HT, 512>(d, q8, w, pool, scale, bt, bias, scores, hist, s);
    if (B * ((d.T_stride + 8191) / 8192) >= 512)
      return launch_e4m3_one<P, HT, 8192>(d, q8, w, pool, scale, bt, bias, scores, hist, s);
    return launch_e4m3_one<P, HT, 4096>(d, q8, w, pool, scale, bt, bias, scores, hist, s);
  }
}

template <int P>
hipError_t launch_e4m3_p(int HT, const BatchDims& d, const uint8_t* q8, const float* w,
                         const uint8_t* pool, const float* scale, const int32_t* bt,
                         const float* bias, float* scores, uint32_t* hist, hipStream_t s) {
  switch (HT) {
    case 1: return launch_e4m3_ht<P, 1>(d, q8, w, pool, scale, bt, bias, scores, hist, s);
    case 2: return launch_e4m3_ht<P, 2>(d, q8, w, pool, scale, bt, bias, scores, hist, s);
    case 3: return launch_e4m3_ht<P, 3>(d, q8, w, pool, scale, bt, bias, scores, hist, s);
    case 4: return launch_e4m3_ht<P, 4>(d, q8, w, pool, scale, bt, bias, scores, hist, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_indexer_e4m3(const BatchDims& d, int H, const uint8_t* q8, const float* w,
                               const uint8_t* pool, const float* scale, const int32_t* bt,
                               const float* bias, float* scores, uint32_t* hist, hipStream_t s) {
  const int HT = H / 16;
  switch (d.P) {
    case 1: return launch_e4m3_p<1>(HT, d, q8, w, pool, scale, bt, bias, scores, hist, s);
    case 2: return launch_e4m3_p<2>(HT, d, q8, w, pool, scale, bt, bias, scores, hist, s);
    case 3: return launch_e4m3_p<3>(HT, d, q8, w, pool, scale, bt, bias, scores, hist, s);
    case 4: return launch_e4m3_p<4>(HT, d, q8, w, pool, scale, bt, bias, scores, hist, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quantize_queries(int rows, int DK, const uint16_t* q, const float* w,
                                   uint8_t* q8, float* w_scaled, hipStream_t s) {
  const dim3 grid((rows + 3) / 4);
  if (DK == 64)
    hipLaunchKernelGGL(quantize_queries_kernel<64>, grid, dim3(256), 0, s, rows, q, w, q8,
                       w_scaled);
  else if (DK == 128)
    hipLaunchKernelGGL(quantize_queries_kernel<128>, grid, dim3(256), 0, s, rows, q, w, q8,
                       w_scaled);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_indexer_f32(const BatchDims& d, int H, int DK, const float* q, const float* w,
                              const float* pool, const int32_t* bt, const float* bias,
                              float* scores, hipStream_t s) {
  dim3 grid((d.T_stride + 255) / 256, d.B * d.P);
  const size_t shm = (size_t)(H * DK + H) * sizeof(float);
  hipLaunchKernelGGL(indexer_f32_kernel, grid, dim3(256), shm, s, d.ctx_len, d.T_stride,
                     d.max_blocks, d.P, H, DK, q, w, pool, bt, bias, scores);
  return hipGetLastError();
}

}  // namespace hs
