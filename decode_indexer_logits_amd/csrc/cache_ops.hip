// KV append, pre-copy of completed pages to the host pool, and demotion of
// resident pages: the steps on either side of a decode step (page "Un
// contexte d'un million sur huit H200", section "Les trois états de
// résidence": full residency copies completed prefix pages to the host ahead
// of time so that they can later give up their block without a copy; mixed
// residency keeps the tail on the GPU and older pages only on the host).
//
// Every choice is made on the device and is deterministic, so the result can
// be compared bit for bit with a sequential definition:
//   - free lists are stacks (blocks[0 .. count-1], top last); an append pops
//     in request order then token order, a demotion pushes in request order
//     then page order;
//   - a pre-copy takes each request's lowest completed pages first;
//   - append and demotion are all-or-nothing: a plan kernel checks the whole
//     batch before anything is written, and the writing kernel reads its
//     verdict from the workspace.
#include "hs_common.h"
#include "hs_launch.h"

namespace hs {
namespace {

constexpr int kPlanNT = 1024;
constexpr int kCopyNT = 256;
constexpr int kPreMax = 1024;       // pages one pre-copy call may take per request

// workspace words
constexpr int kWsAppendGo = 0;      // 1 when the last append plan passed
constexpr int kWsDemoteGo = 1;      // 1 when the last demotion plan passed
constexpr int kWsDemoteBase = 2;    // free-list count before the demotion's pushes
constexpr int kWsPerRequest = 4;    // [B] prefix of pages (append) or blocks (demotion)

// One workgroup: pages each request opens (tokens t with t % 64 == 0 among
// its new ones), their prefix over requests, the range and capacity checks,
// then the pops.  With n_new <= P <= 4 a request opens at most one page.
__global__ __launch_bounds__(kPlanNT) void append_plan_kernel(
    int B, int P, int T_stride, int max_blocks, const int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ n_new, const int32_t* __restrict__ lat_blocks,
    int32_t* __restrict__ lat_count, const int32_t* __restrict__ idx_blocks,
    int32_t* __restrict__ idx_count, int32_t* __restrict__ bt, int32_t* __restrict__ idx_bt,
    float* __restrict__ idx_scale, const float* __restrict__ new_key_scale,
    int32_t* __restrict__ err, int32_t* __restrict__ ws) {
  __shared__ int scan[kPlanNT / kWave + 1];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  int total = 0;
  for (int b0 = 0; b0 < B; b0 += kPlanNT) {
    const int b = b0 + tid;
    int opened = 0;
    if (b < B) {
      const int T = ctx_len[b], n = n_new[b];
      // the page that receives the first new token must exist when it is
      // not opened by it
      const bool partial = n > 0 && T % kBlock != 0;
      if (n < 0 || n > P || T + n > T_stride ||
          (partial && (bt[(size_t)b * max_blocks + T / kBlock] < 0 ||
                       idx_bt[(size_t)b * max_blocks + T / kBlock] < 0)))
        atomicOr(&s_bad, 1);
      else
        opened = (T + n + kBlock - 1) / kBlock - (T + kBlock - 1) / kBlock;
    }
    int tot;
    const int pre = block_exclusive_scan<kPlanNT>(opened, scan, &tot);
    if (b < B) ws[kWsPerRequest + b] = total + pre;
    total += tot;
  }
  __syncthreads();
  const int nl = *lat_count, ni = *idx_count;
  const bool range_bad = s_bad != 0;
  const bool short_of_blocks = total > nl || total > ni;
  if (range_bad || short_of_blocks) {
    if (tid == 0) {
      atomicOr(err, (range_bad ? kDevErrAppendRange : 0) |
                        (short_of_blocks ? kDevErrAppendNoBlock : 0));
      ws[kWsAppendGo] = 0;
    }
    return;
  }
  for (int b = tid; b < B; b += kPlanNT) {
    const int T = ctx_len[b], n = n_new[b];
    int k = ws[kWsPerRequest + b];
    for (int i = 0; i < n; ++i) {
      const int t = T + i;
      if (t % kBlock) continue;
      const int p = t / kBlock;
      const int lb = lat_blocks[nl - 1 - k], ib = idx_blocks[ni - 1 - k];
      bt[(size_t)b * max_blocks + p] = lb;
      idx_bt[(size_t)b * max_blocks + p] = ib;
      if (idx_scale) idx_scale[ib] = new_key_scale[(size_t)b * P + i];
      ++k;
    }
  }
  __syncthreads();
  if (tid == 0) {
    *lat_count = nl - total;
    *idx_count = ni - total;
    ws[kWsAppendGo] = 1;
  }
}

// One workgroup per request: the new tokens' latent rows (every layer, with
// their scales) and indexer keys, then the context length.
__global__ __launch_bounds__(kCopyNT) void append_copy_kernel(
    int P, int max_blocks, int L, int row_bytes, int key_bytes, int64_t pool_layer_rows,
    int32_t* __restrict__ ctx_len, const int32_t* __restrict__ n_new,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ idx_bt,
    const uint8_t* __restrict__ new_rows, const float* __restrict__ new_row_scale,
    const uint8_t* __restrict__ new_keys, uint8_t* __restrict__ pool,
    float* __restrict__ row_scale, uint8_t* __restrict__ idx_pool,
    const int32_t* __restrict__ ws) {
  if (ws[kWsAppendGo] == 0) return;
  const int b = blockIdx.x;
  const int T = ctx_len[b], n = n_new[b];
  const int rv = row_bytes / 16, kv = key_bytes / 16;
  for (int i = 0; i < n; ++i) {
    const int t = T + i, p = t / kBlock, r = t % kBlock;
    const int64_t row = (int64_t)bt[(size_t)b * max_blocks + p] * kBlock + r;
    const int64_t krow = (int64_t)idx_bt[(size_t)b * max_blocks + p] * kBlock + r;
    for (int x = threadIdx.x; x < L * rv + kv; x += kCopyNT) {
      if (x < L * rv) {
        const int l = x / rv, c = x % rv;
        const uint4 v = reinterpret_cast<const uint4*>(
            new_rows + (((size_t)b * P + i) * L + l) * row_bytes)[c];
        reinterpret_cast<uint4*>(pool + ((size_t)l * pool_layer_rows + row) * row_bytes)[c] = v;
      } else {
        const int c = x - L * rv;
        reinterpret_cast<uint4*>(idx_pool + (size_t)krow * key_bytes)[c] =
            reinterpret_cast<const uint4*>(new_keys + ((size_t)b * P + i) * key_bytes)[c];
      }
    }
    if (row_scale && threadIdx.x < L)
      row_scale[(size_t)threadIdx.x * pool_layer_rows + row] =
          new_row_scale[((size_t)b * P + i) * L + threadIdx.x];
  }
  __syncthreads();
  if (threadIdx.x == 0) ctx_len[b] = T + n;
}

// One workgroup per request: the lowest completed pages that are resident
// and have no host copy (at most max_pages), found with a block-wide scan,
// then copied row block by row block to their host slot (row b*T_stride +
// 64p), every layer with its scales, and recorded in host_bt.
__global__ __launch_bounds__(kCopyNT) void precopy_kernel(
    int T_stride, int max_blocks, int L, int row_bytes, int64_t pool_layer_rows,
    int64_t host_layer_rows, int64_t host_pitch, int max_pages,
    const int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ bt, int64_t* __restrict__ host_bt,
    const uint8_t* __restrict__ pool, const float* __restrict__ row_scale,
    uint8_t* __restrict__ host_rows, float* __restrict__ host_scale) {
  __shared__ int scan[kCopyNT / kWave + 1];
  __shared__ int s_pages[kPreMax];
  const int b = blockIdx.x;
  const int full = ctx_len[b] / kBlock;
  const int32_t* btb = bt + (size_t)b * max_blocks;
  int64_t* hbb = host_bt + (size_t)b * max_blocks;
  int found = 0;
  for (int p0 = 0; p0 < full && found < max_pages; p0 += kCopyNT) {
    const int p = p0 + threadIdx.x;
    const int want = (p < full && btb[p] >= 0 && hbb[p] < 0) ? 1 : 0;
    int tot;
    const int pre = block_exclusive_scan<kCopyNT>(want, scan, &tot);
    if (want && found + pre < max_pages) s_pages[found + pre] = p;
    found = min(found + tot, max_pages);
  }
  __syncthreads();
  const int rv = row_bytes / 16;
  const int per_page = L * kBlock * rv;           // 16-byte chunks of one page, all layers
  for (int x = threadIdx.x; x < found * per_page; x += kCopyNT) {
    const int k = x / per_page, y = x % per_page;
    const int l = y / (kBlock * rv), z = y % (kBlock * rv);
    const int p = s_pages[k];
    const int r = z / rv, c = z % rv;
    const int64_t src = (int64_t)btb[p] * kBlock;
    const int64_t h = (int64_t)b * T_stride + (int64_t)p * kBlock + r;
    reinterpret_cast<uint4*>(host_rows + ((int64_t)l * host_layer_rows + h * host_pitch) *
                                             row_bytes)[c] =
        reinterpret_cast<const uint4*>(pool + ((size_t)l * pool_layer_rows + src) * row_bytes)[z];
  }
  if (row_scale)
    for (int x = threadIdx.x; x < found * L * kBlock; x += kCopyNT) {
      const int k = x / (L * kBlock), l = (x / kBlock) % L, r = x % kBlock;
      const int p = s_pages[k];
      host_scale[(int64_t)l * host_layer_rows +
                 ((int64_t)b * T_stride + (int64_t)p * kBlock + r) * host_pitch] =
          row_scale[(size_t)l * pool_layer_rows + (int64_t)btb[p] * kBlock + r];
    }
  // readers of host_bt run in later launches, after these copies complete
  for (int k = threadIdx.x; k < found; k += kCopyNT)
    hbb[s_pages[k]] = (int64_t)b * T_stride + (int64_t)s_pages[k] * kBlock;
}

// Demotion, pass 1 (one workgroup per request): how many of its lowest
// eligible pages (resident, with a host copy, outside the tail) it gives up.
__global__ __launch_bounds__(kCopyNT) void demote_count_kernel(
    int max_blocks, int tail_pages, const int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ n_demote, const int32_t* __restrict__ bt,
    const int64_t* __restrict__ host_bt, int32_t* __restrict__ ws) {
  __shared__ int scan[kCopyNT / kWave + 1];
  const int b = blockIdx.x;
  const int T = ctx_len[b];
  const int lim = T > 0 ? (T - 1) / kBlock - tail_pages + 1 : 0;   // pages [0, lim) may go
  const int want_n = max(n_demote[b], 0);
  const int32_t* btb = bt + (size_t)b * max_blocks;
  const int64_t* hbb = host_bt + (size_t)b * max_blocks;
  int found = 0;
  for (int p0 = 0; p0 < lim && found < want_n; p0 += kCopyNT) {
    const int p = p0 + threadIdx.x;
    const int ok = (p < lim && btb[p] >= 0 && hbb[p] >= 0) ? 1 : 0;
    int tot;
    block_exclusive_scan<kCopyNT>(ok, scan, &tot);
    found += tot;
  }
  if (threadIdx.x == 0) ws[kWsPerRequest + b] = min(found, want_n);
}

// Demotion, pass 2 (one workgroup): prefix over requests, capacity check,
// the new top of the free list.
__global__ __launch_bounds__(kPlanNT) void demote_plan_kernel(
    int B, int capacity, int32_t* __restrict__ count, int32_t* __restrict__ err,
    int32_t* __restrict__ ws) {
  __shared__ int scan[kPlanNT / kWave + 1];
  int total = 0;
  for (int b0 = 0; b0 < B; b0 += kPlanNT) {
    const int b = b0 + threadIdx.x;
    const int c = b < B ? ws[kWsPerRequest + b] : 0;
    int tot;
    const int pre = block_exclusive_scan<kPlanNT>(c, scan, &tot);
    if (b < B) ws[kWsPerRequest + b] = total + pre;
    total += tot;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int base = *count;
    if (base + total > capacity) {
      atomicOr(err, kDevErrDemoteFull);
      ws[kWsDemoteGo] = 0;
    } else {
      ws[kWsDemoteGo] = 1;
      ws[kWsDemoteBase] = base;
      *count = base + total;
    }
  }
}

// Demotion, pass 3 (one workgroup per request): the same pages again, their
// blocks pushed at the request's offset, and the pages marked host-only.
__global__ __launch_bounds__(kCopyNT) void demote_push_kernel(
    int max_blocks, int tail_pages, const int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ n_demote, int32_t* __restrict__ bt,
    const int64_t* __restrict__ host_bt, int32_t* __restrict__ blocks,
    const int32_t* __restrict__ ws) {
  __shared__ int scan[kCopyNT / kWave + 1];
  if (ws[kWsDemoteGo] == 0) return;
  const int b = blockIdx.x;
  const int T = ctx_len[b];
  const int lim = T > 0 ? (T - 1) / kBlock - tail_pages + 1 : 0;
  const int want_n = max(n_demote[b], 0);
  int32_t* btb = bt + (size_t)b * max_blocks;
  const int64_t* hbb = host_bt + (size_t)b * max_blocks;
  const int base = ws[kWsDemoteBase] + ws[kWsPerRequest + b];
  int found = 0;
  for (int p0 = 0; p0 < lim && found < want_n; p0 += kCopyNT) {
    const int p = p0 + threadIdx.x;
    const int blk = p < lim ? btb[p] : -1;
    const int ok = (blk >= 0 && hbb[p] >= 0) ? 1 : 0;
    int tot;
    const int pre = block_exclusive_scan<kCopyNT>(ok, scan, &tot);
    if (ok && found + pre < want_n) {
      blocks[base + found + pre] = blk;
      btb[p] = -1;
    }
    found += tot;
  }
}

}  // namespace

size_t cache_workspace_bytes(int B) { return (size_t)(kWsPerRequest + B) * sizeof(int32_t); }

hipError_t launch_append_tokens(const BatchDims& d, int32_t* ctx_len, const int32_t* n_new,
                                const ResidencyArgs& r, const void* new_rows,
                                const float* new_row_scale, int key_bytes, void* idx_pool,
                                float* idx_scale, int32_t* idx_bt, const void* new_keys,
                                const float* new_key_scale, const FreeListArgs& lat,
                                const FreeListArgs& idx, void* ws, hipStream_t s) {
  int32_t* w = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(append_plan_kernel, dim3(1), dim3(kPlanNT), 0, s, d.B, d.P, d.T_stride,
                     d.max_blocks, ctx_len, n_new, lat.blocks, lat.count, idx.blocks, idx.count,
                     const_cast<int32_t*>(r.bt), idx_bt, idx_scale, new_key_scale, r.err, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(append_copy_kernel, dim3(d.B), dim3(kCopyNT), 0, s, d.P, d.max_blocks, r.L,
                     kDLat * r.kv_bytes, key_bytes, r.pool_layer_rows, ctx_len, n_new, r.bt,
                     idx_bt, static_cast<const uint8_t*>(new_rows), new_row_scale,
                     static_cast<const uint8_t*>(new_keys), static_cast<uint8_t*>(r.pool),
                     r.row_scale, static_cast<uint8_t*>(idx_pool), w);
  return hipGetLastError();
}

hipError_t launch_precopy_pages(const BatchDims& d, const ResidencyArgs& r, int max_pages,
                                hipStream_t s) {
  hipLaunchKernelGGL(precopy_kernel, dim3(d.B), dim3(kCopyNT), 0, s, d.T_stride, d.max_blocks,
                     r.L, kDLat * r.kv_bytes, r.pool_layer_rows, r.host_layer_rows, r.host_row_pitch,
                     min(max_pages, kPreMax), d.ctx_len, r.bt,
                     const_cast<int64_t*>(r.host_bt), static_cast<const uint8_t*>(r.pool),
                     r.row_scale,
                     static_cast<uint8_t*>(const_cast<void*>(r.host_rows)),
                     const_cast<float*>(r.host_scale));
  return hipGetLastError();
}

hipError_t launch_demote_pages(const BatchDims& d, const ResidencyArgs& r,
                               const int32_t* n_demote, int tail_pages,
                               const FreeListArgs& lat, void* ws, hipStream_t s) {
  int32_t* w = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(demote_count_kernel, dim3(d.B), dim3(kCopyNT), 0, s, d.max_blocks,
                     tail_pages, d.ctx_len, n_demote, r.bt, r.host_bt, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(demote_plan_kernel, dim3(1), dim3(kPlanNT), 0, s, d.B, lat.capacity,
                     lat.count, r.err, w);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(demote_push_kernel, dim3(d.B), dim3(kCopyNT), 0, s, d.max_blocks,
                     tail_pages, d.ctx_len, n_demote, const_cast<int32_t*>(r.bt), r.host_bt,
                     lat.blocks, w);
  return hipGetLastError();
}

int precopy_max_pages() { return kPreMax; }

}  // namespace hs
