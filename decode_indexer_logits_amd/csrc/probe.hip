// Bandwidth probes used by the benchmark to state measured ceilings beside the
// published peaks.  They compute nothing of the method and are built into a
// library of their own (libhsprobe.so), separate from the decode-step library.
//
//   hsp_read_stream  reads n 16-byte words once, a grid-stride loop with four
//                    independent loads per thread (the plain HBM read rate)
//   hsp_host_gather  copies scattered rows from pinned host memory to HBM
//                    (zero-copy reads, the access pattern of the fault copy)
//   hsp_read_pages   reads the indexer's key pages in the indexer's own order
//                    (one workgroup of four waves per 8192-token tile, pages
//                    through the block table, two pages in flight per wave), with
//                    no products and no score writes
//
// The two read probes fold what they read into one word that is stored only
// when it equals an impossible value, so the loads are not removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 64;
constexpr int kTile = 8192;
constexpr int kRowBytes = 128;   // indexer key row (D = 128, E4M3)

__global__ __launch_bounds__(256) void read_stream_kernel(const uint4* __restrict__ p, size_t n,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ b.y ^ c.z ^ d.w;
  }
  for (; i < n; i += stride) acc ^= p[i].x;
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void read_pages_kernel(const int32_t* __restrict__ ctx_len,
                                                         int max_blocks,
                                                         const uint8_t* __restrict__ pool,
                                                         const int32_t* __restrict__ bt,
                                                         uint32_t* __restrict__ sink) {
  const int b = blockIdx.y;
  const int tile0 = blockIdx.x * kTile;
  const int T = ctx_len[b];
  if (tile0 >= T) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int npages = min(kTile / kBlock, (T - 1 - tile0) / kBlock + 1);
  const int32_t* btb = bt + (size_t)b * max_blocks + tile0 / kBlock;
  const int blk_l = lane < npages ? btb[lane] : 0;
  const int blk_h = kWave + lane < npages ? btb[kWave + lane] : 0;
  auto page_blk = [&](int pi) {
    return pi >= kWave ? __builtin_amdgcn_readlane(blk_h, pi - kWave)
                       : __builtin_amdgcn_readlane(blk_l, pi);
  };
  // lane (n, g): 16 bytes of each 64-byte half of token 16j + n's row
  auto load_page = [&](int pi, uint4* buf) {
    const uint8_t* kp = pool + (size_t)page_blk(pi) * kBlock * kRowBytes + n * kRowBytes + 16 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 2; ++v)
        buf[j * 2 + v] = *reinterpret_cast<const uint4*>(kp + 16 * j * kRowBytes + 64 * v);
  };
  constexpr int W = 4;
  const int npw = (npages - wave + W - 1) / W;
  auto page_of = [&](int k) { return min(wave + k * W, npages - 1); };
  uint32_t acc = 0;
  uint4 bufA[8], bufB[8];
  load_page(page_of(0), bufA);
  load_page(page_of(1), bufB);
  for (int k = 0; k < npw; k += 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= bufA[i].x ^ bufA[i].y ^ bufA[i].z ^ bufA[i].w;
    load_page(page_of(k + 2), bufA);
    if (k + 1 < npw) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc ^= bufB[i].x ^ bufB[i].y ^ bufB[i].z ^ bufB[i].w;
    }
    load_page(page_of(k + 3), bufB);
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.y * gridDim.x + blockIdx.x] = acc;
}

// Zero-copy gather of n rows of row_bytes (a multiple of 16) from device-mapped
// pinned host memory into device memory: rows[i] is the byte offset of row i.
// Eight rows per workgroup of 256 threads, 16-byte words.
__global__ __launch_bounds__(256) void host_gather_kernel(const uint8_t* __restrict__ host,
                                                          const int64_t* __restrict__ rows, int n,
                                                          int row_bytes, uint8_t* __restrict__ dst) {
  const int r0 = blockIdx.x * 8;
  const int words = row_bytes / 16;
  for (int w = threadIdx.x; w < 8 * words; w += 256) {
    const int i = r0 + w / words, c = w % words;
    if (i >= n) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(host + rows[i] + 16 * c);
    *reinterpret_cast<uint4*>(dst + (int64_t)i * row_bytes + 16 * c) = v;
  }
}

}  // namespace

extern "C" {

// Copies n rows of row_bytes from the device-mapped pinned host address `host`
// (offsets rows[0..n), 16-byte aligned) to dst (n * row_bytes bytes).
int hsp_host_gather(const void* host, const int64_t* rows, int n, int row_bytes, void* dst,
                    hipStream_t stream) {
  if (!host || !rows || !dst || n < 1 || row_bytes < 16 || row_bytes % 16)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(host_gather_kernel, dim3((n + 7) / 8), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(host), rows, n, row_bytes,
                     static_cast<uint8_t*>(dst));
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) from device memory `src`
// with `workgroups` workgroups of 256 threads; `sink` holds `workgroups` words
// (never written in practice).  Returns a hipError_t value.
int hsp_read_stream(const void* src, size_t bytes, int workgroups, uint32_t* sink,
                    hipStream_t stream) {
  if (!src || !sink || bytes % 16 || workgroups <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_stream_kernel, dim3(workgroups), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return (int)hipGetLastError();
}

// Reads every visible key page of B requests (ctx_len[b] tokens each, block
// table bt [B, max_blocks], pool [*, 64, 128] bytes) in the order of the
// one-position indexer.  T_stride: the token stride the grid is sized for.
// `sink` holds B * ceil(T_stride / 8192) words.
int hsp_read_pages(const int32_t* ctx_len, int B, int T_stride, int max_blocks,
                   const uint8_t* pool, const int32_t* bt, uint32_t* sink, hipStream_t stream) {
  if (!ctx_len || !pool || !bt || !sink || B <= 0 || T_stride <= 0 ||
      max_blocks * kBlock < T_stride)
    return (int)hipErrorInvalidValue;
  const dim3 grid((T_stride + kTile - 1) / kTile, B);
  hipLaunchKernelGGL(read_pages_kernel, grid, dim3(256), 0, stream, ctx_len, max_blocks, pool, bt,
                     sink);
  return (int)hipGetLastError();
}

}  // extern "C"
