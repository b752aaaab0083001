// Device-side helpers shared by the gfx950 kernels of the decode step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

constexpr int kBlock = 64;      // tokens per page
constexpr int kDLat = 576;      // latent row: 512 compressed + 64 rotary
constexpr int kDVal = 512;      // value part of a latent row
constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Two OCP E4M3FN codes (bytes 0,1 of `w`, or bytes 2,3 when `hi`) -> two bf16
// packed in one dword, with gfx950's scaled converter at scale 1.  Every E4M3
// value is exact in bf16 (3 mantissa bits, exponents 2^-9 .. 2^8).
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                        : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight E4M3 codes (two dwords) -> eight bf16 (an MFMA operand fragment).
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4_t r;
  r[0] = e4m3x2_to_bf16x2(lo, false);
  r[1] = e4m3x2_to_bf16x2(lo, true);
  r[2] = e4m3x2_to_bf16x2(hi, false);
  r[3] = e4m3x2_to_bf16x2(hi, true);
  return __builtin_bit_cast(bf16x8_t, r);
}

// max(x, 0) for a finite float as one integer max on its bits: a set sign bit
// makes the integer negative, so -x and -0.0 both become +0.0.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  u32x4_t r = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16x16x32 bf16 matrix-core product with fp32 accumulation:
//   D[16x16] = A[16x32] * B[32x16] + C.
// Lane l holds A[l%16][8*(l/16) .. +8], B[8*(l/16) .. +8][l%16] and
// D[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(8))) int i32x8_t;

// 16x16x128 E4M3 x E4M3 matrix-core product with fp32 accumulation (the
// f8f6f4 instruction with both operand formats E4M3 and no block scales):
//   D[16x16] = A[16x128] * B[128x16] + C.
// Lane l holds A[l%16][32*(l/16) .. +32] and B[32*(l/16) .. +32][l%16], byte
// i of its eight dwords being contraction index 32*(l/16) + i; D as for the
// 16x16x32 product.  Every product of two E4M3 values is exact in fp32.
__device__ __forceinline__ f32x4_t mfma16x16x128_e4m3(i32x8_t a, i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8_t as_i32x8(uint4 lo, uint4 hi) {
  return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key);
// -0.0 is folded onto +0.0 so that equal scores get equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Sum over the four 16-lane rows of a wave, in every lane of column lane % 16:
// (row0 + row1) + (row2 + row3), the same additions as a butterfly over lane
// distances 16 then 32, done with gfx950's row-swap permutes instead of LDS
// permutes.
__device__ __forceinline__ float sum_rows16(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t y = __float_as_uint(s);
  const auto c = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Four such sums at once, each landing in one row: v[j] is this lane's part of
// column-sum j, and row g of the result holds column-sum g, with the same
// additions in the same order as sum_rows16(v[g]).  Three swaps instead of
// eight: the first permute pairs rows 0/1 and 2/3 of two sums (odd rows of
// its first operand trade places with even rows of its second), the second
// trades the upper half of the first operand with the lower half of the
// second.
__device__ __forceinline__ float sum_rows16_x4(float v0, float v1, float v2, float v3) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
  const float x = __uint_as_float(a[0]) + __uint_as_float(a[1]);   // rows 0,2: sum 0; rows 1,3: sum 1
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
  const float y = __uint_as_float(b[0]) + __uint_as_float(b[1]);   // rows 0,2: sum 2; rows 1,3: sum 3
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Maximum over the four 16-lane rows (same pattern as sum_rows16).
__device__ __forceinline__ float max_rows16(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const float s = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t y = __float_as_uint(s);
  const auto c = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// Reductions over the whole wave (every lane receives the result): quad
// butterflies and the half-row / row mirrors as DPP moves, then the two row
// swaps.  All 64 lanes must be active.
template <typename Op>
__device__ __forceinline__ uint32_t wave_allreduce_u32(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row mirror
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op((uint32_t)a[0], (uint32_t)a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op((uint32_t)c[0], (uint32_t)c[1]);
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  return (int)wave_allreduce_u32((uint32_t)v, [](uint32_t x, uint32_t y) { return x + y; });
}

__device__ __forceinline__ int wave_min_i32(int v) {
  return (int)wave_allreduce_u32(
      (uint32_t)v, [](uint32_t x, uint32_t y) { return (uint32_t)min((int)x, (int)y); });
}

__device__ __forceinline__ float wave_max_xor(float v, int from) {
  for (int o = from; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4 and 8 lanes inside each 16-lane row (lanes without a source add
// zero), then lane 15 of rows 0 and 2 into rows 1 and 3, then lane 31 into
// rows 2 and 3.  All 64 lanes must be active.
__device__ __forceinline__ int wave_inclusive_scan_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return x;
}

// Exclusive prefix sum over a block of NT threads (at most 16 waves); every
// thread must call it.  `scratch` holds NT/64 + 1 ints.  Returns the thread's
// exclusive prefix; *total receives the block sum.  Each wave scans its lanes
// with DPP, the wave sums meet in LDS, and every wave scans the (at most 16)
// wave sums in its first row: two barriers, no serial loop.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  constexpr int NW = NT / kWave;
  static_assert(NT % kWave == 0 && NW >= 1 && NW <= 16, "one to sixteen whole waves");
  const int lane = lane_id();
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int x = wave_inclusive_scan_i32(v);
  if (lane == kWave - 1) scratch[wid] = x;
  __syncthreads();
  int ws = lane < NW ? scratch[lane] : 0;
  ws += __builtin_amdgcn_update_dpp(0, ws, 0x111, 0xF, 0xF, false);
  ws += __builtin_amdgcn_update_dpp(0, ws, 0x112, 0xF, 0xF, false);
  ws += __builtin_amdgcn_update_dpp(0, ws, 0x114, 0xF, 0xF, false);
  ws += __builtin_amdgcn_update_dpp(0, ws, 0x118, 0xF, 0xF, false);
  const int before = wid ? __builtin_amdgcn_readlane(ws, wid - 1) : 0;
  *total = __builtin_amdgcn_readlane(ws, NW - 1);
  __syncthreads();   // the next call may rewrite scratch
  return before + x - v;
}

}  // namespace hs
