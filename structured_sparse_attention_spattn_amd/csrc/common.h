// Shared device-side definitions for the gfx950 kernels: vector types, MFMA
// wrappers, the kernel argument blocks and the band-tile scheduler.
//
// Band-tile scheduling (no page gives a kernel; the band itself is the
// "Making Every Head Count" Figure 1 partition): for a block of query rows
// [i_min, i_max] and head band [lo, hi] the reachable keys are
// j in [max(0, i_min - hi), i_max - lo]; a key tile is FULL when every pair
// it forms with the rows is in band, PARTIAL otherwise.  Only tiles in the
// reachable range are ever visited, so work is proportional to the band.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spattn.h"

namespace spattn {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Band bounds of every head, carried in the kernel argument block.
struct Bands {
  int32_t lo[SPATTN_MAX_HEADS];
  int32_t hi[SPATTN_MAX_HEADS];
};

// ----------------------------------------------------------------- MFMA
// 32x32x16 bf16 -> f32.  Operand layout (lane l, group g = l / 32):
//   A: row l % 32, k-slots 8g .. 8g+7;   B: column l % 32, k-slots 8g .. 8g+7
//   C: column l % 32, register r holds row 8*(r/4) + 4*g + (r%4).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 32x32x2 f32: A row l % 32, k-slot g; B column l % 32, k-slot g; C as above.
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// A-operand row permutation used for the score products: MFMA row
// r = 8a + 4g + c (a < 4, g < 2, c < 4) is fed from tile row
// 16*(a/2) + 8g + 4*(a%2) + c.  With it, accumulator registers 0..7 of a lane
// in group g hold tile rows 8g .. 8g+7 and registers 8..15 hold rows
// 16+8g .. 16+8g+7: eight contiguous rows each, which is exactly the k-slot
// set the same lane supplies to a following 32x32x16 product.
__device__ __forceinline__ int perm_row(int r) {
  const int a = r >> 3, g = (r >> 2) & 1, c = r & 3;
  return ((a >> 1) << 4) + (g << 3) + ((a & 1) << 2) + c;
}
// Tile row held in accumulator register i by a lane of group g under perm_row.
__device__ __forceinline__ int perm_reg_row(int i, int g) {
  return ((i >> 3) << 4) + (g << 3) + (i & 7);
}

// ------------------------------------------------------------- LDS tiles
// Row stride (bf16 elements) of a row-major [rows][D] tile in LDS.  The
// padding makes three access patterns bank-conflict free on the 64 x 4-byte
// LDS banks: 16-byte row reads under perm_row, 16-byte chunk stores, and the
// transposing 8-byte reads of kmajor_operand.
template <int D>
struct TileRow {
  static constexpr int kStride = D == 128 ? D + 24 : D + 8;
};

// ds_read_b64_tr_b16: within every group of 16 lanes, source lane j names 4
// consecutive bf16 M[j][0..3]; destination lane l receives
// {M[l/4][l%4], M[l/4+4][l%4], M[l/4+8][l%4], M[l/4+12][l%4]}.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(bf16x4, r);
}

// 32x32x16 operand whose k index runs down the rows of a row-major LDS tile:
// lane l (group g = l/32) receives rows kbase + 8g .. kbase + 8g + 7 of column
// n0 + (l % 32), i.e. the k-slots 8g .. 8g+7 of MFMA row/column l % 32.
__device__ __forceinline__ bf16x8 kmajor_operand(const bf16* tile, int stride, int kbase, int n0, int lane) {
  const int grp = lane >> 4, j = lane & 15, g = lane >> 5;
  const bf16* src = tile + (kbase + 8 * g + (j >> 2)) * stride + n0 + 16 * (grp & 1) + 4 * (j & 3);
  const bf16x4 a = lds_read_tr4(src);
  const bf16x4 b = lds_read_tr4(src + 4 * stride);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Global -> register -> LDS copy of ROWS rows of a [N][D] bf16 tensor, rows
// past N read as zero.  16-byte chunks, chunk index fastest across threads
// (coalesced global reads, conflict-free LDS stores).
template <int ROWS, int D, int THREADS>
struct TileCopy {
  static constexpr int kCpr = D / 8;  // chunks per row
  static constexpr int kPer = ROWS * kCpr / THREADS;
  static_assert(kPer * THREADS == ROWS * kCpr, "tile must split evenly over the threads");
  u32x4 r[kPer];
  __device__ __forceinline__ void load(const bf16* __restrict__ src, int row0, int N, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + THREADS * i;
      const int row = row0 + c / kCpr;
      r[i] = row < N ? *(const u32x4*)(src + (size_t)row * D + (c % kCpr) * 8) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(bf16* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + THREADS * i;
      *(u32x4*)(dst + (c / kCpr) * TileRow<D>::kStride + (c % kCpr) * 8) = r[i];
    }
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)x[j];
  return r;
}

// ------------------------------------------------------------ scheduler
struct KeySpan {
  int first, last;  // inclusive; empty when last < first
};

// Keys reachable from query rows [i_min, i_max] (i_max <= N-1) in band [lo, hi].
__host__ __device__ __forceinline__ KeySpan band_key_span(int i_min, int i_max, int lo, int hi) {
  KeySpan s;
  if (hi < lo || i_max < lo) {
    s.first = 0;
    s.last = -1;
    return s;
  }
  s.first = i_min - hi > 0 ? i_min - hi : 0;
  s.last = i_max - lo;
  return s;
}

// Query rows that reach key rows [j_min, j_max] in band [lo, hi], clipped to N-1.
__host__ __device__ __forceinline__ KeySpan band_query_span(int j_min, int j_max, int lo, int hi, int N) {
  KeySpan s;
  if (hi < lo || j_min + lo > N - 1) {
    s.first = 0;
    s.last = -1;
    return s;
  }
  s.first = j_min + lo;
  s.last = j_max + hi < N - 1 ? j_max + hi : N - 1;
  return s;
}

// Every pair of query rows [i_min, i_max] x key rows [j_min, j_max] in band?
__host__ __device__ __forceinline__ bool tile_full(int i_min, int i_max, int j_min, int j_max, int lo, int hi) {
  return (i_min - j_max >= lo) && (i_max - j_min <= hi);
}

// Does some pair of the two row ranges lie in band (with j <= i)?
__host__ __device__ __forceinline__ bool tile_meets(int i_min, int i_max, int j_min, int j_max, int lo, int hi) {
  if (hi < lo) return false;
  // distances covered: [i_min - j_max, i_max - j_min]; need overlap with [lo, hi]
  return (i_max - j_min >= lo) && (i_min - j_max <= hi);
}

// Workgroup -> logical work item, so that consecutive logical items land on
// the same XCD (the hardware deals workgroups to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int xcd = pid % kXcd, slot = pid / kXcd;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

}  // namespace spattn
