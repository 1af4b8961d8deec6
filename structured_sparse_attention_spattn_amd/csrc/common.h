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

// ------------------------------------------------------------ sequences
// The rows one (sequence, head) owns.  Fixed length (cu == nullptr): B
// sequences of N tokens in a [B, H, N, d] tensor, head h of sequence b at rows
// (b H + h) N + i.  Packed variable length: sequence s holds tokens cu[s] ..
// cu[s+1] - 1 of a [H, T, d] tensor (T tokens in all), head h of it at rows
// h T + cu[s] + i; N is then the longest sequence and only sizes the grid.
// The band is the caller's table (clipped to a packed sequence's length) or,
// for packed sequences without one (own_bdp), the Balanced Distance
// Partitioning table of the sequence's own length ("Making Every Head Count",
// Figure 1 caption: widths floor(n/H) or ceil(n/H), the wider ones first).
// Host side: the packed layout of a launch (cu == nullptr: fixed length).
struct Packed {
  const int32_t* cu;
  int T;
  int own_bdp;
};
struct SeqHead {
  size_t row0;  // row of token 0
  int n;        // tokens in the sequence
  int lo, hi;   // the head's band
};
// A packed sequence's view is clamped so that no kernel indexes outside the
// [H, T, d] tensors whatever cu holds: its first token o lies in [0, T], its
// length n in [0, min(N, T - o)] (N = the longest sequence, which sizes the
// grid; tokens of a longer sequence past N are not computed).  Offsets that
// decrease give an empty sequence.
__host__ __device__ __forceinline__ SeqHead seq_head(const int32_t* cu, int T, int own_bdp, int H, int N,
                                                     const Bands& b, int s, int h) {
  SeqHead r;
  if (cu == nullptr) {
    r.row0 = ((size_t)s * H + h) * N;
    r.n = N;
    r.lo = b.lo[h];
    r.hi = b.hi[h];
    return r;
  }
  const int c0 = cu[s], c1 = cu[s + 1];
  const int o = c0 < 0 ? 0 : (c0 > T ? T : c0);
  const int e = c1 < o ? o : (c1 > T ? T : c1);
  r.n = e - o < N ? e - o : N;
  r.row0 = (size_t)h * T + o;
  if (own_bdp) {
    const int base = r.n / H, extra = r.n % H;
    r.lo = h * base + (h < extra ? h : extra);
    r.hi = r.lo + base + (h < extra ? 1 : 0) - 1;
  } else {
    r.lo = b.lo[h] < r.n ? b.lo[h] : r.n;
    r.hi = b.hi[h] < r.n - 1 ? b.hi[h] : r.n - 1;
  }
  return r;
}

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
// Row-major [rows][D] bf16 tiles in LDS are stored without padding; the 16-byte
// chunks of row r are XOR-permuted by swz<D>(r).  The permutation makes four
// access patterns free of bank conflicts on the 64 x 4-byte LDS banks: the
// 16-byte row reads under perm_row, the transposing 8-byte reads of
// kmajor_operand (the LDS serves 32 lanes of those per cycle), and the 1 KB
// contiguous writes of the direct global -> LDS loads.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128)
    return 4 * (r & 3) + ((r >> 2) & 3);
  else
    return ((r >> 2) & 3) ^ (((r >> 1) & 1) << 2);
}
// Element (row r, column col) of a swizzled tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * D + ((((col >> 3) ^ swz<D>(r))) << 3) + (col & 7);
}

// ds_read_b64_tr_b16: within every group of 16 lanes, source lane j names 4
// consecutive bf16 M[j][0..3]; destination lane l receives
// {M[l/4][l%4], M[l/4+4][l%4], M[l/4+8][l%4], M[l/4+12][l%4]}.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(bf16x4, r);
}

// 32x32x16 operand whose k index runs down the rows of a swizzled tile: lane l
// (group g = l/32) receives rows kbase + 8g .. kbase + 8g + 7 of column
// n0 + (l % 32), i.e. the k-slots 8g .. 8g+7 of MFMA row/column l % 32.
template <int D>
__device__ __forceinline__ bf16x8 kmajor_operand(const bf16* tile, int kbase, int n0, int lane) {
  const int grp = lane >> 4, j = lane & 15, g = lane >> 5;
  const int r = kbase + 8 * g + (j >> 2);
  const int col = n0 + 16 * (grp & 1) + 4 * (j & 3);
  const bf16x4 a = lds_read_tr4(tile + tile_off<D>(r, col));
  const bf16x4 b = lds_read_tr4(tile + tile_off<D>(r + 4, col));
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Per-lane byte offsets inside a swizzled [rows][D] tile for the two operand
// reads of the 32x32x16 products: 16-byte row reads under perm_row (the row
// operand) and the transposing reads of kmajor_operand (the k-major operand).
// Rows r and r + 32 (r + 16 for the transposing reads) share a swizzle, so
// one offset per column block serves every 32-row half; tile and stage bases
// are added on top.
template <int D>
struct LaneOffsets {
  int k[D / 16];      // row reads: row perm_row(l % 32), columns 16 kk + 8 g
  int v[D / 32][2];   // transposing reads: k rows 8 g + (l % 16) / 4 (+ 4), column block dt
  __device__ __forceinline__ LaneOffsets(int lane) {
    const int g = lane >> 5, grp = lane >> 4, j = lane & 15;
    const int krow = perm_row(lane & 31);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) k[kk] = 2 * tile_off<D>(krow, 16 * kk + 8 * g);
    const int r = 8 * g + (j >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int col = 32 * dt + 16 * (grp & 1) + 4 * (j & 3);
      v[dt][0] = 2 * tile_off<D>(r, col);
      v[dt][1] = 2 * tile_off<D>(r + 4, col);
    }
  }
  // Called at the top of every tile: makes the offsets opaque there, so the
  // compiler folds each stage / half constant into the LDS instruction's
  // immediate instead of keeping one hoisted register per combination.
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(k[kk]));
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) asm volatile("" : "+v"(v[dt][0]), "+v"(v[dt][1]));
  }
};

// Row operands (A of S^T = K Q^T): rows row0 + perm_row(l % 32), k-steps 0 .. D/16 - 1.
template <int D>
__device__ __forceinline__ void load_ka(bf16x8* ka, const bf16* ks, const LaneOffsets<D>& off, int row0) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    ka[kk] = *(const bf16x8*)((const char*)ks + off.k[kk] + row0 * D * 2);
}
// k-major operands over tile rows row0 .. row0 + 31 (k) for every 32-column
// block dt: va[2 dt] covers k rows row0 .. +15, va[2 dt + 1] rows row0 + 16 .. +31.
template <int D>
__device__ __forceinline__ void load_va(bf16x8* va, const bf16* vs, const LaneOffsets<D>& off, int row0) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const char* t = (const char*)vs + (row0 + 16 * h) * D * 2;
      const bf16x4 a = lds_read_tr4((const bf16*)(t + off.v[dt][0]));
      const bf16x4 b = lds_read_tr4((const bf16*)(t + off.v[dt][1]));
      va[2 * dt + h] = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
}
// 16-byte row read (8 consecutive columns from col, col % 8 == 0).
template <int D>
__device__ __forceinline__ bf16x8 row_chunk(const bf16* tile, int r, int col) {
  return *(const bf16x8*)(tile + tile_off<D>(r, col));
}

// One direct global -> LDS load (global_load_lds_dwordx4 / _dword): every lane
// sends `bytes` bytes from its own global address to lds_base + bytes * lane.
// Issued from inline assembly so that the compiler does not see an LDS write
// in flight: it would otherwise drain every such load before each LDS read.
// Completion is tracked by the vector-memory counter (wait_vmcnt) and is the
// caller's responsibility.  M0 carries the LDS base and is restored.
__device__ __forceinline__ void lds_dma16(uint32_t lds_base, const void* gaddr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(gaddr)
      : "memory");
}
__device__ __forceinline__ void lds_dma4(uint32_t lds_base, const void* gaddr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(gaddr)
      : "memory");
}
// LDS byte address of p, a pointer into a shared array.  The address-space
// cast of a generic pointer carries a null check (two scalar instructions),
// so the kernels take it once per shared array and add stage and piece
// offsets to it as integers.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const char lchar;
  return (uint32_t)(uintptr_t)(lchar*)p;
}

// Direct global -> LDS copy of ROWS rows of a [N][D] bf16 tensor into a
// swizzled tile: every wave instruction moves 1 KB, lane l landing at byte
// 16 l of it.  Rows past N are clamped to row N - 1 (callers mask them).
// Every wave issues kPer loads; when the tile has fewer 1 KB pieces than there
// are waves, the surplus waves repeat a piece (identical bytes to the same
// place), which keeps the per-wave load count uniform.
template <int ROWS, int D, int WAVES>
struct AsyncTile {
  static constexpr int kRpi = 512 / D;  // rows per 1 KB instruction
  static constexpr int kPieces = ROWS / kRpi;
  static constexpr int kPer = (kPieces + WAVES - 1) / WAVES;
  static_assert(kPieces * kRpi == ROWS && (kPieces % WAVES == 0 || kPieces < WAVES), "uneven tile split");
  // tile: the LDS byte address of the tile's first element
  __device__ __forceinline__ static void load(uint32_t tile, const bf16* __restrict__ src, int row0, int N, int wave,
                                              int lane) {
    const int lr = lane / (D / 8), p = lane % (D / 8);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int rb = ((wave + WAVES * i) % kPieces) * kRpi;
      const int r = rb + lr;
      const int grow = min(row0 + r, N - 1);
      const int c = p ^ swz<D>(r);
      lds_dma16(__builtin_amdgcn_readfirstlane(tile + 2 * rb * D), src + (size_t)grow * D + c * 8);
    }
  }
  // The per-lane source offsets of a wave's pieces relative to the tile's
  // first row (element units): fixed for the whole walk, so a tile that lies
  // inside the rows [0, N) costs one address add per piece.
  struct Offsets {
    int e[kPer];
    __device__ __forceinline__ Offsets(int wave, int lane) {
      const int lr = lane / (D / 8), p = lane % (D / 8);
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int r = ((wave + WAVES * i) % kPieces) * kRpi + lr;
        e[i] = r * D + (p ^ swz<D>(r)) * 8;
      }
    }
  };
  __device__ __forceinline__ static void load(uint32_t tile, const bf16* __restrict__ src, int row0, int N,
                                              const Offsets& o, int wave, int lane) {
    if (row0 + ROWS > N) {  // the sequence's last tile: clamped rows
      load(tile, src, row0, N, wave, lane);
      return;
    }
    const bf16* base = src + (size_t)row0 * D;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int rb = ((wave + WAVES * i) % kPieces) * kRpi;
      lds_dma16(__builtin_amdgcn_readfirstlane(tile + 2 * rb * D), base + o.e[i]);
    }
  }
};

// Make the compiler complete the load that produced x here (it inserts the
// vector-memory wait before this empty statement), so no such wait is left
// inside a loop that also has direct LDS loads in flight.
template <typename T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" ::"v"(x));
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Sum over kk of a[kk] x b[kk] (32x32 output, k = 16 per product), the
// products spread over CH independent accumulators that are added at the end.
// On gfx950 one dependent chain issues as fast as several (8 dependent
// 32x32x16 products measured at 258.6 cycles, the same as 4 chains), so the
// kernels use CH = 1 and save the reduction's VALU work and registers.
template <int KK, int CH = 1>
__device__ __forceinline__ f32x16 mfma_ksum(const bf16x8* a, const bf16x8* b) {
  constexpr int kCh = KK < CH ? KK : CH;
  f32x16 part[kCh];
#pragma unroll
  for (int c = 0; c < kCh; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) part[c][i] = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) part[kk % kCh] = mfma32(a[kk], b[kk], part[kk % kCh]);
#pragma unroll
  for (int c = 1; c < kCh; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) part[0][i] += part[c][i];
  return part[0];
}

// Scheduling pattern for the current region: NM times {one MFMA, up to NT
// transcendental and up to NV other vector-ALU instructions}, so independent
// VALU work issues while each MFMA runs instead of after the last one.
template <int NM, int NT, int NV>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x400, NT, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
}
// Keep the computation of x inside the current region (an empty asm that
// reads it; no instruction is emitted).
template <typename T>
__device__ __forceinline__ void keep_here(const T& x) {
  asm volatile("" ::"v"(x));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Combine the values of lanes l and l ^ 32 (the two 16-row halves of one
// 32x32 accumulator column) without going through LDS: v_permlane32_swap
// exchanges lanes 32..63 of one register with lanes 0..31 of another, so on
// two copies of x it leaves each lane holding its own value in one of them
// and its partner's in the other.  Issued from inline assembly: the compiler's
// intrinsic has been seen to substitute the first result for the second,
// losing the partner's value.  The s_nop covers the wait states a permlane
// swap needs after a VALU write of its operands.
__device__ __forceinline__ void pair_exchange(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_exchange(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_exchange(x, a, b);
  return a + b;
}

// Band mask of one 32x32 score accumulator under perm_row: register i of a
// lane in group g holds key row kb + perm_reg_row(i, g) against query iq;
// the pair is kept when lo <= iq - key <= hi.  base = iq - kb - 8 g - lo,
// width = hi - lo; one unsigned compare per score.
__device__ __forceinline__ void band_mask(float* x, int base, int width) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = ((i >> 3) << 4) + (i & 7);
    x[i] = (uint32_t)(base - c) <= (uint32_t)width ? x[i] : -__builtin_inff();
  }
}
// Same with a second distance range: base2 = iq - kb - 8 g - lo2, width2 = hi2 - lo2.
__device__ __forceinline__ void band_mask2(float* x, int base, int width, int base2, int width2) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = ((i >> 3) << 4) + (i & 7);
    const bool in = (uint32_t)(base - c) <= (uint32_t)width || (uint32_t)(base2 - c) <= (uint32_t)width2;
    x[i] = in ? x[i] : -__builtin_inff();
  }
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)x[j];
  return r;
}

// -------------------------------------------------------------- epilogue
// A wave's 32 x D float32 result tile is staged in LDS and written out as
// whole rows: the MFMA accumulator layout would otherwise send 2- to 8-byte
// pieces of 32 different rows per store instruction.  Staging layout: D floats
// per row, the 16-byte chunks of row r XOR-permuted by r & 15, which keeps
// the accumulator-layout writes and the row reads free of bank conflicts.
template <int D>
__device__ __forceinline__ int stage_off(int r, int col) {
  return r * D + (((col >> 2) ^ (r & 15)) << 2) + (col & 3);
}
// Accumulators of a transposed product X^T (column l % 32 = row of X,
// register i of block dt = column 32 dt + 8 (i / 4) + 4 g + i % 4 of X),
// times `mul`, into the staging tile.  A staging tile may hold only the NC
// columns C0 .. C0 + NC - 1 of X (a 32 x NC tile), so that a kernel whose
// LDS is smaller than 32 x D floats per wave writes its result in D / NC
// passes.
template <int D, int NC = D, int C0 = 0>
__device__ __forceinline__ void stage_transposed(float* st, const f32x16* acc, float mul, int lane) {
  static_assert(NC % 32 == 0 && C0 % 32 == 0 && C0 + NC <= D, "staged column range");
  const int g = lane >> 5, r = lane & 31;
#pragma unroll
  for (int dt = 0; dt < NC / 32; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x16& x = acc[C0 / 32 + dt];
      *(f32x4*)&st[stage_off<NC>(r, 32 * dt + 8 * a + 4 * g)] =
          f32x4{x[4 * a] * mul, x[4 * a + 1] * mul, x[4 * a + 2] * mul, x[4 * a + 3] * mul};
    }
}
// Rows 0 .. nrows - 1 of a 32 x NC staging tile to columns col0 .. col0 +
// NC - 1 of dst + row0 * D (row-major, bfloat16 or float32): every lane
// moves 8 consecutive values of one row, so one store instruction covers
// 512 / NC whole rows.
template <int D, int NC = D>
__device__ __forceinline__ void store_staged(const float* st, void* dst, size_t row0, int nrows, bool f32, int lane,
                                             int col0 = 0) {
  constexpr int kLpr = NC / 8;     // lanes per row
  constexpr int kRpp = 64 / kLpr;  // rows per pass
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's staging writes have landed
#pragma unroll
  for (int pass = 0; pass < 32 / kRpp; ++pass) {
    const int r = pass * kRpp + lane / kLpr;
    const int c = 8 * (lane % kLpr);
    const f32x4 a = *(const f32x4*)&st[stage_off<NC>(r, c)];
    const f32x4 b = *(const f32x4*)&st[stage_off<NC>(r, c + 4)];
    if (r < nrows) {
      const size_t idx = (row0 + r) * D + col0 + c;
      if (f32) {
        *(f32x4*)((float*)dst + idx) = a;
        *(f32x4*)((float*)dst + idx + 4) = b;
      } else {
        *(bf16x8*)((bf16*)dst + idx) = bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                                             (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
      }
    }
  }
}

// A wave's 32 x D transposed result (accumulators times `mul`) to rows
// row0 .. row0 + nrows - 1 of dst, through a staging area of 32 x NC floats
// in one pass (NC = D) or two column passes (NC = D / 2; one wave's LDS
// operations complete in order, so the second pass's writes follow the first
// pass's reads).
template <int D, int NC>
__device__ __forceinline__ void store_result(float* stg, const f32x16* acc, float mul, void* dst, size_t row0,
                                             int nrows, bool f32, int lane) {
  static_assert(NC == D || 2 * NC == D, "one or two column passes");
  stage_transposed<D, NC, 0>(stg, acc, mul, lane);
  store_staged<D, NC>(stg, dst, row0, nrows, f32, lane, 0);
  if constexpr (NC < D) {
    stage_transposed<D, NC, NC>(stg, acc, mul, lane);
    store_staged<D, NC>(stg, dst, row0, nrows, f32, lane, NC);
  }
}

// Zero rows 0 .. nrows - 1 of dst + row0 * D, in the store pattern of
// store_staged (no staging needed for a tile that received no products).
template <int D>
__device__ __forceinline__ void store_zero_rows(void* dst, size_t row0, int nrows, bool f32, int lane) {
  constexpr int kLpr = D / 8;
  constexpr int kRpp = 64 / kLpr;
#pragma unroll
  for (int pass = 0; pass < 32 / kRpp; ++pass) {
    const int r = pass * kRpp + lane / kLpr;
    const int c = 8 * (lane % kLpr);
    if (r < nrows) {
      const size_t idx = (row0 + r) * D + c;
      if (f32) {
        *(f32x4*)((float*)dst + idx) = f32x4{0.f, 0.f, 0.f, 0.f};
        *(f32x4*)((float*)dst + idx + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        *(u32x4*)((bf16*)dst + idx) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
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

// Distance set of one head with the shared local window of "Making Every
// Head Count" (Figure 2 caption: the exclusive-band ablation is the method
// with local sharing removed): the band [lo, hi] joined with [0, w - 1].
// The union is kept as a primary range plus, when the window stays below the
// band with a gap, a second disjoint range [nlo, nhi]; otherwise the second
// range is empty, encoded as a single impossible distance so that the
// unsigned range test "(dist - nlo) <= nhi - nlo" never passes.
struct DistSet {
  int lo, hi;
  int nlo, nhi;
};
constexpr int kNoDistance = -(1 << 30);
__host__ __device__ __forceinline__ DistSet dist_set(int lo, int hi, int w) {
  DistSet s{lo, hi, kNoDistance, kNoDistance};
  if (w > 0) {
    const int wh = w - 1;
    if (hi < lo) {
      s.lo = 0;
      s.hi = wh;
    } else if (wh >= lo - 1) {
      s.lo = 0;
      s.hi = hi > wh ? hi : wh;
    } else {
      s.nlo = 0;
      s.nhi = wh;
    }
  }
  return s;
}
__host__ __device__ __forceinline__ bool has_second(const DistSet& s) { return s.nhi != kNoDistance; }

// Tiles to visit: up to two ascending runs of tile indices, the second
// starting past the first (runs that overlap or touch are merged).  Virtual
// index v in [0, n) maps to tile at(v).
struct TileWalk {
  int a0, na, b0, n;
  int rot;  // a single run starts at tile a0 + rot and wraps around (align_walk)
  __host__ __device__ __forceinline__ int at(int v) const {
    if (v < na) {
      const int t = v + rot;
      return a0 + (t < na ? t : t - na);
    }
    return b0 + (v - na);
  }
};
__host__ __device__ __forceinline__ TileWalk tile_walk(KeySpan s1, KeySpan s2, int tile) {
  const bool e1 = s1.last < s1.first, e2 = s2.last < s2.first;
  TileWalk w{0, 0, 0, 0, 0};
  if (e1 && e2) return w;
  if (e1 || e2) {
    const KeySpan s = e1 ? s2 : s1;
    w.a0 = s.first / tile;
    w.na = w.n = s.last / tile - w.a0 + 1;
    return w;
  }
  int a0 = s1.first / tile, a1 = s1.last / tile, b0 = s2.first / tile, b1 = s2.last / tile;
  if (b0 < a0) {
    int t = a0; a0 = b0; b0 = t;
    t = a1; a1 = b1; b1 = t;
  }
  if (b0 <= a1 + 1) {
    w.a0 = a0;
    w.na = w.n = (a1 > b1 ? a1 : b1) - a0 + 1;
  } else {
    w.a0 = a0;
    w.na = a1 - a0 + 1;
    w.b0 = b0;
    w.n = w.na + b1 - b0 + 1;
  }
  return w;
}
__host__ __device__ __forceinline__ int floor_div(int x, int t) { return x >= 0 ? x / t : -((-x + t - 1) / t); }

// Visit order shared by neighbouring workgroups.  Consecutive tiles of one
// head need overlapping runs of the other operand (with the band's lag), and
// an ascending walk makes each workgroup read a shared tile several steps
// before or after its neighbour, long enough for the tile to leave L2 in
// between.  Instead a single run starts at the tile whose index is 0 modulo
// m, the length of an unclipped run (rows [r0, r1] before clipping to the
// sequence), and wraps around: every workgroup with a full run then visits
// tile x at step x mod m, so workgroups that share x read it at the same step.
// The order of tiles does not change what is summed.
__host__ __device__ __forceinline__ void align_walk(TileWalk& w, int r0, int r1, int tile) {
  if (w.n < 2 || w.na != w.n) return;
  const int m = floor_div(r1, tile) - floor_div(r0, tile) + 1;
  if (m < 2) return;
  const int k = (m - w.a0 % m) % m;
  w.rot = k < w.n ? k : 0;
}

// The tiles one workgroup visits.  A query-major kernel (forward, dQ) owns
// query rows [r0, r0 + own - 1] of a sequence of n rows and visits key tiles of
// `tile` rows; a key-major kernel (dK / dV) owns key rows and visits query
// tiles.  The visited tiles are those meeting the head's distance set, as at
// most two ascending runs; `aligned` rotates a single run (align_walk).
struct WalkShape {
  int own, tile;
  bool key_major, aligned;
};
__host__ __device__ __forceinline__ TileWalk kernel_walk(const WalkShape& ws, int r0, int n, const DistSet& s) {
  const int r1 = (r0 + ws.own - 1 < n - 1) ? r0 + ws.own - 1 : n - 1;
  KeySpan s1, s2{0, -1};
  if (ws.key_major) {
    s1 = band_query_span(r0, r1, s.lo, s.hi, n);
    if (has_second(s)) s2 = band_query_span(r0, r1, s.nlo, s.nhi, n);
  } else {
    s1 = band_key_span(r0, r1, s.lo, s.hi);
    if (has_second(s)) s2 = band_key_span(r0, r1, s.nlo, s.nhi);
  }
  TileWalk w = tile_walk(s1, s2, ws.tile);
  if (ws.aligned) {
    if (ws.key_major)
      align_walk(w, r0 + s.lo, r0 + ws.own - 1 + s.hi, ws.tile);
    else
      align_walk(w, r0 - s.hi, r0 + ws.own - 1 - s.lo, ws.tile);
  }
  return w;
}

// Smallest distance of the set, or n (no distance in [0, n - 1]) when the set
// is empty.  Key j has a query iff j <= n - 1 - min_dist; query i has a key
// iff i >= min_dist.  So the tiles without work are a suffix of the key tiles
// and a prefix of the query tiles.
__host__ __device__ __forceinline__ int min_dist(const DistSet& s, int n) {
  if (has_second(s)) return s.nlo < s.lo ? s.nlo : s.lo;
  return s.hi >= s.lo && s.lo <= n - 1 ? s.lo : n;
}

// Tile tests over the whole distance set (an empty second range never meets
// and is never full).
__host__ __device__ __forceinline__ bool set_meets(int i_min, int i_max, int j_min, int j_max, const DistSet& s) {
  return tile_meets(i_min, i_max, j_min, j_max, s.lo, s.hi) ||
         (has_second(s) && tile_meets(i_min, i_max, j_min, j_max, s.nlo, s.nhi));
}
__host__ __device__ __forceinline__ bool set_full(int i_min, int i_max, int j_min, int j_max, const DistSet& s) {
  return tile_full(i_min, i_max, j_min, j_max, s.lo, s.hi) ||
         (has_second(s) && tile_full(i_min, i_max, j_min, j_max, s.nlo, s.nhi));
}

// Workgroup -> logical work item, so that consecutive logical items land on
// the same XCD (the hardware deals workgroups to the 8 XCDs round-robin).
__host__ __device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int xcd = pid % kXcd, slot = pid / kXcd;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Work item of a launch over (sequence b, head h, row tile t).  With distance
// bands ordered nearest first, a head's rows before its band start have no
// keys, so the work of a (b, h) pair falls with h.  The pairs are ranked
// heaviest first (h ascending, then b) and dealt to the 8 XCDs in
// boustrophedon rounds: XCD x takes ranks x, 15 - x, 16 + x, 31 - x, ...,
// each pair with all its tiles, as one contiguous run of that XCD's
// workgroups (xcd_remap).  Every XCD then holds the same number of pairs, a
// mix of heavy and light heads, in heavy-first order.  The pair count is
// rounded up to a multiple of 8 (work_grid); items of the padding pairs have
// valid == false.
struct WorkItem {
  int b, h, t;
  bool valid;
};
__host__ __device__ __forceinline__ long long work_grid(int B, int H, int n_tiles) {
  return 8LL * ((B * H + 7) / 8) * n_tiles;
}
// descending: the tiles of a pair are dispatched from the last to the first.
// Query-major kernels ask for it: a head's first query tiles have no keys
// and the next few only part of its distance set, so in descending order the
// full-cost tiles start first and the cheap ones last, and the workgroups that
// wait for a slot are cheap ones.  (Key-major kernels already have that order
// ascending: their last key tiles have fewer queries or none.)
__host__ __device__ __forceinline__ WorkItem work_item(int pid, int B, int H, int n_tiles,
                                                     bool descending = false) {
  const int c = (B * H + 7) / 8;  // pairs per XCD
  const int item = xcd_remap(pid, 8 * c * n_tiles);
  const int m = item / n_tiles;
  const int x = m / c, li = m % c;
  const int k = 8 * li + ((li & 1) ? 7 - x : x);
  WorkItem w;
  w.b = k % B;
  w.h = k / B;
  w.t = item % n_tiles;
  if (descending) w.t = n_tiles - 1 - w.t;
  w.valid = k < B * H;
  return w;
}

}  // namespace spattn
