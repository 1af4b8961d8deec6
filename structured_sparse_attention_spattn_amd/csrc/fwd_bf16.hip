// Band-partitioned attention forward, bfloat16 storage / float32 accumulate,
// gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Computes, per head h with band [lo_h, hi_h] ("Making Every Head Count",
// Figure 1 caption: Balanced Distance Partitioning), the masked-set softmax
// attention of "Sparse Attention, Then and Now" section 1 over the keys
// j with lo_h <= i - j <= hi_h, plus the natural-log LSE of each row.
//
// Work decomposition
//   one workgroup = (batch b, head h, query tile of BQ = 128 rows), 4 waves,
//   each wave owns 32 query rows; two workgroups share a CU.  K and V tiles
//   stream into a double-buffered LDS ring with direct global -> LDS loads
//   (no register staging); tile u + 1 is in flight while tile u is used.  The workgroup
//   visits only the key tiles (BK = 64 rows) that intersect the diagonal strip
//   [i - hi_h, i - lo_h] of its rows; inside a tile each wave skips the 32-key
//   halves that miss its own 32-row strip, and masks element-wise only where
//   a half is PARTIAL (a wave-uniform branch).  Workgroups are remapped so
//   consecutive query tiles of one (b, h) run on the same XCD and share the
//   K/V strip through that XCD's L2.
// Products (transposed so no register shuffles are needed between them)
//   S^T (keys x queries) = K Q^T    A = K rows from LDS, B = Q in registers
//   O^T (d x queries)   += V^T P^T  A = V^T read from the row-major V tile
//                                    with the LDS transpose read,
//                                    B = P^T straight from the S^T registers
//   Each lane then owns one query column: the row maximum needs one
//   cross-lane exchange (lanes l and l+32), the row sum none until the end.
//   The score scale is folded into the exponent (one FMA per score).
#include "common.h"

namespace spattn {
namespace {

constexpr int kBQ = 128;
constexpr int kBK = 64;
constexpr int kThreads = 256;

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int B, H, N;
  int n_qt;
  float scale_log2;
  Bands bands;
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs p) {
  constexpr int kTile = kBK * D;  // one K or V tile, bf16 elements
  using Tile = AsyncTile<kBK, D, kThreads / 64>;
  constexpr int kDT = D / 32;      // 32-row output blocks of O^T
  constexpr int kKK = D / 16;      // k-steps of the score product
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const int total = p.B * p.H * p.n_qt;
  const int item = xcd_remap(blockIdx.x, total);
  const int t = item % p.n_qt;
  const int bh = item / p.n_qt;
  const int h = bh % p.H;
  const int N = p.N;
  const int lo = p.bands.lo[h];
  const int hi = p.bands.hi[h];
  const size_t base = (size_t)bh * N * D;
  const bf16* __restrict__ qb = p.q + base;
  const bf16* __restrict__ kb = p.k + base;
  const bf16* __restrict__ vb = p.v + base;
  bf16* __restrict__ ob = p.o + base;
  float* __restrict__ lb = p.lse + (size_t)bh * N;
  const float ninf = -__builtin_inff();

  const int i_tile0 = t * kBQ;
  const int i_tile1 = min(N - 1, i_tile0 + kBQ - 1);
  const KeySpan span = band_key_span(i_tile0, i_tile1, lo, hi);
  if (span.last < span.first) {
    // No row of this tile has a key: output 0, LSE -inf.
    constexpr int kCpr = D / 8;
    for (int c = tid; c < kBQ * kCpr; c += kThreads) {
      const int i = i_tile0 + c / kCpr;
      if (i < N) *(u32x4*)(ob + (size_t)i * D + (c % kCpr) * 8) = u32x4{0, 0, 0, 0};
    }
    for (int r = tid; r < kBQ; r += kThreads)
      if (i_tile0 + r < N) lb[i_tile0 + r] = ninf;
    return;
  }
  const int u_begin = span.first / kBK;
  const int u_end = span.last / kBK + 1;

  const int iw0 = i_tile0 + 32 * wave;
  const int iw1 = min(N - 1, iw0 + 31);
  const bool wave_live = iw0 <= N - 1;
  const int iq = iw0 + c32;

  // Q^T operand: lane holds Q[iq][16kk + 8g .. +7].
  bf16x8 qreg[kKK];
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk)
    qreg[kk] = iq < N ? *(const bf16x8*)(qb + (size_t)iq * D + 16 * kk + 8 * g) : bf16x8{};
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) settle(qreg[kk]);

  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m_run = ninf;  // running row maximum of the raw (unscaled) scores
  float l_run = 0.f;   // this lane's share of the row sum
  const float sl2 = p.scale_log2;

  Tile::load(smem, kb, u_begin * kBK, N, wave, lane);
  Tile::load(smem + kTile, vb, u_begin * kBK, N, wave, lane);

  for (int u = u_begin; u < u_end; ++u) {
    const int s = (u - u_begin) & 1;
    wait_vmcnt<0>();  // this wave's part of tile u has landed
    __syncthreads();  // ... everyone's, and everyone is done with tile u - 1
    if (u + 1 < u_end) {
      bf16* nxt = smem + (s ^ 1) * 2 * kTile;
      Tile::load(nxt, kb, (u + 1) * kBK, N, wave, lane);
      Tile::load(nxt + kTile, vb, (u + 1) * kBK, N, wave, lane);
    }
    const bf16* ks = smem + s * 2 * kTile;
    const bf16* vs = ks + kTile;

    // Scores of both 32-key halves.  Operands are read in batches ahead of
    // their products (sched_barrier keeps the compiler from interleaving each
    // read with its MFMA, which would expose the LDS latency every time).
    float x[2][16];
    bool act[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int jb = u * kBK + 32 * m;
      act[m] = wave_live && tile_meets(iw0, iw1, jb, jb + 31, lo, hi);
      if (act[m]) {
        const int krow = 32 * m + perm_row(c32);
        bf16x8 ka[kKK];
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) ka[kk] = row_chunk<D>(ks, krow, 16 * kk + 8 * g);
        __builtin_amdgcn_sched_barrier(0);
        const f32x16 sacc = mfma_ksum<kKK>(ka, qreg);
        if (tile_full(iw0, iw1, jb, jb + 31, lo, hi)) {
#pragma unroll
          for (int i = 0; i < 16; ++i) x[m][i] = sacc[i];
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int dist = iq - (jb + perm_reg_row(i, g));
            x[m][i] = (dist >= lo && dist <= hi) ? sacc[i] : ninf;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[m][i] = ninf;
      }
    }

    if (act[0] || act[1]) {
      // V^T operands of the first active half: in flight during the softmax.
      const int m0 = act[0] ? 0 : 1;
      bf16x8 va[2 * kDT];
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        va[2 * dt] = kmajor_operand<D>(vs, 32 * m0, 32 * dt, lane);
        va[2 * dt + 1] = kmajor_operand<D>(vs, 32 * m0 + 16, 32 * dt, lane);
      }
      float mx = ninf;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[m][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == ninf ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * sl2);
      const float nms = -m_use * sl2;
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          x[m][i] = fast_exp2(__builtin_fmaf(x[m][i], sl2, nms));
          psum += x[m][i];
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;

      {
        const bf16x8 pb0 = pack8(&x[m0][0]);
        const bf16x8 pb1 = pack8(&x[m0][8]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          acc[dt] = mfma32(va[2 * dt], pb0, acc[dt]);
          acc[dt] = mfma32(va[2 * dt + 1], pb1, acc[dt]);
        }
      }
      if (m0 == 0 && act[1]) {
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          va[2 * dt] = kmajor_operand<D>(vs, 32, 32 * dt, lane);
          va[2 * dt + 1] = kmajor_operand<D>(vs, 48, 32 * dt, lane);
        }
        const bf16x8 pb0 = pack8(&x[1][0]);
        const bf16x8 pb1 = pack8(&x[1][8]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          acc[dt] = mfma32(va[2 * dt], pb0, acc[dt]);
          acc[dt] = mfma32(va[2 * dt + 1], pb1, acc[dt]);
        }
      }
    }
  }

  // ---- epilogue: O = acc / l, LSE = scale * m + ln(sum)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (iq < N) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 w;
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] = (bf16)(acc[dt][4 * a + c] * inv);
        *(bf16x4*)(ob + (size_t)iq * D + 32 * dt + 8 * a + 4 * g) = w;
      }
    if (g == 0) lb[iq] = l_tot > 0.f ? (m_run * sl2 + fast_log2(l_tot)) * kLn2 : ninf;
  }
}

}  // namespace

int launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int N, int d, const Bands& bands, float scale, hipStream_t stream) {
  FwdArgs a;
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.o = (bf16*)o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  a.n_qt = (N + kBQ - 1) / kBQ;
  a.scale_log2 = scale * kLog2e;
  a.bands = bands;
  const long long total = (long long)B * H * a.n_qt;
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  dim3 grid((unsigned)total), block(kThreads);
  if (d == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, block, 0, stream, a);
  else if (d == 64)
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, block, 0, stream, a);
  else
    return SPATTN_E_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

void fwd_bf16_tiles(int* BQ, int* BK) {
  *BQ = kBQ;
  *BK = kBK;
}

}  // namespace spattn
