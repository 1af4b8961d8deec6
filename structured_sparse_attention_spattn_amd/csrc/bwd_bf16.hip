// Backward of band-partitioned attention, bfloat16 storage / float32
// accumulate, gfx950 MFMA (v_mfma_f32_32x32x16_bf16).  The derivative is the
// textbook one of the masked-set softmax ("Sparse Attention, Then and Now",
// section 1) over each head's distance band ("Making Every Head Count",
// Figure 1 caption); the pages give no backward pass:
//     D_i = dO_i . O_i,  P = exp(scale q_i.k_j - LSE_i) on the band,
//     dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
//
// Two deterministic kernels, no atomics:
//   bwd_dq    query-major, one workgroup per (b, h, 128 query rows), 4 waves
//             of 32 rows.  Computes D for its rows (written for the second
//             kernel), then walks the 32-key tiles of its band strip:
//             S^T = K Q^T, dP^T = V dO^T, dS^T, and dQ^T += K^T dS^T (K^T is
//             read from the row-major K tile with the LDS transpose read).
//   bwd_dkdv  key-major, one workgroup per (b, h, 64 key rows), 4 waves in
//             2 pairs of 32 keys.  Walks the 32-row query blocks that reach its
//             keys: S = Q K^T and dV += P^T dO in one wave of a pair, dP = dO V^T,
//             dS and dK += dS^T Q in the other, dK / dV held in registers for
//             the whole walk (dO and Q enter the last two products through the
//             LDS transpose read).
// Both recompute P from the saved LSE with the same band-tile enumeration as
// the forward pass and mask element-wise only on tiles that are not FULL.
#include "common.h"

namespace spattn {
namespace {

constexpr int kThreads = 256;

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  float* dvec;  // written by bwd_dq, read by bwd_dkdv
  void* dq;
  void* dk;
  void* dv;
  int grad_f32;
  int B, H, N;
  int n_tiles;  // query tiles (bwd_dq) or key tiles (bwd_dkdv) per (b, h)
  float scale;
  float scale_log2;
  Bands bands;
};

// Store 4 consecutive float values as bf16 or f32.
__device__ __forceinline__ void store4(void* base, size_t idx, const float* x, bool f32) {
  if (f32) {
    *(f32x4*)((float*)base + idx) = f32x4{x[0], x[1], x[2], x[3]};
  } else {
    bf16x4 w;
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = (bf16)x[c];
    *(bf16x4*)((bf16*)base + idx) = w;
  }
}

// =====================================================================  dQ
constexpr int kDqBQ = 128;    // query rows per workgroup
constexpr int kDqBK = 32;     // key rows per stage
constexpr int kDqStages = 4;  // LDS ring depth: tiles u+1 .. u+3 load while u is used

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs p) {
  constexpr int kTile = kDqBK * D;
  constexpr int kKK = D / 16;
  constexpr int kDT = D / 32;
  using Tile = AsyncTile<kDqBK, D, kThreads / 64>;
  constexpr int kL = 2 * Tile::kPer;  // loads per wave per stage
  __shared__ __attribute__((aligned(16))) bf16 smem[kDqStages * 2 * kTile];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const int total = p.B * p.H * p.n_tiles;
  const int item = xcd_remap(blockIdx.x, total);
  const int t = item % p.n_tiles;
  const int bh = item / p.n_tiles;
  const int h = bh % p.H;
  const int N = p.N;
  const int lo = p.bands.lo[h];
  const int hi = p.bands.hi[h];
  const size_t base = (size_t)bh * N * D;
  const bf16* __restrict__ kb = p.k + base;
  const bf16* __restrict__ vb = p.v + base;

  const int i_tile0 = t * kDqBQ;
  const int iw0 = i_tile0 + 32 * wave;
  const int iw1 = min(N - 1, iw0 + 31);
  const bool wave_live = iw0 <= N - 1;
  const int iq = iw0 + c32;
  const bool row_ok = iq < N;

  // Q and dO operands; D_i = dO_i . O_i from the same lanes.
  bf16x8 qreg[kKK], doreg[kKK];
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    const size_t off = base + (size_t)iq * D + 16 * kk + 8 * g;
    if (row_ok) {
      qreg[kk] = *(const bf16x8*)(p.q + off);
      doreg[kk] = *(const bf16x8*)(p.dout + off);
      const bf16x8 ov = *(const bf16x8*)(p.o + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart += (float)doreg[kk][e] * (float)ov[e];
    } else {
      qreg[kk] = bf16x8{};
      doreg[kk] = bf16x8{};
    }
  }
  const float dval = dpart + __shfl_xor(dpart, 32);
  if (row_ok && g == 0) p.dvec[(size_t)bh * N + iq] = dval;
  const float sl2 = p.scale_log2;
  const float scl = p.scale;
  // exponent offset: P = exp2(s * sl2 - lse2), lse2 = LSE * log2(e)
  const float nlse2 = row_ok ? -p.lse[(size_t)bh * N + iq] * kLog2e : 0.f;
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    settle(qreg[kk]);
    settle(doreg[kk]);
  }
  settle(nlse2);
  settle(dval);

  const int i_tile1 = min(N - 1, i_tile0 + kDqBQ - 1);
  const KeySpan span = band_key_span(i_tile0, i_tile1, lo, hi);

  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  if (span.last >= span.first) {
    const int u_begin = span.first / kDqBK;
    const int u_end = span.last / kDqBK + 1;
    auto issue = [&](int u) {
      bf16* st = smem + ((u - u_begin) % kDqStages) * 2 * kTile;
      Tile::load(st, kb, u * kDqBK, N, wave, lane);
      Tile::load(st + kTile, vb, u * kDqBK, N, wave, lane);
    };
#pragma unroll
    for (int i = 0; i < kDqStages - 1; ++i)
      if (u_begin + i < u_end) issue(u_begin + i);
    for (int u = u_begin; u < u_end; ++u) {
      const int ahead = u_end - 1 - u;  // tiles issued after u and possibly in flight
      if (ahead >= 2)
        wait_vmcnt<2 * kL>();
      else if (ahead == 1)
        wait_vmcnt<kL>();
      else
        wait_vmcnt<0>();
      __syncthreads();  // tile u complete for everyone; tile u - 1 released
      if (u + kDqStages - 1 < u_end) issue(u + kDqStages - 1);
      const bf16* ks = smem + ((u - u_begin) % kDqStages) * 2 * kTile;
      const bf16* vs = ks + kTile;
      const int jb = u * kDqBK;
      if (wave_live && tile_meets(iw0, iw1, jb, jb + 31, lo, hi)) {
        const int prow = perm_row(c32);
        // S^T and dP^T as four independent MFMA chains (even / odd k-steps),
        // operands read two k-steps at a time ahead of their products.
        f32x16 s0, s1, p0, p1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s0[i] = 0.f;
          s1[i] = 0.f;
          p0[i] = 0.f;
          p1[i] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < kKK; kk += 2) {
          const bf16x8 ka0 = row_chunk<D>(ks, prow, 16 * kk + 8 * g);
          const bf16x8 ka1 = row_chunk<D>(ks, prow, 16 * kk + 16 + 8 * g);
          const bf16x8 va0 = row_chunk<D>(vs, prow, 16 * kk + 8 * g);
          const bf16x8 va1 = row_chunk<D>(vs, prow, 16 * kk + 16 + 8 * g);
          __builtin_amdgcn_sched_barrier(0);
          s0 = mfma32(ka0, qreg[kk], s0);
          p0 = mfma32(va0, doreg[kk], p0);
          s1 = mfma32(ka1, qreg[kk + 1], s1);
          p1 = mfma32(va1, doreg[kk + 1], p1);
        }
        f32x16 sacc, pacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[i] = s0[i] + s1[i];
          pacc[i] = p0[i] + p1[i];
        }
        // K^T operands of dQ^T += K^T dS^T, in flight during the dS math
        bf16x8 kt[2 * kDT];
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          kt[2 * dt] = kmajor_operand<D>(ks, 0, 32 * dt, lane);
          kt[2 * dt + 1] = kmajor_operand<D>(ks, 16, 32 * dt, lane);
        }
        float ds[16];
        if (tile_full(iw0, iw1, jb, jb + 31, lo, hi)) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            ds[i] = fast_exp2(__builtin_fmaf(sacc[i], sl2, nlse2)) * (pacc[i] - dval) * scl;
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int dist = iq - (jb + perm_reg_row(i, g));
            const bool ok = row_ok && dist >= lo && dist <= hi;
            const float pe = fast_exp2(__builtin_fmaf(sacc[i], sl2, nlse2));
            ds[i] = ok ? pe * (pacc[i] - dval) * scl : 0.f;
          }
        }
        const bf16x8 d0 = pack8(&ds[0]), d1 = pack8(&ds[8]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          acc[dt] = mfma32(kt[2 * dt], d0, acc[dt]);
          acc[dt] = mfma32(kt[2 * dt + 1], d1, acc[dt]);
        }
      }
    }
  }

  if (row_ok) {
    const bool f32 = p.grad_f32 != 0;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float x4[4] = {acc[dt][4 * a], acc[dt][4 * a + 1], acc[dt][4 * a + 2], acc[dt][4 * a + 3]};
        store4(p.dq, base + (size_t)iq * D + 32 * dt + 8 * a + 4 * g, x4, f32);
      }
  }
}

// =====================================================================  dK dV
// Warp-specialised: 4 waves, 64 keys, two workgroups per CU.  Wave w < 2
// ("P wave") owns keys 32w .. 32w+31 of the tile: S = Q K^T, P, and
// dV += P^T dO.  Wave w + 2 ("dS wave") owns the same keys: dP = dO V^T, then
// -- with P handed over through LDS -- dS = P (dP - D) and dK += dS^T Q.  Each
// wave keeps a single 32 x d accumulator; the two workgroups on a CU run
// their barrier-separated phases independently, so one's LDS reads overlap
// the other's matrix products.
constexpr int kKvBK = 64;     // key rows per workgroup
constexpr int kKvQB = 32;     // query rows per stage
constexpr int kKvStages = 4;  // LDS ring depth: blocks tq+1 .. tq+3 load while tq is used
constexpr int kKvThreads = 256;
constexpr int kKvPairs = kKvThreads / 128;

template <int D>
__global__ __launch_bounds__(kKvThreads, 2) void bwd_dkdv_kernel(BwdArgs p) {
  constexpr int kWaves = kKvThreads / 64;
  constexpr int kTile = kKvQB * D;
  constexpr int kKK = D / 16;
  constexpr int kDT = D / 32;
  using Tile = AsyncTile<kKvQB, D, kWaves>;
  constexpr int kL = 2 * Tile::kPer + 1;  // loads per wave per stage (Q, dO, LSE|D)
  __shared__ __attribute__((aligned(16))) bf16 smem[kKvStages * 2 * kTile];  // [stage][Q, dO]
  // [stage][wave][LSE of the 32 rows | D of the 32 rows]: every wave loads its own copy
  __shared__ __attribute__((aligned(16))) float rowv[kKvStages][kWaves][2 * kKvQB];
  // P handed from P wave w to dS wave w + kKvPairs: [w][lane][16 floats]
  __shared__ __attribute__((aligned(16))) float pbuf[kKvPairs][64][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pwave = wave < kKvPairs;
  const int kw = wave % kKvPairs;  // key group shared by the P / dS wave pair
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const int total = p.B * p.H * p.n_tiles;
  const int item = xcd_remap(blockIdx.x, total);
  const int ut = item % p.n_tiles;
  const int bh = item / p.n_tiles;
  const int h = bh % p.H;
  const int N = p.N;
  const int lo = p.bands.lo[h];
  const int hi = p.bands.hi[h];
  const size_t base = (size_t)bh * N * D;
  const bf16* __restrict__ qb = p.q + base;
  const bf16* __restrict__ dob = p.dout + base;
  const float* __restrict__ lseb = p.lse + (size_t)bh * N;
  const float* __restrict__ ddb = p.dvec + (size_t)bh * N;

  const int j0 = ut * kKvBK;
  const int j1 = min(N - 1, j0 + kKvBK - 1);
  const int kw0 = j0 + 32 * kw;
  const int kw1 = min(N - 1, kw0 + 31);
  const bool wave_live = kw0 <= N - 1;
  const bool wave_keys_full = kw0 + 31 <= N - 1;
  const int kj = kw0 + c32;
  const bool key_ok = kj < N;

  f32x16 acc[kDT];  // dV (P waves) or dK (dS waves)
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  const KeySpan qspan = band_query_span(j0, j1, lo, hi, N);
  if (qspan.last >= qspan.first) {
    // B operand of this wave's score product: K rows (P wave) or V rows (dS wave)
    bf16x8 bop[kKK];
    {
      const bf16* src = pwave ? p.k : p.v;
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk)
        bop[kk] = key_ok ? *(const bf16x8*)(src + base + (size_t)kj * D + 16 * kk + 8 * g) : bf16x8{};
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) settle(bop[kk]);
    }
    const float sl2 = p.scale_log2;
    const float scl = p.scale;
    const int tq_begin = qspan.first / kKvQB;
    const int tq_end = qspan.last / kKvQB + 1;
    auto issue = [&](int tq) {
      const int st = (tq - tq_begin) % kKvStages;
      bf16* t = smem + st * 2 * kTile;
      Tile::load(t, qb, tq * kKvQB, N, wave, lane);
      Tile::load(t + kTile, dob, tq * kKvQB, N, wave, lane);
      const int i = min(tq * kKvQB + (lane & 31), N - 1);
      const float* src = lane < 32 ? lseb + i : ddb + i;
      lds_dma4(__builtin_amdgcn_readfirstlane(lds_addr(&rowv[st][wave][0])), src);
    };
#pragma unroll
    for (int i = 0; i < kKvStages - 1; ++i)
      if (tq_begin + i < tq_end) issue(tq_begin + i);
    for (int tq = tq_begin; tq < tq_end; ++tq) {
      const int ahead = tq_end - 1 - tq;  // blocks issued after tq (at most kKvStages - 2 in flight)
      static_assert(kKvStages == 4, "the wait ladder below assumes a 4-deep ring");
      if (ahead >= 2)
        wait_vmcnt<2 * kL>();
      else if (ahead == 1)
        wait_vmcnt<kL>();
      else
        wait_vmcnt<0>();
      __syncthreads();  // block tq complete for everyone; block tq - 1 released
      if (tq + kKvStages - 1 < tq_end) issue(tq + kKvStages - 1);
      const int s = (tq - tq_begin) % kKvStages;
      const bf16* qs = smem + s * 2 * kTile;
      const bf16* dos = qs + kTile;
      const float* rv = &rowv[s][wave][0];
      const int i0 = tq * kKvQB;
      const int i1 = min(N - 1, i0 + kKvQB - 1);
      const bool act = wave_live && tile_meets(i0, i1, kw0, kw1, lo, hi);
      const bool full = wave_keys_full && i0 + kKvQB - 1 <= N - 1 && tile_full(i0, i1, kw0, kw1, lo, hi);
      const int prow = perm_row(c32);
      // per-lane row values of the 16 rows this lane holds: 16 (r / 8) + 8 g + (r % 8)
      auto rows16 = [&](const float* v, float* out) {
        const f32x4 a = *(const f32x4*)&v[8 * g], b = *(const f32x4*)&v[8 * g + 4];
        const f32x4 c = *(const f32x4*)&v[16 + 8 * g], d = *(const f32x4*)&v[20 + 8 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          out[e] = a[e];
          out[4 + e] = b[e];
          out[8 + e] = c[e];
          out[12 + e] = d[e];
        }
      };
      // ---- phase 1: P waves S -> P (handed over); dS waves dP
      bf16x8 op0{}, op1{};  // packed P (P waves) or dS (dS waves)
      f32x16 sc_;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc_[i] = 0.f;
      if (act) {
        const bf16* at = pwave ? qs : dos;
        bf16x8 aa[kKK];
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) aa[kk] = row_chunk<D>(at, prow, 16 * kk + 8 * g);
        __builtin_amdgcn_sched_barrier(0);
        sc_ = mfma_ksum<kKK>(aa, bop);
        if (pwave) {
          float nl[16], pv[16];
          rows16(rv, nl);
          if (full) {
#pragma unroll
            for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(__builtin_fmaf(sc_[i], sl2, -nl[i] * kLog2e));
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int r = perm_reg_row(i, g);
              const int dist = i0 + r - kj;
              const bool ok = key_ok && i0 + r < N && dist >= lo && dist <= hi;
              const float pe = fast_exp2(__builtin_fmaf(sc_[i], sl2, -nl[i] * kLog2e));
              pv[i] = ok ? pe : 0.f;
            }
          }
          f32x4* dst = (f32x4*)&pbuf[kw][lane][0];
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = f32x4{pv[4 * e], pv[4 * e + 1], pv[4 * e + 2], pv[4 * e + 3]};
          op0 = pack8(&pv[0]);
          op1 = pack8(&pv[8]);
        }
      }
      __syncthreads();  // P of this block visible to the dS waves
      // ---- phase 2: P waves dV += P^T dO; dS waves dS, dK += dS^T Q
      if (act) {
        const bf16* bt = pwave ? dos : qs;
        bf16x8 bb[2 * kDT];
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          bb[2 * dt] = kmajor_operand<D>(bt, 0, 32 * dt, lane);
          bb[2 * dt + 1] = kmajor_operand<D>(bt, 16, 32 * dt, lane);
        }
        if (!pwave) {
          float dd[16], pv[16], ds[16];
          rows16(rv + kKvQB, dd);
          const f32x4* src = (const f32x4*)&pbuf[kw][lane][0];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f32x4 t = src[e];
            pv[4 * e] = t[0];
            pv[4 * e + 1] = t[1];
            pv[4 * e + 2] = t[2];
            pv[4 * e + 3] = t[3];
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) ds[i] = pv[i] * (sc_[i] - dd[i]) * scl;
          op0 = pack8(&ds[0]);
          op1 = pack8(&ds[8]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) acc[dt] = mfma32(op0, bb[2 * dt], acc[dt]);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) acc[dt] = mfma32(op1, bb[2 * dt + 1], acc[dt]);
      }
    }
  }

  // dV (P waves) or dK (dS waves) rows: key kw0 + 8a + 4g + c, features 32dt + c32.
  if (wave_live) {
    const bool f32 = p.grad_f32 != 0;
    void* dst = pwave ? p.dv : p.dk;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kw0 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (j < N) {
          const size_t idx = base + (size_t)j * D + 32 * dt + c32;
          if (f32)
            ((float*)dst)[idx] = acc[dt][i];
          else
            ((bf16*)dst)[idx] = (bf16)acc[dt][i];
        }
      }
  }
}

}  // namespace

static BwdArgs make_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, bool grad_f32,
                         const Bands& bands, float scale, float* dvec) {
  BwdArgs a;
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.o = (const bf16*)o;
  a.dout = (const bf16*)dout;
  a.lse = lse;
  a.dvec = dvec;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.grad_f32 = grad_f32 ? 1 : 0;
  a.B = B;
  a.H = H;
  a.N = N;
  a.n_tiles = 0;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.bands = bands;
  return a;
}

int launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                       void* dq, int B, int H, int N, int d, bool grad_f32, const Bands& bands, float scale,
                       float* dvec, hipStream_t stream) {
  BwdArgs a = make_args(q, k, v, o, lse, dout, dq, nullptr, nullptr, B, H, N, grad_f32, bands, scale, dvec);
  a.n_tiles = (N + kDqBQ - 1) / kDqBQ;
  const long long total = (long long)B * H * a.n_tiles;
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  if (d == 128)
    hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)total), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3((unsigned)total), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

int launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                         void* dv, int B, int H, int N, int d, bool grad_f32, const Bands& bands, float scale,
                         float* dvec, hipStream_t stream) {
  BwdArgs a = make_args(q, k, v, nullptr, lse, dout, nullptr, dk, dv, B, H, N, grad_f32, bands, scale, dvec);
  a.n_tiles = (N + kKvBK - 1) / kKvBK;
  const long long total = (long long)B * H * a.n_tiles;
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  if (d == 128)
    hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3((unsigned)total), dim3(kKvThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3((unsigned)total), dim3(kKvThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

}  // namespace spattn
