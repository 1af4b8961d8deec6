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
//   bwd_dkdv  key-major, one workgroup per (b, h, 128 key rows), 4 waves of 32
//             keys.  Walks the 32-row query blocks that reach its keys:
//             S = Q K^T, dP = dO V^T, dS, dV += P^T dO, dK += dS^T Q, with dK
//             and dV held in registers for the whole walk (dO and Q enter the
//             last two products through the LDS transpose read).
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
constexpr int kDqBQ = 128;  // query rows per workgroup
constexpr int kDqBK = 32;   // key rows per stage

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs p) {
  constexpr int kS = TileRow<D>::kStride;
  constexpr int kTile = kDqBK * kS;
  constexpr int kKK = D / 16;
  constexpr int kDT = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * kTile];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
    TileCopy<kDqBK, D, kThreads> kcp, vcp;
    kcp.load(kb, u_begin * kDqBK, N, tid);
    vcp.load(vb, u_begin * kDqBK, N, tid);
    kcp.store(smem, tid);
    vcp.store(smem + kTile, tid);
    __syncthreads();
    for (int u = u_begin; u < u_end; ++u) {
      const int s = (u - u_begin) & 1;
      const bool has_next = u + 1 < u_end;
      if (has_next) {
        kcp.load(kb, (u + 1) * kDqBK, N, tid);
        vcp.load(vb, (u + 1) * kDqBK, N, tid);
      }
      const bf16* ks = smem + s * 2 * kTile;
      const bf16* vs = ks + kTile;
      const int jb = u * kDqBK;
      if (wave_live && tile_meets(iw0, iw1, jb, jb + 31, lo, hi)) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[i] = 0.f;
          pacc[i] = 0.f;
        }
        const bf16* krow = ks + perm_row(c32) * kS + 8 * g;
        const bf16* vrow = vs + perm_row(c32) * kS + 8 * g;
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) {
          sacc = mfma32(*(const bf16x8*)(krow + 16 * kk), qreg[kk], sacc);
          pacc = mfma32(*(const bf16x8*)(vrow + 16 * kk), doreg[kk], pacc);
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
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          acc[dt] = mfma32(kmajor_operand(ks, kS, 0, 32 * dt, lane), d0, acc[dt]);
          acc[dt] = mfma32(kmajor_operand(ks, kS, 16, 32 * dt, lane), d1, acc[dt]);
        }
      }
      if (has_next) {
        bf16* nxt = smem + (s ^ 1) * 2 * kTile;
        kcp.store(nxt, tid);
        vcp.store(nxt + kTile, tid);
      }
      __syncthreads();
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
constexpr int kKvBK = 128;  // key rows per workgroup
constexpr int kKvQB = 32;   // query rows per stage

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(BwdArgs p) {
  constexpr int kS = TileRow<D>::kStride;
  constexpr int kTile = kKvQB * kS;
  constexpr int kKK = D / 16;
  constexpr int kDT = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * kTile];  // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float lse_s[2][kKvQB];     // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float dd_s[2][kKvQB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  const int kw0 = j0 + 32 * wave;
  const int kw1 = min(N - 1, kw0 + 31);
  const bool wave_live = kw0 <= N - 1;
  const bool wave_keys_full = kw0 + 31 <= N - 1;
  const int kj = kw0 + c32;
  const bool key_ok = kj < N;

  f32x16 dvacc[kDT], dkacc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dvacc[dt][i] = 0.f;
      dkacc[dt][i] = 0.f;
    }

  const KeySpan qspan = band_query_span(j0, j1, lo, hi, N);
  if (qspan.last >= qspan.first) {
    bf16x8 kop[kKK], vop[kKK];
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      const size_t off = base + (size_t)kj * D + 16 * kk + 8 * g;
      kop[kk] = key_ok ? *(const bf16x8*)(p.k + off) : bf16x8{};
      vop[kk] = key_ok ? *(const bf16x8*)(p.v + off) : bf16x8{};
    }
    TileCopy<kKvQB, D, kThreads> qcp, dcp;
    float lse_n = 0.f, dd_n = 0.f;
    auto load_blk = [&](int tq) {
      qcp.load(qb, tq * kKvQB, N, tid);
      dcp.load(dob, tq * kKvQB, N, tid);
      if (tid < kKvQB) {
        const int i = tq * kKvQB + tid;
        lse_n = i < N ? lseb[i] * kLog2e : 0.f;
        dd_n = i < N ? ddb[i] : 0.f;
      }
    };
    auto store_blk = [&](int s) {
      bf16* st = smem + s * 2 * kTile;
      qcp.store(st, tid);
      dcp.store(st + kTile, tid);
      if (tid < kKvQB) {
        lse_s[s][tid] = lse_n;
        dd_s[s][tid] = dd_n;
      }
    };

    const float sl2 = p.scale_log2;
    const float scl = p.scale;
    const int tq_begin = qspan.first / kKvQB;
    const int tq_end = qspan.last / kKvQB + 1;
    load_blk(tq_begin);
    store_blk(0);
    __syncthreads();
    for (int tq = tq_begin; tq < tq_end; ++tq) {
      const int s = (tq - tq_begin) & 1;
      const bool has_next = tq + 1 < tq_end;
      if (has_next) load_blk(tq + 1);
      const bf16* qs = smem + s * 2 * kTile;
      const bf16* dos = qs + kTile;
      const int i0 = tq * kKvQB;
      const int i1 = min(N - 1, i0 + kKvQB - 1);
      // P and dS of this wave's 32 keys x 32 rows; zero when the rows miss the
      // wave's band strip.  The dV / dK products below run unconditionally so
      // their accumulators stay in place across iterations.
      bf16x8 pp0{}, pp1{}, sp0{}, sp1{};
      if (wave_live && tile_meets(i0, i1, kw0, kw1, lo, hi)) {
        // LSE and D of the rows this lane holds: 16 * (r / 8) + 8 g + (r % 8)
        const f32x4 l0 = *(const f32x4*)&lse_s[s][8 * g], l1 = *(const f32x4*)&lse_s[s][8 * g + 4];
        const f32x4 l2 = *(const f32x4*)&lse_s[s][16 + 8 * g], l3 = *(const f32x4*)&lse_s[s][20 + 8 * g];
        const f32x4 e0 = *(const f32x4*)&dd_s[s][8 * g], e1 = *(const f32x4*)&dd_s[s][8 * g + 4];
        const f32x4 e2 = *(const f32x4*)&dd_s[s][16 + 8 * g], e3 = *(const f32x4*)&dd_s[s][20 + 8 * g];
        const float lrow[16] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3],
                                l2[0], l2[1], l2[2], l2[3], l3[0], l3[1], l3[2], l3[3]};
        const float drow_[16] = {e0[0], e0[1], e0[2], e0[3], e1[0], e1[1], e1[2], e1[3],
                                 e2[0], e2[1], e2[2], e2[3], e3[0], e3[1], e3[2], e3[3]};
        const bf16* qrow = qs + perm_row(c32) * kS + 8 * g;
        const bf16* drow = dos + perm_row(c32) * kS + 8 * g;
        const bool full = wave_keys_full && i0 + kKvQB - 1 <= N - 1 && tile_full(i0, i1, kw0, kw1, lo, hi);
        float pv[16], ds[16];
        {
          f32x16 sacc;
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
          for (int kk = 0; kk < kKK; ++kk) sacc = mfma32(*(const bf16x8*)(qrow + 16 * kk), kop[kk], sacc);
          if (full) {
#pragma unroll
            for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(__builtin_fmaf(sacc[i], sl2, -lrow[i]));
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int r = perm_reg_row(i, g);
              const int dist = i0 + r - kj;
              const bool ok = key_ok && i0 + r < N && dist >= lo && dist <= hi;
              const float pe = fast_exp2(__builtin_fmaf(sacc[i], sl2, -lrow[i]));
              pv[i] = ok ? pe : 0.f;
            }
          }
        }
        {
          f32x16 pacc;
#pragma unroll
          for (int i = 0; i < 16; ++i) pacc[i] = 0.f;
#pragma unroll
          for (int kk = 0; kk < kKK; ++kk) pacc = mfma32(*(const bf16x8*)(drow + 16 * kk), vop[kk], pacc);
#pragma unroll
          for (int i = 0; i < 16; ++i) ds[i] = pv[i] * (pacc[i] - drow_[i]) * scl;
        }
        pp0 = pack8(&pv[0]);
        pp1 = pack8(&pv[8]);
        sp0 = pack8(&ds[0]);
        sp1 = pack8(&ds[8]);
      }
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        dvacc[dt] = mfma32(pp0, kmajor_operand(dos, kS, 0, 32 * dt, lane), dvacc[dt]);
        dvacc[dt] = mfma32(pp1, kmajor_operand(dos, kS, 16, 32 * dt, lane), dvacc[dt]);
        dkacc[dt] = mfma32(sp0, kmajor_operand(qs, kS, 0, 32 * dt, lane), dkacc[dt]);
        dkacc[dt] = mfma32(sp1, kmajor_operand(qs, kS, 16, 32 * dt, lane), dkacc[dt]);
      }
      if (has_next) store_blk(s ^ 1);
      __syncthreads();
    }
  }

  // dK, dV rows of this wave: key kw0 + 8a + 4g + c, features 32dt + c32.
  if (wave_live) {
    const bool f32 = p.grad_f32 != 0;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kw0 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (j < N) {
          const size_t idx = base + (size_t)j * D + 32 * dt + c32;
          if (f32) {
            ((float*)p.dk)[idx] = dkacc[dt][i];
            ((float*)p.dv)[idx] = dvacc[dt][i];
          } else {
            ((bf16*)p.dk)[idx] = (bf16)dkacc[dt][i];
            ((bf16*)p.dv)[idx] = (bf16)dvacc[dt][i];
          }
        }
      }
  }
}

}  // namespace

int launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                    void* dq, void* dk, void* dv, int B, int H, int N, int d, bool grad_f32, const Bands& bands,
                    float scale, float* dvec, hipStream_t stream) {
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
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.bands = bands;
  dim3 block(kThreads);
  a.n_tiles = (N + kDqBQ - 1) / kDqBQ;
  long long total = (long long)B * H * a.n_tiles;
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  if (d == 128)
    hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)total), block, 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3((unsigned)total), block, 0, stream, a);
  if (hipGetLastError() != hipSuccess) return SPATTN_E_HIP;
  a.n_tiles = (N + kKvBK - 1) / kKvBK;
  total = (long long)B * H * a.n_tiles;
  if (d == 128)
    hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3((unsigned)total), block, 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3((unsigned)total), block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

}  // namespace spattn
