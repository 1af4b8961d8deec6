// Backward of band-partitioned attention (textbook derivative of the
// masked-set softmax of "Sparse Attention, Then and Now" section 1 over the
// distance bands of "Making Every Head Count" Figure 1; no page gives a
// backward pass).  With P recomputed from the saved LSE:
//     D_i = dO_i . O_i,  dP = dO V^T,  dS = P * (dP - D),
//     dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// Kernels, all on the caller's stream:
//   bwd_pre      D_i for every row; zeroes the float32 dQ accumulator.
//   bwd_bf16     key-major: one workgroup per (b, h, 128-key tile), 4 waves of
//                32 keys; it walks only the 32-row query blocks that reach its
//                keys through the band, keeps dK and dV in registers and adds
//                its dQ share into the float32 accumulator with atomics.
//   bwd_dq_cast  float32 dQ accumulator -> bfloat16 (only for bf16 grads).
//   bwd_f32_*    plain float32 path (one wave per row, wave reductions).
#include "common.h"

namespace spattn {
namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------ preprocess
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                           float* __restrict__ dvec, float* __restrict__ dq_acc,
                                                           long long rows) {
  constexpr int kLanes = D / 8;  // threads per row, 8 elements each
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = gid / kLanes;
  const int part = (int)(gid % kLanes);
  float s = 0.f;
  if (row < rows) {
    const T* po = o + row * D + part * 8;
    const T* pd = dout + row * D + part * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)po[e] * (float)pd[e];
    float* pq = dq_acc + row * D + part * 8;
    *(f32x4*)pq = f32x4{0, 0, 0, 0};
    *(f32x4*)(pq + 4) = f32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int off = kLanes / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && part == 0) dvec[row] = s;
}

// ------------------------------------------------------------ dQ cast
__global__ __launch_bounds__(kThreads) void bwd_dq_cast_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                               long long n8) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *(const f32x4*)(acc + i * 8);
  const f32x4 b = *(const f32x4*)(acc + i * 8 + 4);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (bf16)a[e];
    r[4 + e] = (bf16)b[e];
  }
  *(bf16x8*)(dq + i * 8) = r;
}

// ------------------------------------------------------------ bf16 main
constexpr int kKeys = 128;  // keys per workgroup
constexpr int kQB = 32;     // query rows per step
constexpr int kPad = 8;

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* lse;
  const float* dvec;
  float* dq_acc;
  void* dk;
  void* dv;
  int grad_f32;
  int B, H, N;
  int n_kt;
  float scale;
  float scale_log2;
  Bands bands;
};

template <int D>
struct BwdSmem {
  static constexpr int kRow = D + kPad;       // Q, dO row-major
  static constexpr int kTRow = kQB + kPad;    // Q^T, dO^T
  static constexpr int kSRow = kKeys + kPad;  // dS [query][key], K^T [d][key]
  static constexpr int kQ = 0;
  static constexpr int kDO = kQ + kQB * kRow;
  static constexpr int kQT = kDO + kQB * kRow;
  static constexpr int kDOT = kQT + D * kTRow;
  static constexpr int kDS = kDOT + D * kTRow;
  static constexpr int kKT = kDS + kQB * kSRow;
  static constexpr int kEnd = kKT + D * kSRow;  // bf16 elements
};

template <typename OutT>
__device__ __forceinline__ void store_grad(void* base, size_t idx, float x) {
  ((OutT*)base)[idx] = (OutT)x;
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_bf16_kernel(BwdArgs p) {
  using SM = BwdSmem<D>;
  constexpr int kKK = D / 16;
  constexpr int kDT = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 smem[SM::kEnd];
  __shared__ float lse_s[kQB];
  __shared__ float dd_s[kQB];
  bf16* Qs = smem + SM::kQ;
  bf16* dOs = smem + SM::kDO;
  bf16* QTs = smem + SM::kQT;
  bf16* dOTs = smem + SM::kDOT;
  bf16* dSs = smem + SM::kDS;
  bf16* KTs = smem + SM::kKT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const int total = p.B * p.H * p.n_kt;
  const int item = xcd_remap(blockIdx.x, total);
  const int ut = item % p.n_kt;
  const int bh = item / p.n_kt;
  const int h = bh % p.H;
  const int N = p.N;
  const int lo = p.bands.lo[h];
  const int hi = p.bands.hi[h];
  const size_t base = (size_t)bh * N * D;
  const bf16* __restrict__ qb = p.q + base;
  const bf16* __restrict__ kb = p.k + base;
  const bf16* __restrict__ vb = p.v + base;
  const bf16* __restrict__ dob = p.dout + base;
  const float* __restrict__ lseb = p.lse + (size_t)bh * N;
  const float* __restrict__ ddb = p.dvec + (size_t)bh * N;
  float* __restrict__ dqa = p.dq_acc + base;

  const int j0 = ut * kKeys;
  const int j1 = min(N - 1, j0 + kKeys - 1);
  const int kw0 = j0 + 32 * wave;
  const int kw1 = min(N - 1, kw0 + 31);
  const bool wave_live = kw0 <= N - 1;
  const int kj = kw0 + c32;  // this lane's key (S columns)

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
    // K, V operands (B of S = Q K^T and dP = dO V^T): lane holds row kj.
    bf16x8 kop[kKK], vop[kKK];
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      if (kj < N) {
        kop[kk] = *(const bf16x8*)(kb + (size_t)kj * D + 16 * kk + 8 * g);
        vop[kk] = *(const bf16x8*)(vb + (size_t)kj * D + 16 * kk + 8 * g);
      } else {
        kop[kk] = bf16x8{};
        vop[kk] = bf16x8{};
      }
    }
    // K^T of the whole key tile into LDS (B operand of dQ = dS K).
    {
      constexpr int kChunks = D / 8;
      for (int unit = tid; unit < (kKeys / 4) * kChunks; unit += kThreads) {
        const int kg = unit % (kKeys / 4), dc = unit / (kKeys / 4);
        u32x4 r4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + 4 * kg + r;
          r4[r] = j < N ? *(const u32x4*)(kb + (size_t)j * D + dc * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1, sh = (e & 1) * 16;
          const uint32_t a0 = (r4[0][w] >> sh) & 0xffffu, a1 = (r4[1][w] >> sh) & 0xffffu;
          const uint32_t a2 = (r4[2][w] >> sh) & 0xffffu, a3 = (r4[3][w] >> sh) & 0xffffu;
          *(u32x2*)(KTs + (dc * 8 + e) * SM::kSRow + 4 * kg) = u32x2{a0 | (a1 << 16), a2 | (a3 << 16)};
        }
      }
    }
    const float sl2 = p.scale_log2;
    const float scl = p.scale;
    const int tq_begin = qspan.first / kQB;
    const int tq_end = qspan.last / kQB + 1;
    for (int tq = tq_begin; tq < tq_end; ++tq) {
      const int i0 = tq * kQB;
      const int i1 = min(N - 1, i0 + kQB - 1);
      // ---- stage Q, dO (row-major and transposed), LSE, D
      {
        constexpr int kChunks = D / 8;
        for (int unit = tid; unit < kQB * kChunks; unit += kThreads) {
          const int r = unit / kChunks, cc = unit % kChunks;
          const int i = i0 + r;
          const u32x4 zq = i < N ? *(const u32x4*)(qb + (size_t)i * D + cc * 8) : u32x4{0, 0, 0, 0};
          const u32x4 zd = i < N ? *(const u32x4*)(dob + (size_t)i * D + cc * 8) : u32x4{0, 0, 0, 0};
          *(u32x4*)(Qs + r * SM::kRow + cc * 8) = zq;
          *(u32x4*)(dOs + r * SM::kRow + cc * 8) = zd;
        }
        // transposed copies, 2 rows x 8 features per unit
        for (int unit = tid; unit < (kQB / 2) * kChunks; unit += kThreads) {
          const int rg = unit % (kQB / 2), dc = unit / (kQB / 2);
          const int ia = i0 + 2 * rg, ib = ia + 1;
          const u32x4 qa = ia < N ? *(const u32x4*)(qb + (size_t)ia * D + dc * 8) : u32x4{0, 0, 0, 0};
          const u32x4 qbv = ib < N ? *(const u32x4*)(qb + (size_t)ib * D + dc * 8) : u32x4{0, 0, 0, 0};
          const u32x4 da = ia < N ? *(const u32x4*)(dob + (size_t)ia * D + dc * 8) : u32x4{0, 0, 0, 0};
          const u32x4 dbv = ib < N ? *(const u32x4*)(dob + (size_t)ib * D + dc * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int w = e >> 1, sh = (e & 1) * 16;
            *(uint32_t*)(QTs + (dc * 8 + e) * SM::kTRow + 2 * rg) =
                ((qa[w] >> sh) & 0xffffu) | (((qbv[w] >> sh) & 0xffffu) << 16);
            *(uint32_t*)(dOTs + (dc * 8 + e) * SM::kTRow + 2 * rg) =
                ((da[w] >> sh) & 0xffffu) | (((dbv[w] >> sh) & 0xffffu) << 16);
          }
        }
        if (tid < kQB) {
          const int i = i0 + tid;
          lse_s[tid] = i < N ? lseb[i] * kLog2e : 0.f;
          dd_s[tid] = i < N ? ddb[i] : 0.f;
        }
      }
      __syncthreads();

      const bool act = wave_live && tile_meets(i0, i1, kw0, kw1, lo, hi);
      if (act) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[i] = 0.f;
          pacc[i] = 0.f;
        }
        const bf16* qrow = Qs + perm_row(c32) * SM::kRow + 8 * g;
        const bf16* drow = dOs + perm_row(c32) * SM::kRow + 8 * g;
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) {
          sacc = mfma32(*(const bf16x8*)(qrow + 16 * kk), kop[kk], sacc);
          pacc = mfma32(*(const bf16x8*)(drow + 16 * kk), vop[kk], pacc);
        }
        const bool full = tile_full(i0, i1, kw0, kw1, lo, hi) && (i0 + kQB - 1 <= N - 1);
        float pv[16], ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = perm_reg_row(i, g);
          const int dist = i0 + r - kj;
          const bool ok = full || (i0 + r < N && dist >= lo && dist <= hi);
          const float pe = fast_exp2(sacc[i] * sl2 - lse_s[r]);
          pv[i] = ok ? pe : 0.f;
          ds[i] = pv[i] * (pacc[i] - dd_s[r]) * scl;
        }
        const bf16x8 pp0 = pack8(&pv[0]), pp1 = pack8(&pv[8]);
        const bf16x8 sp0 = pack8(&ds[0]), sp1 = pack8(&ds[8]);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          const bf16* dorow = dOTs + (32 * dt + c32) * SM::kTRow + 8 * g;
          const bf16* qtrow = QTs + (32 * dt + c32) * SM::kTRow + 8 * g;
          dvacc[dt] = mfma32(pp0, *(const bf16x8*)(dorow), dvacc[dt]);
          dvacc[dt] = mfma32(pp1, *(const bf16x8*)(dorow + 16), dvacc[dt]);
          dkacc[dt] = mfma32(sp0, *(const bf16x8*)(qtrow), dkacc[dt]);
          dkacc[dt] = mfma32(sp1, *(const bf16x8*)(qtrow + 16), dkacc[dt]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) dSs[perm_reg_row(i, g) * SM::kSRow + 32 * wave + c32] = (bf16)ds[i];
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) dSs[perm_reg_row(i, g) * SM::kSRow + 32 * wave + c32] = (bf16)0.f;
      }
      __syncthreads();

      // ---- dQ[i0 .. i0+31, :] += dS (32 x 128) K (128 x D)
      {
        constexpr int kSplit = 4 / kDT;  // key splits per output block
        const int dt = wave % kDT;
        const int part = wave / kDT;
        constexpr int kSteps = (kKeys / 16) / kSplit;
        f32x16 qacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) qacc[i] = 0.f;
        const bf16* arow = dSs + c32 * SM::kSRow + 8 * g;
        const bf16* brow = KTs + (32 * dt + c32) * SM::kSRow + 8 * g;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          const int kk = part * kSteps + s;
          qacc = mfma32(*(const bf16x8*)(arow + 16 * kk), *(const bf16x8*)(brow + 16 * kk), qacc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * g + (i & 3);
          if (i0 + r < N) atomicAdd(dqa + (size_t)(i0 + r) * D + 32 * dt + c32, qacc[i]);
        }
      }
      // the next step's staging writes only Q/dO/LSE/D buffers, which every
      // wave finished reading before the barrier above; dS and K^T are read
      // here and rewritten only after the next step's first barrier.
    }
  }

  // ---- dK, dV (rows this wave owns: keys kw0 + 8a + 4g + c)
  if (wave_live) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kw0 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (j < N) {
          const size_t idx = base + (size_t)j * D + 32 * dt + c32;
          if (p.grad_f32) {
            store_grad<float>(p.dk, idx, dkacc[dt][i]);
            store_grad<float>(p.dv, idx, dvacc[dt][i]);
          } else {
            store_grad<bf16>(p.dk, idx, dkacc[dt][i]);
            store_grad<bf16>(p.dv, idx, dvacc[dt][i]);
          }
        }
      }
  }
}

// ------------------------------------------------------------ f32 path
template <int D>
__device__ __forceinline__ float wave_dot(const float* a, const float* b, int lane) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) s += a[e] * b[e];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  (void)lane;
  return s;
}

struct BwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* dout;
  const float* lse;
  const float* dvec;
  float* dq;
  float* dk;
  float* dv;
  int B, H, N;
  float scale;
  Bands bands;
};

// One wave per query row: dQ_i = scale * sum_j dS_ij k_j.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_f32_dq_kernel(BwdF32Args p) {
  constexpr int kE = D / 64;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long rows = (long long)p.B * p.H * p.N;
  if (row >= rows) return;
  const int i = (int)(row % p.N);
  const long long bh = row / p.N;
  const int h = (int)(bh % p.H);
  const int lo = p.bands.lo[h], hi = p.bands.hi[h];
  const size_t base = (size_t)bh * p.N * D;
  float qi[kE], di[kE], acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    qi[e] = p.q[base + (size_t)i * D + lane + 64 * e];
    di[e] = p.dout[base + (size_t)i * D + lane + 64 * e];
    acc[e] = 0.f;
  }
  const float lse = p.lse[row], dd = p.dvec[row];
  const KeySpan ks = band_key_span(i, i, lo, hi);
  for (int j = ks.first; j <= ks.last; ++j) {
    float kj[kE], vj[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      kj[e] = p.k[base + (size_t)j * D + lane + 64 * e];
      vj[e] = p.v[base + (size_t)j * D + lane + 64 * e];
    }
    const float s = wave_dot<D>(qi, kj, lane) * p.scale;
    const float pij = expf(s - lse);
    const float dp = wave_dot<D>(di, vj, lane);
    const float ds = pij * (dp - dd);
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] += ds * kj[e];
  }
#pragma unroll
  for (int e = 0; e < kE; ++e) p.dq[base + (size_t)i * D + lane + 64 * e] = acc[e] * p.scale;
}

// One wave per key row: dK_j = scale * sum_i dS_ij q_i, dV_j = sum_i P_ij dO_i.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_f32_dkdv_kernel(BwdF32Args p) {
  constexpr int kE = D / 64;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long rows = (long long)p.B * p.H * p.N;
  if (row >= rows) return;
  const int j = (int)(row % p.N);
  const long long bh = row / p.N;
  const int h = (int)(bh % p.H);
  const int lo = p.bands.lo[h], hi = p.bands.hi[h];
  const size_t base = (size_t)bh * p.N * D;
  const size_t lbase = (size_t)bh * p.N;
  float kj[kE], vj[kE], dk[kE], dv[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    kj[e] = p.k[base + (size_t)j * D + lane + 64 * e];
    vj[e] = p.v[base + (size_t)j * D + lane + 64 * e];
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const KeySpan qs = band_query_span(j, j, lo, hi, p.N);
  for (int i = qs.first; i <= qs.last; ++i) {
    float qi[kE], di[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      qi[e] = p.q[base + (size_t)i * D + lane + 64 * e];
      di[e] = p.dout[base + (size_t)i * D + lane + 64 * e];
    }
    const float s = wave_dot<D>(qi, kj, lane) * p.scale;
    const float pij = expf(s - p.lse[lbase + i]);
    const float dp = wave_dot<D>(di, vj, lane);
    const float ds = pij * (dp - p.dvec[lbase + i]);
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      dk[e] += ds * qi[e];
      dv[e] += pij * di[e];
    }
  }
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    p.dk[base + (size_t)j * D + lane + 64 * e] = dk[e] * p.scale;
    p.dv[base + (size_t)j * D + lane + 64 * e] = dv[e];
  }
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d, int dtype, int grad_dtype) {
  const size_t rows = (size_t)B * H * N;
  size_t bytes = (rows * sizeof(float) + 255) / 256 * 256;  // D vector
  const bool need_acc = !(dtype == SPATTN_F32 || grad_dtype == SPATTN_F32);
  if (need_acc) bytes += (rows * d * sizeof(float) + 255) / 256 * 256;
  return bytes;
}

int launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, int B, int H, int N, int d, int dtype, int grad_dtype,
               const Bands& bands, float scale, void* workspace, hipStream_t stream) {
  const long long rows = (long long)B * H * N;
  float* dvec = (float*)workspace;
  const size_t dbytes = ((size_t)rows * sizeof(float) + 255) / 256 * 256;
  const bool grads_f32 = dtype == SPATTN_F32 || grad_dtype == SPATTN_F32;
  float* dq_acc = grads_f32 ? (float*)dq : (float*)((char*)workspace + dbytes);

  // preprocess
  {
    const long long threads = rows * (d / 8);
    dim3 grid((unsigned)((threads + kThreads - 1) / kThreads)), block(kThreads);
    if (dtype == SPATTN_BF16) {
      if (d == 128)
        hipLaunchKernelGGL((bwd_pre_kernel<bf16, 128>), grid, block, 0, stream, (const bf16*)o, (const bf16*)dout,
                           dvec, dq_acc, rows);
      else
        hipLaunchKernelGGL((bwd_pre_kernel<bf16, 64>), grid, block, 0, stream, (const bf16*)o, (const bf16*)dout,
                           dvec, dq_acc, rows);
    } else {
      if (d == 128)
        hipLaunchKernelGGL((bwd_pre_kernel<float, 128>), grid, block, 0, stream, (const float*)o,
                           (const float*)dout, dvec, dq_acc, rows);
      else
        hipLaunchKernelGGL((bwd_pre_kernel<float, 64>), grid, block, 0, stream, (const float*)o,
                           (const float*)dout, dvec, dq_acc, rows);
    }
    if (hipGetLastError() != hipSuccess) return SPATTN_E_HIP;
  }

  if (dtype == SPATTN_BF16) {
    BwdArgs a;
    a.q = (const bf16*)q;
    a.k = (const bf16*)k;
    a.v = (const bf16*)v;
    a.dout = (const bf16*)dout;
    a.lse = lse;
    a.dvec = dvec;
    a.dq_acc = dq_acc;
    a.dk = dk;
    a.dv = dv;
    a.grad_f32 = grads_f32 ? 1 : 0;
    a.B = B;
    a.H = H;
    a.N = N;
    a.n_kt = (N + kKeys - 1) / kKeys;
    a.scale = scale;
    a.scale_log2 = scale * kLog2e;
    a.bands = bands;
    const long long total = (long long)B * H * a.n_kt;
    if (total > 0x7fffffffLL) return SPATTN_E_ARG;
    dim3 grid((unsigned)total), block(kThreads);
    if (d == 128)
      hipLaunchKernelGGL(bwd_bf16_kernel<128>, grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL(bwd_bf16_kernel<64>, grid, block, 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPATTN_E_HIP;
    if (!grads_f32) {
      const long long n8 = rows * d / 8;
      dim3 g2((unsigned)((n8 + kThreads - 1) / kThreads));
      hipLaunchKernelGGL(bwd_dq_cast_kernel, g2, block, 0, stream, dq_acc, (bf16*)dq, n8);
      if (hipGetLastError() != hipSuccess) return SPATTN_E_HIP;
    }
    return SPATTN_OK;
  }

  BwdF32Args a;
  a.q = (const float*)q;
  a.k = (const float*)k;
  a.v = (const float*)v;
  a.dout = (const float*)dout;
  a.lse = lse;
  a.dvec = dvec;
  a.dq = (float*)dq;
  a.dk = (float*)dk;
  a.dv = (float*)dv;
  a.B = B;
  a.H = H;
  a.N = N;
  a.scale = scale;
  a.bands = bands;
  dim3 grid((unsigned)((rows + 3) / 4)), block(kThreads);
  if (d == 128) {
    hipLaunchKernelGGL(bwd_f32_dq_kernel<128>, grid, block, 0, stream, a);
    hipLaunchKernelGGL(bwd_f32_dkdv_kernel<128>, grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL(bwd_f32_dq_kernel<64>, grid, block, 0, stream, a);
    hipLaunchKernelGGL(bwd_f32_dkdv_kernel<64>, grid, block, 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

}  // namespace spattn
