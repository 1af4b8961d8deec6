// Band-partitioned attention forward in float32 throughout, gfx950 fp32 MFMA
// (v_mfma_f32_32x32x2_f32: full float32 products, no reduced-precision
// inputs).  Same computation as the bfloat16 kernel: the masked-set softmax of
// "Sparse Attention, Then and Now" section 1 over each head's distance band
// ("Making Every Head Count", Figure 1 caption).
//
// One workgroup = (b, h, 64 query rows), 2 waves of 32 rows; key tiles of
// 32 rows staged in LDS (double buffered), visited only inside the band
// strip.  A workgroup's walk covers the strips of all its waves, and a wave
// idles at the tile barrier on tiles outside its own, so two waves per
// workgroup waste less than four.  S^T = K Q^T and O^T += V^T P^T as in the bfloat16 kernel; with a
// k-depth of 2 per product the operands are single floats, so V is read
// row-major from LDS without a transpose.  In S^T, product kk takes feature
// kk in lanes 0-31 and feature D/2 + kk in lanes 32-63, so a lane's K
// operands for four consecutive products are one 16-byte LDS read.
#include "common.h"

namespace spattn {
namespace {

constexpr int kBQ = 64;        // query rows per workgroup of fwd_f32_kernel (2 waves)
constexpr int kFwdThreads = 128;
constexpr int kBK = 32;
constexpr int kThreads = 256;  // the split kernel's workgroup (4 waves)
// query-major: 64 rows own 32-key tiles, ascending
constexpr WalkShape kWalk{kBQ, kBK, false, false};

struct FwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, H, N;  // sequences (B), heads, tokens per sequence (the longest, when packed)
  int n_qt;
  int local_window;  // shared local window width (0: exclusive bands)
  float scale_log2;
  const int32_t* cu;  // packed sequence offsets [B + 1] (device), or null
  int T;              // packed: tokens per head
  int own_bdp;        // packed: each sequence's own BDP bands
  Bands bands;
};

template <int D>
struct F32Smem {
  static constexpr int kKRow = D + 4;  // 16-byte rows; 16 lanes' row reads on distinct banks
  static constexpr int kVRow = D + 8;  // rows 4 apart land 32 banks apart
  static constexpr int kKStage = kBK * kKRow;
  static constexpr int kStage = kKStage + kBK * kVRow;
};

template <int D>
__global__ __launch_bounds__(kFwdThreads) void fwd_f32_kernel(FwdF32Args p) {
  using SM = F32Smem<D>;
  constexpr int kDT = D / 32;
  constexpr int kKK = D / 2;
  constexpr int kLoads = kBK * D / 4 / kFwdThreads;  // float4 loads per thread per tensor
  __shared__ __align__(16) float smem[2 * SM::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const WorkItem wi = work_item(blockIdx.x, p.B, p.H, p.n_qt, true);
  if (!wi.valid) return;  // padding pair
  const int t = wi.t;
  const int h = wi.h;
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, wi.b, h);
  const int N = sh.n;
  if (t * kBQ >= N) return;  // past the end of a packed sequence
  // the head's distance set: its band, joined with the local window if any
  const DistSet dset = dist_set(sh.lo, sh.hi, p.local_window);
  const int lo = dset.lo;
  const int hi = dset.hi;
  const size_t base = sh.row0 * D;
  const float* __restrict__ qb = p.q + base;
  const float* __restrict__ kb = p.k + base;
  const float* __restrict__ vb = p.v + base;
  float* __restrict__ ob = p.o + base;
  float* __restrict__ lb = p.lse + sh.row0;
  const float ninf = -__builtin_inff();

  const int i_tile0 = t * kBQ;
  const TileWalk walk = kernel_walk(kWalk, i_tile0, N, dset);
  if (walk.n == 0) {
    for (int c = tid; c < kBQ * (D / 4); c += kFwdThreads) {
      const int r = c / (D / 4), cc = c % (D / 4);
      if (i_tile0 + r < N) *(f32x4*)(ob + (size_t)(i_tile0 + r) * D + cc * 4) = f32x4{0, 0, 0, 0};
    }
    for (int r = tid; r < kBQ; r += kFwdThreads)
      if (i_tile0 + r < N) lb[i_tile0 + r] = ninf;
    return;
  }
  const int iw0 = i_tile0 + 32 * wave;
  const int iw1 = min(N - 1, iw0 + 31);
  const bool wave_live = iw0 <= N - 1;
  const int iq = iw0 + c32;

  f32x4 qreg[kKK / 4];  // features g * D/2 .. g * D/2 + D/2 - 1 of row iq
#pragma unroll
  for (int c = 0; c < kKK / 4; ++c)
    qreg[c] = iq < N ? *(const f32x4*)(qb + (size_t)iq * D + g * kKK + 4 * c) : f32x4{0, 0, 0, 0};

  f32x4 kreg[kLoads], vreg[kLoads];
  auto load_tile = [&](int u) {
    const int j0 = u * kBK;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + kFwdThreads * r;
      const int row = c / (D / 4), col = c % (D / 4);
      const int j = j0 + row;
      kreg[r] = j < N ? *(const f32x4*)(kb + (size_t)j * D + col * 4) : f32x4{0, 0, 0, 0};
      vreg[r] = j < N ? *(const f32x4*)(vb + (size_t)j * D + col * 4) : f32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int s) {
    float* ks = smem + s * SM::kStage;
    float* vs = ks + SM::kKStage;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + kFwdThreads * r;
      const int row = c / (D / 4), col = c % (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ks[row * SM::kKRow + col * 4 + e] = kreg[r][e];
        vs[row * SM::kVRow + col * 4 + e] = vreg[r][e];
      }
    }
  };

  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m_run = ninf, l_run = 0.f;
  const float sl2 = p.scale_log2;

  load_tile(walk.at(0));
  store_tile(0);
  __syncthreads();

  for (int v = 0; v < walk.n; ++v) {
    const int s = v & 1;
    const bool has_next = v + 1 < walk.n;
    if (has_next) load_tile(walk.at(v + 1));
    const float* ks = smem + s * SM::kStage;
    const float* vs = ks + SM::kKStage;
    const int jb = walk.at(v) * kBK;
    const bool act = wave_live && set_meets(iw0, iw1, jb, jb + 31, dset);
    if (act) {
      f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
      for (int c = 0; c < kKK / 4; ++c) {
        const f32x4 ka = *(const f32x4*)(ks + c32 * SM::kKRow + g * kKK + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc = mfma32_f32(ka[e], qreg[c][e], sacc);
      }
      float x[16];
      const bool full = set_full(iw0, iw1, jb, jb + 31, dset);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = jb + 8 * (i >> 2) + 4 * g + (i & 3);
        const int dist = iq - j;
        const bool in = (dist >= lo && dist <= hi) || (dist >= dset.nlo && dist <= dset.nhi);
        x[i] = (full || in) ? sacc[i] * sl2 : ninf;
      }
      float mx = ninf;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == ninf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = fast_exp2(x[i] - m_use);
        psum += x[i];
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = 8 * (i >> 2) + 4 * g + (i & 3);
          acc[dt] = mfma32_f32(vs[j * SM::kVRow + 32 * dt + c32], x[i], acc[dt]);
        }
      }
    }
    if (has_next) store_tile(s ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (iq < N) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 w;
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] = acc[dt][4 * a + c] * inv;
        *(f32x4*)(ob + (size_t)iq * D + 32 * dt + 8 * a + 4 * g) = w;
      }
    if (g == 0) lb[iq] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : ninf;
  }
}


// Small problems, where there are too few 128-row query tiles to occupy the
// chip: one workgroup per 32-row query tile, and its four waves split the
// key tiles of the tile's walk (wave w takes tiles w, w + 4, ...).  Each wave
// stages its own K / V tile in its own LDS area and keeps its own online
// softmax state; at the end the four (maximum, sum, output) triples are merged
// through LDS, the same merge as across the chunks of a single wave.
constexpr int kSplitBQ = 32;
// query-major: 32 rows own 32-key tiles, ascending (wave w takes visits w, w + 4, ...)
constexpr WalkShape kSplitWalk{kSplitBQ, kBK, false, false};
constexpr int kSplitMaxTiles = 512;  // 128-row tiles below which the key split is used (2 per CU)

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_split_kernel(FwdF32Args p) {
  using SM = F32Smem<D>;
  constexpr int kDT = D / 32;
  constexpr int kKK = D / 2;
  constexpr int kWaves = kThreads / 64;
  constexpr int kWaveLoads = kBK * D / 4 / 64;  // float4 loads per lane per tensor (a wave loads a tile)
  constexpr int kRedRow = D + 4;                // merge rows: 16-byte aligned, spread over banks
  static_assert(kWaves * 32 * kRedRow + 2 * kWaves * 32 <= kWaves * SM::kStage, "merge area");
  __shared__ __align__(16) float smem[kWaves * SM::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const WorkItem wi = work_item(blockIdx.x, p.B, p.H, p.n_qt, true);
  if (!wi.valid) return;  // padding pair
  const int t = wi.t;
  const int h = wi.h;
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, wi.b, h);
  const int N = sh.n;
  if (t * kSplitBQ >= N) return;  // past the end of a packed sequence
  const DistSet dset = dist_set(sh.lo, sh.hi, p.local_window);
  const int lo = dset.lo;
  const int hi = dset.hi;
  const size_t base = sh.row0 * D;
  const float* __restrict__ qb = p.q + base;
  const float* __restrict__ kb = p.k + base;
  const float* __restrict__ vb = p.v + base;
  float* __restrict__ ob = p.o + base;
  float* __restrict__ lb = p.lse + sh.row0;
  const float ninf = -__builtin_inff();

  const int i0 = t * kSplitBQ;
  const int i1 = min(N - 1, i0 + kSplitBQ - 1);
  const TileWalk walk = kernel_walk(kSplitWalk, i0, N, dset);
  if (walk.n == 0) {
    for (int c = tid; c < kSplitBQ * (D / 4); c += kThreads) {
      const int r = c / (D / 4), cc = c % (D / 4);
      if (i0 + r < N) *(f32x4*)(ob + (size_t)(i0 + r) * D + cc * 4) = f32x4{0, 0, 0, 0};
    }
    if (tid < kSplitBQ && i0 + tid < N) lb[i0 + tid] = ninf;
    return;
  }
  const int iq = i0 + c32;

  f32x4 qreg[kKK / 4];  // features g * D/2 .. g * D/2 + D/2 - 1 of row iq
#pragma unroll
  for (int c = 0; c < kKK / 4; ++c)
    qreg[c] = iq < N ? *(const f32x4*)(qb + (size_t)iq * D + g * kKK + 4 * c) : f32x4{0, 0, 0, 0};

  float* ks = smem + wave * SM::kStage;
  float* vs = ks + SM::kKStage;
  // One tensor's tile (rows jb .. jb + 31) into this wave's LDS area.
  auto stage = [&](const float* src, float* dst, int row_stride, int jb) {
    f32x4 r4[kWaveLoads];
#pragma unroll
    for (int r = 0; r < kWaveLoads; ++r) {
      const int c = lane + 64 * r;
      const int j = jb + c / (D / 4);
      r4[r] = j < N ? *(const f32x4*)(src + (size_t)j * D + (c % (D / 4)) * 4) : f32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < kWaveLoads; ++r) {
      const int c = lane + 64 * r;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(c / (D / 4)) * row_stride + (c % (D / 4)) * 4 + e] = r4[r][e];
    }
  };
  // Orders this wave's LDS writes before its reads (and reads before the next
  // writes): LDS instructions of one wave complete in order, so only the
  // compiler's ordering has to be pinned.
  auto wave_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m_run = ninf, l_run = 0.f;
  const float sl2 = p.scale_log2;

  for (int v = wave; v < walk.n; v += kWaves) {
    const int jb = walk.at(v) * kBK;
    if (!set_meets(i0, i1, jb, jb + kBK - 1, dset)) continue;
    wave_sync();  // the previous tile's reads are issued before it is overwritten
    stage(kb, ks, SM::kKRow, jb);
    stage(vb, vs, SM::kVRow, jb);
    wave_sync();
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < kKK / 4; ++c) {
      const f32x4 ka = *(const f32x4*)(ks + c32 * SM::kKRow + g * kKK + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc = mfma32_f32(ka[e], qreg[c][e], sacc);
    }
    float x[16];
    const bool full = set_full(i0, i1, jb, jb + kBK - 1, dset);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = jb + 8 * (i >> 2) + 4 * g + (i & 3);
      const int dist = iq - j;
      const bool in = (dist >= lo && dist <= hi) || (dist >= dset.nlo && dist <= dset.nhi);
      x[i] = (full || in) ? sacc[i] * sl2 : ninf;
    }
    float mx = ninf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == ninf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = fast_exp2(x[i] - m_use);
      psum += x[i];
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = 8 * (i >> 2) + 4 * g + (i & 3);
        acc[dt] = mfma32_f32(vs[j * SM::kVRow + 32 * dt + c32], x[i], acc[dt]);
      }
    }
  }

  // ---- merge the four waves' partial results (query row c32 of each)
  __syncthreads();  // every wave is done with its tiles: the LDS becomes the merge area
  float* red_o = smem;                             // [wave][row][kRedRow]
  float* red_m = smem + kWaves * 32 * kRedRow;     // [wave][row]
  float* red_l = red_m + kWaves * 32;              // [wave][row]
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      red_o[(wave * 32 + c32) * kRedRow + 32 * dt + 8 * (i >> 2) + 4 * g + (i & 3)] = acc[dt][i];
  const float l_w = l_run + __shfl_xor(l_run, 32);
  if (g == 0) {
    red_m[wave * 32 + c32] = m_run;
    red_l[wave * 32 + c32] = l_w;
  }
  __syncthreads();
  for (int c = tid; c < kSplitBQ * (D / 4); c += kThreads) {
    const int r = c / (D / 4), col = c % (D / 4);
    const int i = i0 + r;
    if (i >= N) continue;
    float M = ninf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w * 32 + r]);
    float L = 0.f;
    f32x4 o4{0, 0, 0, 0};
    if (M != ninf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = red_m[w * 32 + r];
        const float f = mw == ninf ? 0.f : fast_exp2(mw - M);
        L += red_l[w * 32 + r] * f;
        const f32x4 pw = *(const f32x4*)&red_o[(w * 32 + r) * kRedRow + 4 * col];
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] += pw[e] * f;
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) o4[e] *= inv;
    *(f32x4*)(ob + (size_t)i * D + 4 * col) = o4;
    if (col == 0) lb[i] = L > 0.f ? (M + fast_log2(L)) * kLn2 : ninf;
  }
}

}  // namespace

int launch_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, const Bands& bands, int local_window, float scale, const Packed& pk,
                   hipStream_t stream) {
  FwdF32Args a;
  a.q = (const float*)q;
  a.k = (const float*)k;
  a.v = (const float*)v;
  a.o = (float*)o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  const bool split = (long long)B * H * ((N + 127) / 128) < kSplitMaxTiles;
  a.n_qt = split ? (N + kSplitBQ - 1) / kSplitBQ : (N + kBQ - 1) / kBQ;
  a.cu = pk.cu;
  a.T = pk.T;
  a.own_bdp = pk.own_bdp;
  a.local_window = local_window;
  a.scale_log2 = scale * kLog2e;
  a.bands = bands;
  const long long total = work_grid(B, H, a.n_qt);
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  dim3 grid((unsigned)total), block(split ? kThreads : kFwdThreads);
  if (d == 128 && split)
    hipLaunchKernelGGL(fwd_f32_split_kernel<128>, grid, block, 0, stream, a);
  else if (d == 64 && split)
    hipLaunchKernelGGL(fwd_f32_split_kernel<64>, grid, block, 0, stream, a);
  else if (d == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, a);
  else if (d == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, a);
  else
    return SPATTN_E_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

void fwd_f32_tiles(int* BQ, int* BK) {
  *BQ = kBQ;
  *BK = kBK;
}

// The walk of the float32 forward launch for B * H sequences of N rows (the
// key-split kernel below 512 tiles of 128 rows, as launch_fwd_f32 decides).
WalkShape fwd_f32_walk(int B, int H, int N) {
  const bool split = (long long)B * H * ((N + 127) / 128) < kSplitMaxTiles;
  return split ? kSplitWalk : kWalk;
}

}  // namespace spattn
