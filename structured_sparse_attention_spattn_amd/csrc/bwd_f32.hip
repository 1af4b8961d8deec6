// Backward of band-partitioned attention in float32 throughout, on gfx950
// fp32 MFMA (v_mfma_f32_32x32x2_f32: full float32 products).  The same
// derivative as the bfloat16 kernels (the textbook derivative of the
// masked-set softmax of "Sparse Attention, Then and Now" section 1 over the
// distance bands of "Making Every Head Count" Figure 1):
//     dP = dO V^T,  dS = P * (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
// with P recomputed from the saved natural-log LSE.  The dQ kernels form
// D_i = dO_i . O_i for their own rows and store -D_i in the workspace for the
// dK/dV kernels.
//
// With a k-depth of 2 per product every operand is a single float, so both
// orientations of a staged tile come straight from LDS: a lane reads along a
// row (k-slot = feature) for S and dP, and down a column (k-slot = row of the
// tile) for the products that contract over rows.  No transposes.  In S and
// dP, product kk takes feature kk in lanes 0-31 and feature D/2 + kk in lanes
// 32-63, so that a lane's operands for four consecutive products are four
// consecutive floats of one row: one 16-byte LDS read per four products.
//
//   bwd_f32_dq_kernel    workgroup = (b, h, 32*W query rows), W waves of 32
//                        rows; the 32-row K/V tiles of the band strip are
//                        staged in LDS (double buffered) and shared by the
//                        waves.  Per tile: S^T = K Q^T, dP^T = V dO^T,
//                        dQ^T += K^T dS^T.
//   bwd_f32_dkdv_kernel  workgroup = (b, h, 32*W key rows); 32-row Q/dO tiles
//                        with their -LSE*log2(e) and -D staged in LDS.  Per
//                        tile: S = Q K^T, dP = dO V^T, dV^T += dO^T P,
//                        dK^T += Q^T dS.
// W = 2: a workgroup's tile walk covers the band strips of all its waves,
// and each wave idles (at the tile barrier) on the tiles outside its own
// strip, so wider workgroups waste more; two waves per workgroup measured
// faster than four at every size.  Every gradient row is written once, by the
// wave that owns it: no atomics, deterministic results.  At d = 128 the operand
// rows and accumulators take about 390-430 registers, one wave per SIMD; at
// d = 64 both kernels are held to 256 for two waves per SIMD.
//
//   bwd_f32_*_split_kernel  small launches (too few 64-row tiles to occupy
//                        the chip): one workgroup per 32-row tile, its four
//                        waves splitting the tile walk, partial gradients
//                        added through LDS.
#include "common.h"

namespace spattn {
namespace {

constexpr int kT = 32;  // a wave's own rows, and the rows of a staged tile
constexpr int kW = 2;   // waves per workgroup
// Walks: a workgroup of w waves owns w * 32 rows and visits 32-row tiles of the
// other operand, ascending (the split kernels: w = 1, visits dealt over waves).
__host__ __device__ constexpr WalkShape dq_walk(int w) { return WalkShape{kT * w, kT, false, false}; }
__host__ __device__ constexpr WalkShape dkdv_walk(int w) { return WalkShape{kT * w, kT, true, false}; }

struct F32BwdArgs {
  const float* q;
  const float* k;
  const float* v;
  const float* dout;
  const float* o;  // dQ kernels only
  const float* lse;
  float* dvec;  // -D_i: written by the dQ kernels, read by the dK/dV kernels
  float* dq;
  float* dk;
  float* dv;
  int B, H, N;       // sequences (B), heads, tokens per sequence (the longest, when packed)
  int n_tiles;       // row tiles per (sequence, head): 32 * kW rows, or 32 for the split kernels
  int local_window;  // shared local window width (0: exclusive bands)
  float scale;
  float scale_log2;
  const int32_t* cu;  // packed sequence offsets [B + 1] (device), or null
  int T;              // packed: tokens per head
  int own_bdp;        // packed: each sequence's own BDP bands
  Bands bands;
};

// Staged tile rows: stride D + 4 keeps rows 16-byte aligned and puts the
// 16-byte row reads of 16 consecutive lanes on distinct banks; the
// column-wise reads (rows 4 apart per half-wave) meet at most two-way.
template <int D>
constexpr int kRow = D + 4;

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row of the 32x32 accumulator held in register r of a lane in half g.
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// -D_i = -(dO_i . O_i) for the row a lane pair holds: each half-wave has
// features g * D/2 .. g * D/2 + D/2 - 1 of dO in registers and reads the same
// features of O; the two halves are added across lanes l and l ^ 32.
template <int D>
__device__ __forceinline__ float neg_d(const float* __restrict__ orow, const f32x4* dreg, bool ok) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const f32x4 o4 = ok ? *(const f32x4*)(orow + 4 * c) : f32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) s += o4[e] * dreg[c][e];
  }
  return -(s + __shfl_xor(s, 32));
}

// Nothing is scheduled across this point.
__device__ __forceinline__ void fence_sched() { __builtin_amdgcn_sched_barrier(0); }

// Row-wise products: acc1 += A1 B1^T, acc2 += A2 B2^T over D features, with
// A1, A2 the rows c32 of two staged tiles (this half-wave's D/2 features) and
// B1, B2 the lane's own operand rows in registers.  The 16-byte operand reads
// run two groups of four products ahead, fenced so that the compiler keeps
// the distance (measured neutral against its own order, which issues each
// read just before its products).
template <int D>
__device__ __forceinline__ void row_products(const float* a1, const float* a2, const f32x4* b1, const f32x4* b2,
                                             f32x16& acc1, f32x16& acc2) {
  constexpr int kC = D / 8;  // groups of four products
  f32x4 x1[kC], x2[kC];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    x1[c] = *(const f32x4*)(a1 + 4 * c);
    x2[c] = *(const f32x4*)(a2 + 4 * c);
  }
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    if (c + 2 < kC) {
      x1[c + 2] = *(const f32x4*)(a1 + 4 * (c + 2));
      x2[c + 2] = *(const f32x4*)(a2 + 4 * (c + 2));
    }
    fence_sched();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc1 = mfma32_f32(x1[c][e], b1[c][e], acc1);
      acc2 = mfma32_f32(x2[c][e], b2[c][e], acc2);
    }
    fence_sched();
  }
}

// Rows [r0, r0 + 32) of one [rows, D] float tensor, through registers into an
// LDS tile of stride kRow<D>; rows past n read as zero.
template <int D, int THR>
struct OneTile {
  static constexpr int kLoads = kT * D / 4 / THR;  // float4 per thread
  f32x4 a[kLoads];
  __device__ __forceinline__ void load(const float* __restrict__ src, int r0, int n, int tid) {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + THR * r;
      const int row = r0 + c / (D / 4), col = c % (D / 4);
      a[r] = row < n ? *(const f32x4*)(src + (size_t)row * D + col * 4) : f32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(float* dst, int tid) const {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + THR * r;
      const int row = c / (D / 4), col = c % (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[row * kRow<D> + col * 4 + e] = a[r][e];
    }
  }
};

// The same for two tensors at once.
template <int D, int THR>
struct PairTile {
  static constexpr int kLoads = kT * D / 4 / THR;  // float4 per thread per tensor
  f32x4 a[kLoads], b[kLoads];
  __device__ __forceinline__ void load(const float* __restrict__ sa, const float* __restrict__ sb, int r0, int n,
                                       int tid) {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + THR * r;
      const int row = r0 + c / (D / 4), col = c % (D / 4);
      const bool ok = row < n;
      a[r] = ok ? *(const f32x4*)(sa + (size_t)row * D + col * 4) : f32x4{0, 0, 0, 0};
      b[r] = ok ? *(const f32x4*)(sb + (size_t)row * D + col * 4) : f32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(float* ta, float* tb, int tid) const {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int c = tid + THR * r;
      const int row = c / (D / 4), col = c % (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ta[row * kRow<D> + col * 4 + e] = a[r][e];
        tb[row * kRow<D> + col * 4 + e] = b[r][e];
      }
    }
  }
};

// Writes a wave's 32 x D accumulator (transposed: register rows are features,
// lanes are rows of the output) times mul to rows row0 + c32 of dst.
template <int D>
__device__ __forceinline__ void store_rows(float* __restrict__ dst, const f32x16* acc, float mul, int row, bool ok,
                                           int g) {
  if (!ok) return;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 w;
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = acc[dt][4 * a + c] * mul;
      *(f32x4*)(dst + (size_t)row * D + 32 * dt + 8 * a + 4 * g) = w;
    }
}

// ------------------------------------------------------------ dQ (query-major)
template <int D, int W>
__global__ __launch_bounds__(64 * W, D == 64 ? 2 : 1) void bwd_f32_dq_kernel(F32BwdArgs p) {
  constexpr int kThr = 64 * W;
  constexpr int kKK = D / 2;
  constexpr int kDT = D / 32;
  constexpr int kTensor = kT * kRow<D>;
  constexpr int kStage = 2 * kTensor;  // K tile, then V tile
  __shared__ __align__(16) float smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const WorkItem wi = work_item(blockIdx.x, p.B, p.H, p.n_tiles, true);
  if (!wi.valid) return;  // padding pair
  const int t = wi.t;
  const int h = wi.h;
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, wi.b, h);
  const int N = sh.n;
  const int i0 = t * kT * W;
  if (i0 >= N) return;  // past the end of a packed sequence
  const int i1 = min(N - 1, i0 + kT * W - 1);
  const DistSet dset = dist_set(sh.lo, sh.hi, p.local_window);
  const size_t base = sh.row0 * D;
  const float* __restrict__ kb = p.k + base;
  const float* __restrict__ vb = p.v + base;

  const TileWalk walk = kernel_walk(dq_walk(W), i0, N, dset);

  const int iw0 = i0 + kT * wave;
  const int iw1 = min(N - 1, iw0 + kT - 1);
  const bool live = iw0 < N;
  const int iq = iw0 + c32;
  const bool row_ok = iq < N;

  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) acc[dt] = zero16();

  f32x4 qreg[kKK / 4], dreg[kKK / 4];  // features g * D/2 .. g * D/2 + D/2 - 1 of row iq
#pragma unroll
  for (int c = 0; c < kKK / 4; ++c)
    dreg[c] = row_ok ? *(const f32x4*)(p.dout + base + (size_t)iq * D + g * kKK + 4 * c) : f32x4{0, 0, 0, 0};
  // -D of every row, keys or not: the dK/dV kernel reads it for all rows of
  // its query tiles
  const float nd = neg_d<D>(p.o + base + (size_t)iq * D + g * kKK, dreg, row_ok);
  if (row_ok && g == 0) p.dvec[sh.row0 + iq] = nd;

  if (walk.n > 0) {
#pragma unroll
    for (int c = 0; c < kKK / 4; ++c)
      qreg[c] = row_ok ? *(const f32x4*)(p.q + base + (size_t)iq * D + g * kKK + 4 * c) : f32x4{0, 0, 0, 0};
    // P = exp2(s * scale * log2(e) - LSE * log2(e)); rows past N use 0 (their
    // results are never stored).
    const float nl2 = row_ok ? -p.lse[sh.row0 + iq] * kLog2e : 0.f;
    const float sl2 = p.scale_log2;

    PairTile<D, kThr> st;
    st.load(kb, vb, walk.at(0) * kT, N, tid);
    st.store(smem, smem + kTensor, tid);
    __syncthreads();

    for (int v = 0; v < walk.n; ++v) {
      const int s = v & 1;
      const bool has_next = v + 1 < walk.n;
      if (has_next) st.load(kb, vb, walk.at(v + 1) * kT, N, tid);
      const float* ks = smem + s * kStage;
      const float* vs = ks + kTensor;
      const int jb = walk.at(v) * kT;
      if (live && set_meets(iw0, iw1, jb, jb + kT - 1, dset)) {
        // S^T and dP^T: rows = the tile's keys, columns = this wave's queries
        f32x16 sacc = zero16(), pacc = zero16();
        row_products<D>(ks + c32 * kRow<D> + g * kKK, vs + c32 * kRow<D> + g * kKK, qreg, dreg, sacc, pacc);
        const bool full = set_full(iw0, iw1, jb, jb + kT - 1, dset);
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dist = iq - (jb + acc_row(r, g));
          const bool in = full || (dist >= dset.lo && dist <= dset.hi) || (dist >= dset.nlo && dist <= dset.nhi);
          const float pr = in ? fast_exp2(__builtin_fmaf(sacc[r], sl2, nl2)) : 0.f;
          ds[r] = pr * (pacc[r] + nd);
        }
        // dQ^T += K^T dS^T: k-slot g of product r is key acc_row(r, g)
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt)
            acc[dt] = mfma32_f32(ks[acc_row(r, g) * kRow<D> + 32 * dt + c32], ds[r], acc[dt]);
      }
      if (has_next) st.store(smem + (s ^ 1) * kStage, smem + (s ^ 1) * kStage + kTensor, tid);
      __syncthreads();
    }
  }
  store_rows<D>(p.dq + base, acc, p.scale, iq, row_ok, g);
}

// ------------------------------------------------------------ dK, dV (key-major)
template <int D, int W>
__global__ __launch_bounds__(64 * W, D == 64 ? 2 : 1) void bwd_f32_dkdv_kernel(F32BwdArgs p) {
  constexpr int kThr = 64 * W;
  constexpr int kKK = D / 2;
  constexpr int kDT = D / 32;
  constexpr int kTensor = kT * kRow<D>;
  constexpr int kStage = 2 * kTensor + 2 * kT;  // Q tile, dO tile, -LSE*log2(e), -D
  __shared__ __align__(16) float smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const WorkItem wi = work_item(blockIdx.x, p.B, p.H, p.n_tiles, false);
  if (!wi.valid) return;  // padding pair
  const int t = wi.t;
  const int h = wi.h;
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, wi.b, h);
  const int N = sh.n;
  const int j0 = t * kT * W;
  if (j0 >= N) return;  // past the end of a packed sequence
  const int j1 = min(N - 1, j0 + kT * W - 1);
  const DistSet dset = dist_set(sh.lo, sh.hi, p.local_window);
  const size_t base = sh.row0 * D;
  const float* __restrict__ qb = p.q + base;
  const float* __restrict__ db = p.dout + base;
  const float* __restrict__ lb = p.lse + sh.row0;
  const float* __restrict__ nb = p.dvec + sh.row0;

  const TileWalk walk = kernel_walk(dkdv_walk(W), j0, N, dset);

  const int jw0 = j0 + kT * wave;
  const int jw1 = min(N - 1, jw0 + kT - 1);
  const bool live = jw0 < N;
  const int jk = jw0 + c32;
  const bool row_ok = jk < N;

  f32x16 dk[kDT], dv[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  if (walk.n > 0) {
    f32x4 kreg[kKK / 4], vreg[kKK / 4];  // features g * D/2 .. g * D/2 + D/2 - 1 of row jk
#pragma unroll
    for (int c = 0; c < kKK / 4; ++c) {
      const size_t at = base + (size_t)jk * D + g * kKK + 4 * c;
      kreg[c] = row_ok ? *(const f32x4*)(p.k + at) : f32x4{0, 0, 0, 0};
      vreg[c] = row_ok ? *(const f32x4*)(p.v + at) : f32x4{0, 0, 0, 0};
    }
    const float sl2 = p.scale_log2;

    // The next tile is staged in two halves, each through its own registers:
    // its Q rows and (threads < 32) one row's -LSE*log2(e) and -D while S and
    // dP are formed, its dO rows while dV and dK are.  Rows past N get
    // P = exp2(-inf) = 0 and -D = 0.
    OneTile<D, kThr> st;
    float nl_r = 0.f, nd_r = 0.f;
    auto load_q = [&](int ib) {
      st.load(qb, ib, N, tid);
      if (tid < kT) {
        const int i = ib + tid;
        nl_r = i < N ? -lb[i] * kLog2e : -__builtin_inff();
        nd_r = i < N ? nb[i] : 0.f;
      }
    };
    auto store_q = [&](int s) {
      float* qs = smem + s * kStage;
      st.store(qs, tid);
      if (tid < kT) {
        qs[2 * kTensor + tid] = nl_r;
        qs[2 * kTensor + kT + tid] = nd_r;
      }
    };
    load_q(walk.at(0) * kT);
    store_q(0);
    st.load(db, walk.at(0) * kT, N, tid);
    st.store(smem + kTensor, tid);
    __syncthreads();

    for (int v = 0; v < walk.n; ++v) {
      const int s = v & 1;
      const bool has_next = v + 1 < walk.n;
      const int inext = has_next ? walk.at(v + 1) * kT : 0;
      if (has_next) load_q(inext);
      const float* qs = smem + s * kStage;
      const float* dos = qs + kTensor;
      const float* nls = qs + 2 * kTensor;
      const float* nds = nls + kT;
      const int ib = walk.at(v) * kT;
      const int ie = min(N - 1, ib + kT - 1);
      if (live && set_meets(ib, ie, jw0, jw1, dset)) {
        // S and dP: rows = the tile's queries, columns = this wave's keys
        f32x16 sacc = zero16(), pacc = zero16();
        row_products<D>(qs + c32 * kRow<D> + g * kKK, dos + c32 * kRow<D> + g * kKK, kreg, vreg, sacc, pacc);
        if (has_next) {
          store_q(s ^ 1);
          st.load(db, inext, N, tid);
        }
        const bool full = set_full(ib, ie, jw0, jw1, dset);
        float pr[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = acc_row(r, g);
          const int dist = ib + il - jk;
          const bool in = full || (ib + il < N && ((dist >= dset.lo && dist <= dset.hi) ||
                                                   (dist >= dset.nlo && dist <= dset.nhi)));
          pr[r] = in ? fast_exp2(__builtin_fmaf(sacc[r], sl2, nls[il])) : 0.f;
          ds[r] = pr[r] * (pacc[r] + nds[il]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS: k-slot g of product r is query acc_row(r, g)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = acc_row(r, g);
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt) {
            dv[dt] = mfma32_f32(dos[il * kRow<D> + 32 * dt + c32], pr[r], dv[dt]);
            dk[dt] = mfma32_f32(qs[il * kRow<D> + 32 * dt + c32], ds[r], dk[dt]);
          }
        }
      } else if (has_next) {
        store_q(s ^ 1);
        st.load(db, inext, N, tid);
      }
      if (has_next) st.store(smem + (s ^ 1) * kStage + kTensor, tid);
      __syncthreads();
    }
  }
  store_rows<D>(p.dk + base, dk, p.scale, jk, row_ok, g);
  store_rows<D>(p.dv + base, dv, 1.f, jk, row_ok, g);
}

// ------------------------------------------------------------ small launches
// Too few 64-row tiles to occupy the chip: one workgroup per 32-row tile, and
// its four waves split the tile's walk (wave w takes visits w, w + 4, ...),
// each staging its own tiles in its own LDS area.  The partial gradients are
// plain sums over the visited tiles, so the four are added through LDS in
// wave order (deterministic) and the workgroup writes the rows once.
constexpr int kSplitWaves = 4;
constexpr int kSplitMaxTiles = 512;  // 64-row tiles below which the walk is split

// Orders this wave's LDS accesses around a rewrite of its own area: LDS
// instructions of one wave complete in order, so only the compiler's
// ordering has to be pinned.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Rows [r0, r0 + 32) of a [rows, D] float tensor into an LDS tile of stride
// kRow<D>, by the 64 lanes of one wave; rows past n are zero.
template <int D>
__device__ __forceinline__ void wave_stage(const float* __restrict__ src, float* dst, int r0, int n, int lane) {
#pragma unroll
  for (int r = 0; r < kT * D / 4 / 64; ++r) {
    const int c = lane + 64 * r;
    const int row = c / (D / 4), col = c % (D / 4);
    const f32x4 x = r0 + row < n ? *(const f32x4*)(src + (size_t)(r0 + row) * D + col * 4) : f32x4{0, 0, 0, 0};
    *(f32x4*)(dst + row * kRow<D> + col * 4) = x;
  }
}

// Sum of the four waves' 32 x D accumulators (transposed as in store_rows)
// times mul, written to rows row0 .. row0 + 31 (< n) of dst.  red holds
// 4 * 32 * kRow<D> floats; the caller has synchronised the workgroup.
template <int D>
__device__ __forceinline__ void merge_rows(float* red, const f32x16* acc, float mul, float* __restrict__ dst,
                                           int row0, int n, int tid) {
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, c32 = lane & 31;
  float* mine = red + wave * kT * kRow<D>;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 w;
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = acc[dt][4 * a + c];
      *(f32x4*)(mine + c32 * kRow<D> + 32 * dt + 8 * a + 4 * g) = w;
    }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kT * D / 4 / (64 * kSplitWaves); ++r) {
    const int c = tid + 64 * kSplitWaves * r;
    const int row = c / (D / 4), col = c % (D / 4);
    f32x4 sum = *(const f32x4*)(red + row * kRow<D> + col * 4);
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) sum += *(const f32x4*)(red + w * kT * kRow<D> + row * kRow<D> + col * 4);
    if (row0 + row < n) *(f32x4*)(dst + (size_t)(row0 + row) * D + col * 4) = sum * mul;
  }
}

template <int D>
__global__ __launch_bounds__(64 * kSplitWaves) void bwd_f32_dq_split_kernel(F32BwdArgs p) {
  constexpr int kKK = D / 2;
  constexpr int kDT = D / 32;
  constexpr int kTensor = kT * kRow<D>;
  constexpr int kArea = 2 * kTensor;  // one wave's K tile, then V tile
  static_assert(kSplitWaves * kT * kRow<D> <= kSplitWaves * kArea, "merge area");
  __shared__ __align__(16) float smem[kSplitWaves * kArea];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const WorkItem wi = work_item(blockIdx.x, p.B, p.H, p.n_tiles, true);
  if (!wi.valid) return;  // padding pair
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, wi.b, wi.h);
  const int N = sh.n;
  const int i0 = wi.t * kT;
  if (i0 >= N) return;  // past the end of a packed sequence
  const int i1 = min(N - 1, i0 + kT - 1);
  const DistSet dset = dist_set(sh.lo, sh.hi, p.local_window);
  const size_t base = sh.row0 * D;

  const TileWalk walk = kernel_walk(dq_walk(1), i0, N, dset);

  const int iq = i0 + c32;
  const bool row_ok = iq < N;
  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) acc[dt] = zero16();

  f32x4 qreg[kKK / 4], dreg[kKK / 4];
#pragma unroll
  for (int c = 0; c < kKK / 4; ++c)
    dreg[c] = row_ok ? *(const f32x4*)(p.dout + base + (size_t)iq * D + g * kKK + 4 * c) : f32x4{0, 0, 0, 0};
  // -D of every row, keys or not (wave 0 stores it for the dK/dV kernel)
  const float nd = neg_d<D>(p.o + base + (size_t)iq * D + g * kKK, dreg, row_ok);
  if (wave == 0 && row_ok && g == 0) p.dvec[sh.row0 + iq] = nd;

  if (walk.n > wave) {
#pragma unroll
    for (int c = 0; c < kKK / 4; ++c)
      qreg[c] = row_ok ? *(const f32x4*)(p.q + base + (size_t)iq * D + g * kKK + 4 * c) : f32x4{0, 0, 0, 0};
    const float nl2 = row_ok ? -p.lse[sh.row0 + iq] * kLog2e : 0.f;
    const float sl2 = p.scale_log2;
    float* ks = smem + wave * kArea;
    float* vs = ks + kTensor;
    for (int v = wave; v < walk.n; v += kSplitWaves) {
      const int jb = walk.at(v) * kT;
      wave_sync();
      wave_stage<D>(p.k + base, ks, jb, N, lane);
      wave_stage<D>(p.v + base, vs, jb, N, lane);
      wave_sync();
      if (!set_meets(i0, i1, jb, jb + kT - 1, dset)) continue;
      f32x16 sacc = zero16(), pacc = zero16();
      row_products<D>(ks + c32 * kRow<D> + g * kKK, vs + c32 * kRow<D> + g * kKK, qreg, dreg, sacc, pacc);
      const bool full = set_full(i0, i1, jb, jb + kT - 1, dset);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dist = iq - (jb + acc_row(r, g));
        const bool in = full || (dist >= dset.lo && dist <= dset.hi) || (dist >= dset.nlo && dist <= dset.nhi);
        const float pr = in ? fast_exp2(__builtin_fmaf(sacc[r], sl2, nl2)) : 0.f;
        ds[r] = pr * (pacc[r] + nd);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
          acc[dt] = mfma32_f32(ks[acc_row(r, g) * kRow<D> + 32 * dt + c32], ds[r], acc[dt]);
    }
  }
  __syncthreads();  // every wave is done with its tile area
  merge_rows<D>(smem, acc, p.scale, p.dq + base, i0, N, tid);
}

template <int D>
__global__ __launch_bounds__(64 * kSplitWaves) void bwd_f32_dkdv_split_kernel(F32BwdArgs p) {
  constexpr int kKK = D / 2;
  constexpr int kDT = D / 32;
  constexpr int kTensor = kT * kRow<D>;
  constexpr int kArea = 2 * kTensor + 2 * kT;  // one wave's Q tile, dO tile, -LSE*log2(e), -D
  static_assert(kSplitWaves * kT * kRow<D> <= kSplitWaves * kArea, "merge area");
  __shared__ __align__(16) float smem[kSplitWaves * kArea];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const WorkItem wi = work_item(blockIdx.x, p.B, p.H, p.n_tiles, false);
  if (!wi.valid) return;  // padding pair
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, wi.b, wi.h);
  const int N = sh.n;
  const int j0 = wi.t * kT;
  if (j0 >= N) return;  // past the end of a packed sequence
  const int j1 = min(N - 1, j0 + kT - 1);
  const DistSet dset = dist_set(sh.lo, sh.hi, p.local_window);
  const size_t base = sh.row0 * D;
  const float* __restrict__ lb = p.lse + sh.row0;
  const float* __restrict__ nb = p.dvec + sh.row0;

  const TileWalk walk = kernel_walk(dkdv_walk(1), j0, N, dset);

  const int jk = j0 + c32;
  const bool row_ok = jk < N;
  f32x16 dk[kDT], dv[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  if (walk.n > wave) {
    f32x4 kreg[kKK / 4], vreg[kKK / 4];
#pragma unroll
    for (int c = 0; c < kKK / 4; ++c) {
      const size_t at = base + (size_t)jk * D + g * kKK + 4 * c;
      kreg[c] = row_ok ? *(const f32x4*)(p.k + at) : f32x4{0, 0, 0, 0};
      vreg[c] = row_ok ? *(const f32x4*)(p.v + at) : f32x4{0, 0, 0, 0};
    }
    const float sl2 = p.scale_log2;
    float* qs = smem + wave * kArea;
    float* dos = qs + kTensor;
    float* nls = qs + 2 * kTensor;
    float* nds = nls + kT;
    for (int v = wave; v < walk.n; v += kSplitWaves) {
      const int ib = walk.at(v) * kT;
      const int ie = min(N - 1, ib + kT - 1);
      wave_sync();
      wave_stage<D>(p.q + base, qs, ib, N, lane);
      wave_stage<D>(p.dout + base, dos, ib, N, lane);
      if (lane < kT) {
        const int i = ib + lane;
        nls[lane] = i < N ? -lb[i] * kLog2e : -__builtin_inff();
        nds[lane] = i < N ? nb[i] : 0.f;
      }
      wave_sync();
      if (!set_meets(ib, ie, j0, j1, dset)) continue;
      f32x16 sacc = zero16(), pacc = zero16();
      row_products<D>(qs + c32 * kRow<D> + g * kKK, dos + c32 * kRow<D> + g * kKK, kreg, vreg, sacc, pacc);
      const bool full = set_full(ib, ie, j0, j1, dset);
      float pr[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = acc_row(r, g);
        const int dist = ib + il - jk;
        const bool in = full || (ib + il < N && ((dist >= dset.lo && dist <= dset.hi) ||
                                                 (dist >= dset.nlo && dist <= dset.nhi)));
        pr[r] = in ? fast_exp2(__builtin_fmaf(sacc[r], sl2, nls[il])) : 0.f;
        ds[r] = pr[r] * (pacc[r] + nds[il]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = acc_row(r, g);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          dv[dt] = mfma32_f32(dos[il * kRow<D> + 32 * dt + c32], pr[r], dv[dt]);
          dk[dt] = mfma32_f32(qs[il * kRow<D> + 32 * dt + c32], ds[r], dk[dt]);
        }
      }
    }
  }
  __syncthreads();  // every wave is done with its tile area
  merge_rows<D>(smem, dk, p.scale, p.dk + base, j0, N, tid);
  __syncthreads();  // the merge area is rewritten
  merge_rows<D>(smem, dv, 1.f, p.dv + base, j0, N, tid);
}

F32BwdArgs make_f32_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, const Bands& bands,
                         int local_window, float scale, float* dvec, const Packed& pk, int rows_per_tile) {
  F32BwdArgs a;
  a.q = (const float*)q;
  a.k = (const float*)k;
  a.v = (const float*)v;
  a.o = (const float*)o;
  a.dout = (const float*)dout;
  a.lse = lse;
  a.dvec = dvec;
  a.dq = (float*)dq;
  a.dk = (float*)dk;
  a.dv = (float*)dv;
  a.B = B;
  a.H = H;
  a.N = N;
  a.n_tiles = (N + rows_per_tile - 1) / rows_per_tile;
  a.local_window = local_window;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.cu = pk.cu;
  a.T = pk.T;
  a.own_bdp = pk.own_bdp;
  a.bands = bands;
  return a;
}


// the walk-splitting kernels when the 64-row tiles would not occupy the chip
bool split_launch(int B, int H, int N) {
  return (long long)B * H * ((N + kW * kT - 1) / (kW * kT)) < kSplitMaxTiles;
}

}  // namespace

// The walks the float32 backward launches for B * H sequences of N rows use.
WalkShape bwd_f32_dq_walk(int B, int H, int N) { return dq_walk(split_launch(B, H, N) ? 1 : kW); }
WalkShape bwd_f32_dkdv_walk(int B, int H, int N) { return dkdv_walk(split_launch(B, H, N) ? 1 : kW); }

int launch_bwd_dq_f32(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                      void* dq, int B, int H, int N, int d, const Bands& bands, int local_window, float scale,
                      float* dvec, const Packed& pk, hipStream_t stream) {
  const bool split = split_launch(B, H, N);
  F32BwdArgs a = make_f32_args(q, k, v, o, lse, dout, dq, nullptr, nullptr, B, H, N, bands, local_window, scale,
                               dvec, pk, split ? kT : kW * kT);
  const long long total = work_grid(B, H, a.n_tiles);
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  const dim3 grid((unsigned)total), block(64 * kW);
  if (split) {
    if (d == 128)
      hipLaunchKernelGGL(bwd_f32_dq_split_kernel<128>, grid, dim3(64 * kSplitWaves), 0, stream, a);
    else
      hipLaunchKernelGGL(bwd_f32_dq_split_kernel<64>, grid, dim3(64 * kSplitWaves), 0, stream, a);
  } else if (d == 128)
    hipLaunchKernelGGL((bwd_f32_dq_kernel<128, kW>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_f32_dq_kernel<64, kW>), grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

int launch_bwd_dkdv_f32(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                        void* dv, int B, int H, int N, int d, const Bands& bands, int local_window, float scale,
                        float* dvec, const Packed& pk, hipStream_t stream) {
  const bool split = split_launch(B, H, N);
  F32BwdArgs a = make_f32_args(q, k, v, nullptr, lse, dout, nullptr, dk, dv, B, H, N, bands, local_window,
                               scale, dvec, pk, split ? kT : kW * kT);
  const long long total = work_grid(B, H, a.n_tiles);
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  const dim3 grid((unsigned)total), block(64 * kW);
  if (split) {
    if (d == 128)
      hipLaunchKernelGGL(bwd_f32_dkdv_split_kernel<128>, grid, dim3(64 * kSplitWaves), 0, stream, a);
    else
      hipLaunchKernelGGL(bwd_f32_dkdv_split_kernel<64>, grid, dim3(64 * kSplitWaves), 0, stream, a);
  } else if (d == 128)
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<128, kW>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<64, kW>), grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

}  // namespace spattn
