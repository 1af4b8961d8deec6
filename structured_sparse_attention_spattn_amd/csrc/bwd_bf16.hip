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
//             of 32 rows.  Computes D for its rows (-D and -LSE log2(e) are
//             written for the second kernel), then walks the 32-key tiles of
//             its band strip:
//             S^T = K Q^T, dP^T = V dO^T, dS^T, and dQ^T += K^T dS^T (K^T is
//             read from the row-major K tile with the LDS transpose read).
//   bwd_dkdv  key-major, one workgroup per (b, h, 64 key rows), 4 waves in
//             2 pairs of 32 keys.  Walks the 32-row query blocks that reach its
//             keys: S = Q K^T and dV += P^T dO in one wave of a pair, dP = dO V^T,
//             dS and dK += dS^T Q in the other, dK / dV held in registers for
//             the whole walk (dO and Q enter the last two products through the
//             LDS transpose read).  When the two pairs' query blocks are offset
//             by one, the second pair runs a block ahead (stepped schedule).
// Both recompute P from the saved LSE with the same band-tile enumeration as
// the forward pass and mask element-wise only on tiles that are not FULL.
#include "common.h"

namespace spattn {
namespace {

constexpr int kZeroGroup = 4;  // query tiles without keys zeroed by one dQ workgroup

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  float* dvec;  // -D_i = -dO_i . O_i: written by bwd_dq, read by bwd_dkdv
  float* nl2;   // -LSE_i * log2(e): written by bwd_dq, read by bwd_dkdv
  void* dq;
  void* dk;
  void* dv;
  int grad_f32;
  int B, H, N;
  int n_tiles;  // query tiles (bwd_dq) or key tiles (bwd_dkdv) per (b, h)
  const int32_t* cu;  // packed sequence offsets [B + 1] (device), or null
  int T;              // packed: tokens per head
  int own_bdp;        // packed: each sequence's own BDP bands
  int local_window;  // shared local window width (0: exclusive bands)
  float scale;
  float scale_log2;
  Bands bands;
};

// =====================================================================  dQ
constexpr int kDqWaves = 4;   // waves per workgroup, 32 query rows each
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqBQ = 32 * kDqWaves;  // query rows per workgroup
constexpr int kDqBK = 32;     // key rows per stage
constexpr int kDqStages = 4;  // LDS ring depth: tiles u+1 .. u+3 load while u is used
constexpr int kDqOcc = 2;     // waves per SIMD the register budget allows
// query-major: the workgroup's rows own 32-key tiles, a single run rotated (align_walk)
constexpr WalkShape kDqWalk{kDqBQ, kDqBK, false, true};

template <int D, bool TWO>
__global__ __launch_bounds__(kDqThreads, kDqOcc) void bwd_dq_kernel(BwdArgs p) {
  constexpr int kTile = kDqBK * D;
  constexpr int kKK = D / 16;
  constexpr int kDT = D / 32;
  using Tile = AsyncTile<kDqBK, D, kDqWaves>;
  constexpr int kL = 2 * Tile::kPer;  // loads per wave per stage
  __shared__ __attribute__((aligned(16))) bf16 smem[kDqStages * 2 * kTile];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const WorkItem wi = work_item(blockIdx.x, p.B, p.H, p.n_tiles, true);
  if (!wi.valid) return;  // padding pair
  const int t = wi.t;
  const int h = wi.h;
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, wi.b, h);
  const int N = sh.n;
  if (t * kDqBQ >= N) return;  // past the end of a packed sequence
  // the head's distance set: its band, joined with the local window if any
  const DistSet dset = dist_set(sh.lo, sh.hi, TWO ? p.local_window : 0);
  const int lo = dset.lo;
  const int hi = dset.hi;
  // Query tiles without keys (a prefix of the tiles) only get zero rows of dQ
  // and of the two row vectors (finite values keep a later dK/dV block that
  // overlaps these rows finite):
  // the first of every kZeroGroup of them writes the group, the others exit.
  {
    const int md = min_dist(dset, N);
    const int tiles = (N + kDqBQ - 1) / kDqBQ;
    const int n_inact = md >= N ? tiles : md / kDqBQ;
    if (t < n_inact) {
      if (t % kZeroGroup != 0) return;
      for (int tt = t; tt < min(t + kZeroGroup, n_inact); ++tt) {
        const int r0 = tt * kDqBQ + 32 * wave;
        if (r0 > N - 1) continue;
        store_zero_rows<D>(p.dq, sh.row0 + r0, min(32, N - r0), p.grad_f32 != 0, lane);
        if (lane < 32 && r0 + lane < N) p.dvec[sh.row0 + r0 + lane] = 0.f;
        if (lane < 32 && r0 + lane < N) p.nl2[sh.row0 + r0 + lane] = 0.f;
      }
      return;
    }
  }
  const size_t base = sh.row0 * D;
  const bf16* __restrict__ kb = p.k + base;
  const bf16* __restrict__ vb = p.v + base;

  const int i_tile0 = t * kDqBQ;
  const int iw0 = i_tile0 + 32 * wave;
  const int iw1 = min(N - 1, iw0 + 31);
  const bool wave_live = iw0 <= N - 1;
  const int iq = iw0 + c32;
  const bool row_ok = iq < N;

  // key tiles to visit, in order; the ring holds visit v in stage v % kDqStages
  const TileWalk walk = kernel_walk(kDqWalk, i_tile0, N, dset);
  const int n_visit = walk.n;
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  auto issue = [&](int v) {
    const uint32_t st = smem_lds + (uint32_t)((v % kDqStages) * 2 * kTile * 2);
    const int u = walk.at(v);
    Tile::load(st, kb, u * kDqBK, N, wave, lane);
    Tile::load(st + 2 * kTile, vb, u * kDqBK, N, wave, lane);
  };
  // Ring prefill first: its round trip overlaps that of the row loads below
  // (the wait for those covers both).
#pragma unroll
  for (int i = 0; i < kDqStages - 1; ++i)
    if (i < n_visit) issue(i);

  // Q and dO operands; D_i = dO_i . O_i from the same lanes.  All row
  // chunks are requested before the first is used, so the prologue costs one
  // memory round trip, not one per chunk.  A tile none of whose rows has a
  // key loads nothing: its D (never used with a nonzero P) and dQ are 0.
  bf16x8 qreg[kKK], doreg[kKK];
  float dval = 0.f, nlse2 = 0.f;  // nlse2: P = exp2(s * sl2 + nlse2), nlse2 = -LSE log2(e)
  if (n_visit > 0) {
    const int ir = min(iq, N - 1);  // rows past N read the last row, then count as zero
    const size_t roff = base + (size_t)ir * D + 8 * g;
    bf16x8 oreg[kKK];
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      qreg[kk] = *(const bf16x8*)(p.q + roff + 16 * kk);
      doreg[kk] = *(const bf16x8*)(p.dout + roff + 16 * kk);
      oreg[kk] = *(const bf16x8*)(p.o + roff + 16 * kk);
    }
    const float lse_i = p.lse[sh.row0 + ir];
    float dpart = 0.f;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart += (float)doreg[kk][e] * (float)oreg[kk][e];
    dpart += __shfl_xor(dpart, 32);  // lanes l and l ^ 32 hold the two halves of one row
    dval = row_ok ? dpart : 0.f;
    nlse2 = row_ok ? -lse_i * kLog2e : 0.f;
    if (!row_ok) {
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) {
        qreg[kk] = bf16x8{};
        doreg[kk] = bf16x8{};
      }
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      qreg[kk] = bf16x8{};
      doreg[kk] = bf16x8{};
    }
  }
  if (row_ok && g == 0) {
    p.dvec[sh.row0 + iq] = -dval;
    p.nl2[sh.row0 + iq] = nlse2;
  }
  const float sl2 = p.scale_log2;
  const float scl = p.scale;
  // -D in every register of a 32 x 32 accumulator: the dP^T chain starts
  // from it (as its first product's C operand), so it ends at dP - D
  f32x16 nd16;
#pragma unroll
  for (int i = 0; i < 16; ++i) nd16[i] = -dval;
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    settle(qreg[kk]);
    settle(doreg[kk]);
  }
  settle(nlse2);
  settle(dval);

  f32x16 acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  if (n_visit > 0) {
    LaneOffsets<D> off(lane);
    for (int v = 0; v < n_visit; ++v) {
      // visits issued after v and possibly in flight
      const int ahead = min(kDqStages - 2, n_visit - 1 - v);
      if (kDqStages >= 4 && ahead >= 2)
        wait_vmcnt<2 * kL>();
      else if (kDqStages >= 3 && ahead >= 1)
        wait_vmcnt<kL>();
      else
        wait_vmcnt<0>();
      __syncthreads();  // tile of visit v complete for everyone; visit v - 1 released
      if (v + kDqStages - 1 < n_visit) issue(v + kDqStages - 1);
      const bf16* ks = smem + (v % kDqStages) * 2 * kTile;
      const bf16* vs = ks + kTile;
      off.refresh();
      const int jb = walk.at(v) * kDqBK;
      bool meets, full;
      if constexpr (TWO) {
        meets = set_meets(iw0, iw1, jb, jb + 31, dset);
        full = set_full(iw0, iw1, jb, jb + 31, dset);
      } else {
        meets = tile_meets(iw0, iw1, jb, jb + 31, lo, hi);
        full = tile_full(iw0, iw1, jb, jb + 31, lo, hi);
      }
      if (wave_live && meets) {
        // S^T first, then dP^T with the exponentials of S^T issued between
        // its products (one accumulator chain each; a dependent chain costs
        // nothing extra when other work sits between its steps).
        bf16x8 opa[kKK];
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) opa[kk] = *(const bf16x8*)((const char*)ks + off.k[kk]);
        __builtin_amdgcn_sched_barrier(0);
        const f32x16 sacc = mfma_ksum<kKK, 1>(opa, qreg);
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) opa[kk] = *(const bf16x8*)((const char*)vs + off.k[kk]);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 pacc = nd16;
        float pe[16];
        // fixed order: one dP^T product, then its share of the exponentials
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) {
          pacc = mfma32(opa[kk], doreg[kk], pacc);
#pragma unroll
          for (int i = kk * 16 / kKK; i < (kk + 1) * 16 / kKK; ++i)
            pe[i] = fast_exp2(__builtin_fmaf(sacc[i], sl2, nlse2));
          __builtin_amdgcn_sched_barrier(0);
        }
        // K^T operands of dQ^T += K^T dS^T, in flight during the dS math
        bf16x8 kt[2 * kDT];
        load_va<D>(kt, ks, off, 0);
        // dS = P (dP - D), the scale applied to dQ once at the store; on a
        // partial tile the band is applied by selection (P may overflow out
        // of band)
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = pe[i] * pacc[i];
        if (!full) {
          const int mb = iq - jb - 8 * g - lo;  // (iq - key - lo) + c for register i
          const uint32_t width = (uint32_t)(hi - lo);
          const int mb2 = iq - jb - 8 * g - dset.nlo;
          const uint32_t width2 = (uint32_t)(dset.nhi - dset.nlo);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int c = ((i >> 3) << 4) + (i & 7);  // perm_reg_row(i, 0)
            bool in = (uint32_t)(mb - c) <= width;
            if constexpr (TWO) in = in || (uint32_t)(mb2 - c) <= width2;
            ds[i] = in && row_ok ? ds[i] : 0.f;
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

  if (n_visit == 0) {  // no keys: zero rows, written directly
    if (wave_live) store_zero_rows<D>(p.dq, sh.row0 + iw0, min(32, N - iw0), p.grad_f32 != 0, lane);
    return;
  }
  __syncthreads();  // every wave is done with the K / V ring: it becomes the output staging area
  if (wave_live) {
    // dQ = scale sum dS K; 32 x 64 floats per wave fit the ring at any depth
    constexpr int kNC = kDqWaves * 32 * D * 4 <= (int)sizeof(smem) ? D : D / 2;
    static_assert(kDqWaves * 32 * kNC * 4 <= (int)sizeof(smem), "output staging fits the K / V ring");
    store_result<D, kNC>((float*)smem + wave * 32 * kNC, acc, scl, p.dq, sh.row0 + iw0, min(32, N - iw0),
                         p.grad_f32 != 0, lane);
  }
}

// =====================================================================  dK dV
// Warp-specialised: 4 waves, 64 keys, two workgroups per CU.  Wave w < 2
// ("P wave") owns keys 32w .. 32w+31 of the tile: S = Q K^T, P -- handed to
// its partner through LDS -- and dV += P^T dO.  Wave w + 2 ("dS wave") owns
// the same keys: dP = dO V^T for the current query block and, one block
// behind, dS = P (dP - D) and dK += dS^T Q with the P its partner handed over
// in the previous iteration.  The lag leaves one barrier per block and no
// wait of one role on the other inside it: P is double-buffered by block
// parity, and the ring keeps the previous block's Q tile until the dS wave
// is done with it (blocks tq - 1 .. tq + 2 occupy the four stages).  Each
// wave keeps a single 32 x d accumulator.
constexpr int kKvBK = 64;     // key rows per workgroup
constexpr int kKvQB = 32;     // query rows per stage
// key-major: 64 key rows own 32-row query blocks, ascending
constexpr WalkShape kKvWalk{kKvBK, kKvQB, true, false};
constexpr int kKvStages = 4;  // LDS ring depth
constexpr int kKvAhead = 2;   // blocks tq + 1 .. tq + kKvAhead in flight while tq is used
constexpr int kKvThreads = 256;
constexpr int kKvPairs = kKvThreads / 128;
static_assert(kKvAhead + 2 <= kKvStages, "ring holds the lagging block, the current one and the prefetched ones");

typedef _Float16 f16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

// Eight values as float16 (round toward zero; P lies in [0, 1]).
__device__ __forceinline__ f16x8 pack8_f16(const float* x) {
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const auto h2 = __builtin_amdgcn_cvt_pkrtz(x[j], x[j + 1]);
    r[j] = h2[0];
    r[j + 1] = h2[1];
  }
  return r;
}

template <int D, bool TWO>
__global__ __launch_bounds__(kKvThreads, 2) void bwd_dkdv_kernel(BwdArgs p) {
  constexpr int kWaves = kKvThreads / 64;
  constexpr int kTile = kKvQB * D;
  constexpr int kKK = D / 16;
  constexpr int kDT = D / 32;
  using Tile = AsyncTile<kKvQB, D, kWaves>;
  constexpr int kL = 2 * Tile::kPer + 1;  // loads per wave per stage (Q, dO, row values)
  __shared__ __attribute__((aligned(16))) bf16 smem[kKvStages * 2 * kTile];  // [stage][Q, dO]
  // [stage][wave][-LSE log2(e) of the 32 rows | -D of the 32 rows]: every
  // wave loads its own copy
  __shared__ __attribute__((aligned(16))) float rowv[kKvStages][kWaves][2 * kKvQB];
  // P from P wave w to dS wave w + kKvPairs, [block parity][pair][half][lane]:
  // each half of a lane's 16 values is one 1 KB contiguous row of 16-byte
  // pieces, so writes and reads are single conflict-free sweeps.
  __shared__ __attribute__((aligned(16))) f16 pbuf[2][kKvPairs][2][64][8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pwave = wave < kKvPairs;
  const int kw = wave % kKvPairs;  // key group shared by the P / dS wave pair
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const WorkItem wi = work_item(blockIdx.x, p.B, p.H, p.n_tiles, false);
  if (!wi.valid) return;  // padding pair
  const int ut = wi.t;
  const int h = wi.h;
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, wi.b, h);
  const int N = sh.n;
  if (ut * kKvBK >= N) return;  // past the end of a packed sequence
  // the head's distance set: its band, joined with the local window if any
  const DistSet dset = dist_set(sh.lo, sh.hi, TWO ? p.local_window : 0);
  const int lo = dset.lo;
  const int hi = dset.hi;
  const size_t base = sh.row0 * D;
  const bf16* __restrict__ qb = p.q + base;
  const bf16* __restrict__ dob = p.dout + base;
  const float* __restrict__ nl2b = p.nl2 + sh.row0;
  const float* __restrict__ ddb = p.dvec + sh.row0;

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

  // query blocks to visit, in order; visit v sits in ring stage v % kKvStages
  const TileWalk walk = kernel_walk(kKvWalk, j0, N, dset);
  const int n_visit = walk.n;
  // Stepped schedule.  The second key pair (keys 32 .. 63 of the tile) never
  // needs the walk's first query block when the first pair never needs its
  // last: the second pair then runs one block ahead of the first and the
  // workgroup takes n_visit - 1 steps instead of n_visit, with no step spent
  // on a block that misses a pair's keys.  Step t: this wave's visit is
  // t + voff; waits, barriers and ring loads follow the step.
  bool shifted = false;
  if (n_visit >= 2 && j0 + 32 <= N - 1 && !(TWO && has_second(dset))) {
    const int a1 = j0 + 31, b0 = j0 + 32, b1 = min(N - 1, j0 + 63);
    const int f0 = walk.at(0) * kKvQB, f1 = min(N - 1, f0 + kKvQB - 1);
    const int l0 = walk.at(n_visit - 1) * kKvQB, l1 = min(N - 1, l0 + kKvQB - 1);
    shifted = !tile_meets(f0, f1, b0, b1, lo, hi) && !tile_meets(l0, l1, j0, a1, lo, hi);
  }
  const int n_step = shifted ? n_visit - 1 : n_visit;
  const int voff = shifted && kw == 1 ? 1 : 0;
  if (n_visit > 0) {
    const float sl2 = p.scale_log2;
    const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));
    const uint32_t rowv_lds = __builtin_amdgcn_readfirstlane(lds_addr(&rowv[0][0][0]));
    auto issue = [&](int v) {
      const int st = v % kKvStages;
      const int tq = walk.at(v);
      const uint32_t t = smem_lds + (uint32_t)(st * 2 * kTile * 2);
      Tile::load(t, qb, tq * kKvQB, N, wave, lane);
      Tile::load(t + 2 * kTile, dob, tq * kKvQB, N, wave, lane);
      const int i = min(tq * kKvQB + (lane & 31), N - 1);
      const float* src = lane < 32 ? nl2b + i : ddb + i;
      lds_dma4(rowv_lds + (uint32_t)((st * kWaves + wave) * 2 * kKvQB * 4), src);
    };
    // Ring prefill first: its round trip overlaps that of the row loads below.
#pragma unroll
    for (int i = 0; i < kKvAhead; ++i)
      if (i < n_visit) issue(i);
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
    // dS wave, visit v (one iteration late): dS = P (dP - D), dP - D coming
    // straight out of the dP chain, and
    // dK^T += Q^T dS (the scale is applied to dK once, at the store).  P comes masked from the P wave (0 outside the band and
    // on rows past N), so no mask is needed here.
    auto ds_dk = [&](int v, const f32x16& dpv) {
      const int st = v % kKvStages;
      const bf16* qs = smem + st * 2 * kTile;
      bf16x8 bb[2 * kDT];
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        bb[2 * dt] = kmajor_operand<D>(qs, 0, 32 * dt, lane);
        bb[2 * dt + 1] = kmajor_operand<D>(qs, 16, 32 * dt, lane);
      }
      float ds[16];
      const f16x8 pa = *(const f16x8*)&pbuf[v & 1][kw][0][lane][0];
      const f16x8 pb = *(const f16x8*)&pbuf[v & 1][kw][1][lane][0];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ds[i] = (float)pa[i] * dpv[i];
        ds[8 + i] = (float)pb[i] * dpv[8 + i];
      }
      const bf16x8 op0 = pack8(&ds[0]), op1 = pack8(&ds[8]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) acc[dt] = mfma32(bb[2 * dt], op0, acc[dt]);
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) acc[dt] = mfma32(bb[2 * dt + 1], op1, acc[dt]);
    };

    // Top of every step t, for both roles (same barrier sequence): wait for
    // this wave's loads of the visits step t uses -- visit t (those of t + 1
    // may stay in flight), or t + 1 on the stepped schedule (nothing in
    // flight) -- then the barrier: those visits complete for everyone, step
    // t - 1 finished everywhere, so the stage of visit t - 2 is free and the
    // P of the previous visit is visible; then visit t + kKvAhead is loaded.
    auto block_start = [&](int t) {
      if (!shifted && t + 1 < n_step)
        wait_vmcnt<kL>();
      else
        wait_vmcnt<0>();
      __syncthreads();
    };
    // The ring loads of visit t + kKvAhead are issued in the middle of a
    // dependent MFMA chain (score or dP), whose stalls absorb their issue cost.
    auto prefetch = [&](int t) {
      if (t + kKvAhead < n_visit) issue(t + kKvAhead);
    };
    // sum over kk of a[kk] x b[kk] as one dependent chain, with the prefetch
    // of step t after the first half of the products
    // init: the accumulator's starting value (0 for S; -D of the block's rows
    // for dP, so the chain ends at dP - D)
    auto chain_with_prefetch = [&](const bf16x8* a, int t, const float* init) {
      f32x16 c;
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = init[i];
#pragma unroll
      for (int kk = 0; kk < kKK / 2; ++kk) c = mfma32(a[kk], bop[kk], c);
      prefetch(t);
#pragma unroll
      for (int kk = kKK / 2; kk < kKK; ++kk) c = mfma32(a[kk], bop[kk], c);
      return c;
    };
    auto block_act = [&](int v) {
      const int i0 = walk.at(v) * kKvQB;
      const int i1 = min(N - 1, i0 + kKvQB - 1);
      if constexpr (TWO)
        return wave_live && set_meets(i0, i1, kw0, kw1, dset);
      else
        return wave_live && tile_meets(i0, i1, kw0, kw1, lo, hi);
    };

    // Both roles run every visit of the walk with the same straight-line
    // body: a block whose rows miss this wave's keys gets P = 0 from the P
    // wave (so the dS wave's dK update adds zeros), instead of branching
    // around the products -- branches there made the compiler shuttle the
    // 32 x d accumulators between register sets on every block.
    if (pwave) {
      // dV += P^T dO runs one block late as well, so the exponentials of
      // block v issue between the dV products of block v - 1 (whose dO tile
      // the ring still holds for the dS wave's Q).
      LaneOffsets<D> off(lane);
      bf16x8 pp0{}, pp1{};  // packed P of the previous block
      auto dv_operands = [&](int v, bf16x8* bb) {
        const bf16* dos = smem + (v % kKvStages) * 2 * kTile + kTile;
        load_va<D>(bb, dos, off, 0);
      };
      // within-tile row offset of accumulator register i, less 8 g
      auto creg = [](int i) { return ((i >> 3) << 4) + (i & 7); };
      auto p_block = [&](int t, auto has_prev) {
        block_start(t);
        const int v = t + voff;
        off.refresh();
        const int s = v % kKvStages;
        const bf16* qs = smem + s * 2 * kTile;
        const int i0 = walk.at(v) * kKvQB;
        const int i1 = min(N - 1, i0 + kKvQB - 1);
        // block flags first: their branches then sit before the products,
        // not between the exponentials and the products they interleave with
        const bool act = block_act(v);
        bool full_set;
        if constexpr (TWO)
          full_set = set_full(i0, i1, kw0, kw1, dset);
        else
          full_set = tile_full(i0, i1, kw0, kw1, lo, hi);
        const bool full = act && wave_keys_full && i0 + kKvQB - 1 <= N - 1 && full_set;
        bf16x8 aa[kKK];
        load_ka<D>(aa, qs, off, 0);
        __builtin_amdgcn_sched_barrier(0);
        const float zero16[16] = {};
        const f32x16 sc_ = chain_with_prefetch(aa, t, zero16);
        __builtin_amdgcn_sched_barrier(0);
        float nl[16], pv[16];
        rows16(&rowv[s][wave][0], nl);
        if constexpr (decltype(has_prev)::value) {
          bf16x8 bb[2 * kDT];
          dv_operands(v - 1, bb);
          // fixed order: one dV product of block v - 1, then its share of
          // the exponentials of block v
#pragma unroll
          for (int m = 0; m < 2 * kDT; ++m) {
            const int dt = m % kDT;
            acc[dt] = mfma32(bb[2 * dt + (m < kDT ? 0 : 1)], m < kDT ? pp0 : pp1, acc[dt]);
#pragma unroll
            for (int i = m * 16 / (2 * kDT); i < (m + 1) * 16 / (2 * kDT); ++i)
              pv[i] = fast_exp2(__builtin_fmaf(sc_[i], sl2, nl[i]));
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(__builtin_fmaf(sc_[i], sl2, nl[i]));
        }
        if (!full) {
          // Element mask: query row r = creg(i) + 8 g of the block is kept iff
          // it is below N and its distance to key kj lies in a range of the
          // set, i.e. 0 <= r - (kj + lo - i0) <= hi - lo (and likewise for
          // the second range); nothing is kept on a lane whose key is past N
          // or in a block that misses the wave's keys.  Moving 8 g to the
          // per-lane bounds leaves one compare per range and element.
          const bool keep = act && key_ok;
          const int rlim = N - i0 - 8 * g;  // creg(i) < rlim  <=>  row below N
          const int mb = kj + lo - i0 - 8 * g;
          const uint32_t width = (uint32_t)(hi - lo);
          int mb2 = kNoDistance;  // no second range: the test below never passes
          uint32_t width2 = 0;
          if constexpr (TWO) {
            if (has_second(dset)) {
              mb2 = kj + dset.nlo - i0 - 8 * g;
              width2 = (uint32_t)(dset.nhi - dset.nlo);
            }
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            bool in = (uint32_t)(creg(i) - mb) <= width;
            if constexpr (TWO) in = in | ((uint32_t)(creg(i) - mb2) <= width2);
            in = in & keep & (creg(i) < rlim);
            pv[i] = in ? pv[i] : 0.f;
          }
        }
        *(f16x8*)&pbuf[v & 1][kw][0][lane][0] = pack8_f16(&pv[0]);
        *(f16x8*)&pbuf[v & 1][kw][1][lane][0] = pack8_f16(&pv[8]);
        pp0 = pack8(&pv[0]);
        pp1 = pack8(&pv[8]);
      };
      p_block(0, std::false_type{});
      for (int t = 1; t < n_step; ++t) p_block(t, std::true_type{});
      __syncthreads();  // matches the dS waves' final barrier
      {
        bf16x8 bb[2 * kDT];
        dv_operands(n_step - 1 + voff, bb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) acc[dt] = mfma32(bb[2 * dt], pp0, acc[dt]);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) acc[dt] = mfma32(bb[2 * dt + 1], pp1, acc[dt]);
      }
    } else {
      // dP of block v into dp_new, then dS and dK of block v - 1 from dp_old;
      // the two dP registers alternate (loop unrolled by two), so nothing is
      // copied between blocks.
      auto d_block = [&](int t, f32x16& dp_new, const f32x16& dp_old, auto has_prev) {
        block_start(t);
        const int v = t + voff;
        const bf16* dos = smem + (v % kKvStages) * 2 * kTile + kTile;
        bf16x8 aa[kKK];
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) aa[kk] = row_chunk<D>(dos, prow, 16 * kk + 8 * g);
        float nd[16];  // -D of the block's rows (visit v has landed)
        rows16(&rowv[v % kKvStages][wave][kKvQB], nd);
        __builtin_amdgcn_sched_barrier(0);
        dp_new = chain_with_prefetch(aa, t, nd);
        if constexpr (decltype(has_prev)::value) ds_dk(v - 1, dp_old);
      };
      f32x16 dpa, dpb{};  // dpb: unused by the first block (no previous one)
      d_block(0, dpa, dpb, std::false_type{});
      int t = 1;
      for (; t + 1 < n_step; t += 2) {
        d_block(t, dpb, dpa, std::true_type{});
        d_block(t + 1, dpa, dpb, std::true_type{});
      }
      if (t < n_step) {
        d_block(t, dpb, dpa, std::true_type{});
        __syncthreads();  // P of the last block visible
        ds_dk(t + voff, dpb);
      } else {
        __syncthreads();  // P of the last block visible
        ds_dk(t - 1 + voff, dpa);
      }
    }
  }

  // dV (P waves) or dK = scale dS^T Q (dS waves), rows kw0 .. kw0 + 31; the
  // accumulators hold the transposed products dV^T and (dK / scale)^T.  A
  // tile without queries writes its zero rows directly.
  void* const dst = pwave ? p.dv : p.dk;
  const int nrows = min(32, N - kw0);
  if (n_visit == 0) {
    if (wave_live) store_zero_rows<D>(dst, sh.row0 + kw0, nrows, p.grad_f32 != 0, lane);
    return;
  }
  __syncthreads();  // ring and P buffers no longer read: the ring becomes the output staging area
  if (wave_live) {
    float* stg = (float*)smem + wave * 32 * D;
    stage_transposed<D>(stg, acc, pwave ? 1.f : p.scale, lane);
    store_staged<D>(stg, dst, sh.row0 + kw0, nrows, p.grad_f32 != 0, lane);
  }
}

}  // namespace

static BwdArgs make_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, bool grad_f32,
                         const Bands& bands, float scale, float* dvec, float* nl2, const Packed& pk) {
  BwdArgs a;
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.o = (const bf16*)o;
  a.dout = (const bf16*)dout;
  a.lse = lse;
  a.dvec = dvec;
  a.nl2 = nl2;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.grad_f32 = grad_f32 ? 1 : 0;
  a.B = B;
  a.H = H;
  a.N = N;
  a.n_tiles = 0;
  a.cu = pk.cu;
  a.T = pk.T;
  a.own_bdp = pk.own_bdp;
  a.local_window = 0;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.bands = bands;
  return a;
}

int launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                       void* dq, int B, int H, int N, int d, bool grad_f32, const Bands& bands, int local_window,
                       float scale, float* dvec, float* nl2, const Packed& pk, hipStream_t stream) {
  BwdArgs a = make_args(q, k, v, o, lse, dout, dq, nullptr, nullptr, B, H, N, grad_f32, bands, scale, dvec, nl2, pk);
  a.n_tiles = (N + kDqBQ - 1) / kDqBQ;
  a.local_window = local_window;
  const long long total = work_grid(B, H, a.n_tiles);
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  const dim3 grid((unsigned)total), block(kDqThreads);
  const bool two = local_window > 0;
  if (d == 128 && !two)
    hipLaunchKernelGGL((bwd_dq_kernel<128, false>), grid, block, 0, stream, a);
  else if (d == 128)
    hipLaunchKernelGGL((bwd_dq_kernel<128, true>), grid, block, 0, stream, a);
  else if (!two)
    hipLaunchKernelGGL((bwd_dq_kernel<64, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<64, true>), grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

int launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                         void* dv, int B, int H, int N, int d, bool grad_f32, const Bands& bands, int local_window,
                         float scale, float* dvec, float* nl2, const Packed& pk, hipStream_t stream) {
  BwdArgs a = make_args(q, k, v, nullptr, lse, dout, nullptr, dk, dv, B, H, N, grad_f32, bands, scale, dvec, nl2, pk);
  a.n_tiles = (N + kKvBK - 1) / kKvBK;
  a.local_window = local_window;
  const long long total = work_grid(B, H, a.n_tiles);
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  const dim3 grid((unsigned)total), block(kKvThreads);
  const bool two = local_window > 0;
  if (d == 128 && !two)
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, false>), grid, block, 0, stream, a);
  else if (d == 128)
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, true>), grid, block, 0, stream, a);
  else if (!two)
    hipLaunchKernelGGL((bwd_dkdv_kernel<64, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<64, true>), grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

// The walks of the two bfloat16 backward kernels.
WalkShape bwd_bf16_dq_walk() { return kDqWalk; }
WalkShape bwd_bf16_dkdv_walk() { return kKvWalk; }

}  // namespace spattn
