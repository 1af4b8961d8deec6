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
//   each wave owns 32 query rows.  K and V tiles (BKT = 64 keys at d = 64,
//   32 at d = 128) stream into a ring of LDS stages with direct global -> LDS
//   loads (no register staging), one or two tiles ahead of the one in use.
//   The workgroup visits only the key tiles that intersect the diagonal
//   strip [i - hi_h, i - lo_h] of its rows; inside a tile each wave skips
//   the 32-key halves that miss its own 32-row strip, and masks element-wise
//   only where a half is PARTIAL (a wave-uniform branch).  Workgroups are
//   remapped so consecutive query tiles of one (b, h) run on the same XCD
//   and share the K/V strip through that XCD's L2, and the costliest query
//   tiles (the last ones of a sequence) are dispatched first.
// Products (transposed so no register shuffles are needed between them)
//   S^T (keys x queries) = K Q^T    A = K rows from LDS, B = Q in registers
//   O^T (d x queries)   += V^T P^T  A = V^T read from the row-major V tile
//                                    with the LDS transpose read,
//                                    B = P^T straight from the S^T registers
//   Each lane then owns one query column: the row maximum needs one
//   cross-lane exchange (lanes l and l+32), the row sum none until the end.
//   The score scale is folded into the exponent (one FMA per score).
#include <type_traits>

#include "common.h"

namespace spattn {
namespace {


struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int B, H, N;  // sequences (B), heads, tokens per sequence (the longest, when packed)
  int n_qt;
  const int32_t* cu;  // packed sequence offsets [B + 1] (device), or null
  int T;              // packed: tokens per head
  int own_bdp;        // packed: each sequence's own BDP bands
  int local_window;  // shared local window width (0: exclusive bands)
  float scale_log2;
  Bands bands;
};

// Online-softmax state of one wave: O^T accumulator blocks, the reference
// maximum of every query column (raw score units) with the exponent offset of
// its probabilities, and this lane's share of the row sum relative to that
// reference; plus what each of the two tests below keeps.
template <int D>
struct OnlineState {
  f32x16 acc[D / 32];
  float m_ref;
  float nms;    // exponent offset of the probabilities: -m_ref log2(e) scale (0 while m_ref is -inf)
  float l_run;
  float m_thr;  // maximum test: m_ref + kProbBoundLog2 / (log2(e) scale), -inf while m_ref is
  bool ready;   // sum test: no row of the wave has m_ref = -inf (wave-uniform)
};

// The reference of a row is moved (to the row's running maximum, rescaling
// what was accumulated) only when one of its probabilities could pass
// 2^kProbBoundLog2; until then numerator and denominator share the reference,
// so the result is the same softmax.  The decision is wave-uniform, and with
// scores of moderate range only a row's first half takes it.  Two tests:
//   maximum test: each lane compares the maximum of its 16 scores with m_thr;
//   sum test: once every row of the wave has a reference, the probabilities
//     are taken against it first; when the 16 of a lane sum to at most
//     2^kProbBoundLog2 each of them is at most that and the reference stays,
//     so the other halves never form a row maximum.  Otherwise the wave
//     recomputes the half's scores and moves the reference.
constexpr float kProbBoundLog2 = 8.0f;
constexpr float kProbBound = 256.0f;  // 2^kProbBoundLog2

// Row maximum of one 32-key half, the new reference (the running maximum),
// the correction factor of the state accumulated so far (1 where the
// reference stays, 0 where there was none) and the exponent offset
// -m_ref * scale_log2 of the probabilities.
__device__ __forceinline__ void reference_update(const float* x, float& m_ref, float sl2, float& alpha, bool& moved,
                                                 float& nms) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
  mx = pair_max(mx);
  const float m_new = fmaxf(m_ref, mx);
  moved = __ballot(m_new > m_ref) != 0;
  alpha = m_new == m_ref ? 1.f : fast_exp2((m_ref - m_new) * sl2);
  m_ref = m_new;
  nms = -(m_ref == -__builtin_inff() ? 0.f : m_ref) * sl2;
}

// Probabilities of one half against the exponent offset nms (in place), their
// float32 sum (the row sum, and through it the LSE, stays at float32
// accuracy), packed as the P^T operand.
__device__ __forceinline__ float probs(float* x, float sl2, float nms, bf16x8& p0, bf16x8& p1) {
  x[0] = fast_exp2(__builtin_fmaf(x[0], sl2, nms));
  float sum = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    x[i] = fast_exp2(__builtin_fmaf(x[i], sl2, nms));
    sum += x[i];
  }
  p0 = pack8(&x[0]);
  p1 = pack8(&x[8]);
  return sum;
}

template <int D>
__device__ __forceinline__ void rescale(OnlineState<D>& st, float alpha) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.acc[dt][i] *= alpha;
}

template <int D>
__device__ __forceinline__ void pv(OnlineState<D>& st, const bf16x8* va, bf16x8 p0, bf16x8 p1) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    st.acc[dt] = mfma32(va[2 * dt], p0, st.acc[dt]);
    st.acc[dt] = mfma32(va[2 * dt + 1], p1, st.acc[dt]);
  }
}

// The forward kernel: one 32-key half at a time with a single straight-line
// body (no software pipelining across halves, so the state is one
// accumulator set and one score block) and a register budget for OCC
// workgroups per CU, so the other waves of each SIMD hide one wave's
// dependent MFMA / softmax chain.  K / V arrive in tiles of BKT keys (32 or
// 64: one or two halves) through a ring of STAGES LDS stages, STAGES - 1
// tiles ahead.  Per half: scores S^T = K Q^T, the element mask only where
// the half is PARTIAL for this wave's rows, the reference update, P and its
// row sum, O^T += V^T P^T.
template <int D, int BKT, int STAGES, int OCC, bool SUM_TEST, int WAVES = 4>
struct FwdCfg {
  static constexpr int kD = D, kBKT = BKT, kStages = STAGES, kOcc = OCC, kWaves = WAVES;
  static constexpr bool kSumTest = SUM_TEST;  // the sum test of the reference, else the maximum test
  static constexpr int kBQ = 32 * WAVES;  // query rows per workgroup (32 per wave)
  static constexpr int kThreads = 64 * WAVES;
  // query-major: the workgroup's rows own BKT-key tiles, a single run rotated (align_walk)
  static constexpr WalkShape walk{kBQ, BKT, false, true};
};
// d = 64: 64-key tiles, two stages (32 KB of LDS), at most 128 VGPRs: four
// workgroups per CU; the sum test (its halves are VALU-bound: 4 % faster than
// the maximum test at B2 H12 N10000).  d = 128: 32-key tiles, three stages
// (48 KB), at most 168 VGPRs: three workgroups per CU (measured against 64-key
// tiles at two per CU and a four-stage ring at two per CU: 115 vs 122 and
// 125 us at B8 H16 N4096; and against a cross-half pipelined kernel at two per
// CU: 124 us); the maximum test (the sum test's recompute path spills there).
using Fwd64 = FwdCfg<64, 64, 2, 4, true>;
using Fwd128 = FwdCfg<128, 32, 3, 3, false>;

template <typename C, bool TWO>
__global__ __launch_bounds__(C::kThreads, C::kOcc) void fwd_bf16_kernel(FwdArgs p) {
  constexpr int D = C::kD;
  constexpr int BKT = C::kBKT;
  constexpr int STAGES = C::kStages;
  constexpr int kTile = BKT * D;  // one K or V tile, bf16 elements
  constexpr int kBQ = C::kBQ;
  constexpr int kThreads = C::kThreads;
  using Tile = AsyncTile<BKT, D, C::kWaves>;
  constexpr int kL = 2 * Tile::kPer;  // loads per wave per tile (K and V)
  constexpr int kDT = D / 32;
  constexpr int kKK = D / 16;
  __shared__ __attribute__((aligned(16))) bf16 smem[STAGES * 2 * kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int c32 = lane & 31;

  const WorkItem wi = work_item(blockIdx.x, p.B, p.H, p.n_qt, true);
  if (!wi.valid) return;  // padding pair
  const int t = wi.t;
  const int h = wi.h;
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, wi.b, h);
  const int N = sh.n;
  if (t * kBQ >= N) return;  // past the end of a packed sequence
  const DistSet dset = dist_set(sh.lo, sh.hi, TWO ? p.local_window : 0);
  const int lo = dset.lo;
  const int hi = dset.hi;
  const size_t base = sh.row0 * D;
  const bf16* __restrict__ qb = p.q + base;
  const bf16* __restrict__ kb = p.k + base;
  const bf16* __restrict__ vb = p.v + base;
  bf16* __restrict__ ob = p.o + base;
  float* __restrict__ lb = p.lse + sh.row0;
  const float ninf = -__builtin_inff();

  const int i_tile0 = t * kBQ;
  const TileWalk walk = kernel_walk(C::walk, i_tile0, N, dset);
  if (walk.n == 0) {
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
  const int iw0 = i_tile0 + 32 * wave;
  const int iw1 = min(N - 1, iw0 + 31);
  const bool wave_live = iw0 <= N - 1;
  const int iq = iw0 + c32;

  const typename Tile::Offsets toff(wave, lane);
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  auto issue = [&](int v) {
    const uint32_t st = smem_lds + (uint32_t)((v % STAGES) * 2 * kTile * 2);
    const int u = walk.at(v);
    Tile::load(st, kb, u * BKT, N, toff, wave, lane);
    Tile::load(st + 2 * kTile, vb, u * BKT, N, toff, wave, lane);
  };
  // the ring prefill before the Q loads: the round trips overlap
#pragma unroll
  for (int i = 0; i < STAGES - 1; ++i)
    if (i < walk.n) issue(i);

  // Q^T operand: lane holds Q[iq][16kk + 8g .. +7].
  bf16x8 qreg[kKK];
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk)
    qreg[kk] = iq < N ? *(const bf16x8*)(qb + (size_t)iq * D + 16 * kk + 8 * g) : bf16x8{};
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) settle(qreg[kk]);
  LaneOffsets<D> off(lane);

  OnlineState<D> st;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.acc[dt][i] = 0.f;
  st.m_ref = ninf;
  st.nms = 0.f;
  st.m_thr = ninf;
  st.ready = false;
  st.l_run = 0.f;
  const float sl2 = p.scale_log2;

  // One 32-key half M (compile-time) of the tile in stage S.
  auto half = [&](auto stage, auto half_idx, int jb) {
    constexpr int S = decltype(stage)::value;
    constexpr int M = decltype(half_idx)::value;
    const int j0 = jb + 32 * M;
    bool meets, full;
    if constexpr (TWO) {
      meets = wave_live && set_meets(iw0, iw1, j0, j0 + 31, dset);
      full = set_full(iw0, iw1, j0, j0 + 31, dset);
    } else {
      meets = wave_live && tile_meets(iw0, iw1, j0, j0 + 31, lo, hi);
      full = tile_full(iw0, iw1, j0, j0 + 31, lo, hi);
    }
    if (!meets) return;
    const bf16* ks = smem + S * 2 * kTile;
    const bf16* vs = ks + kTile;
    // S^T of the half, masked to the distance set where the half is partial
    // for this wave's rows
    auto scores = [&](float* x, const LaneOffsets<D>& o) {
      bf16x8 ka[kKK];
      load_ka<D>(ka, ks, o, 32 * M);
      const f32x16 sc = mfma_ksum<kKK, 1>(ka, qreg);
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = sc[i];
      if (!full) {
        const int rb = iq - j0 - 8 * g;
        if constexpr (TWO)
          band_mask2(x, rb - lo, hi - lo, rb - dset.nlo, dset.nhi - dset.nlo);
        else
          band_mask(x, rb - lo, hi - lo);
      }
    };
    // new references for the wave's rows (wave-uniform)
    auto take_reference = [&](const float* x) {
      float alpha;
      bool moved;
      reference_update(x, st.m_ref, sl2, alpha, moved, st.nms);
      st.ready = __ballot(st.m_ref == -__builtin_inff()) == 0;
      st.m_thr = st.m_ref == -__builtin_inff() ? -__builtin_inff() : st.m_ref + kProbBoundLog2 / sl2;
      if (moved) {
        rescale<D>(st, alpha);
        st.l_run *= alpha;
      }
    };
    // the row sum and O^T += V^T P^T
    auto finish = [&](float s, bf16x8 p0, bf16x8 p1) {
      st.l_run += s;
      bf16x8 va[2 * kDT];
      load_va<D>(va, vs, off, 32 * M);
      pv<D>(st, va, p0, p1);
    };
    float x[16];
    scores(x, off);
    bf16x8 p0, p1;
    if constexpr (C::kSumTest) {
      if (st.ready) {
        const float s = probs(x, sl2, st.nms, p0, p1);
        if (__ballot(!(s <= kProbBound)) == 0) {
          finish(s, p0, p1);
          return;
        }
        // the scores again from the K tile, still in its stage (the empty
        // asm with a memory clobber makes the compiler reload the operands
        // instead of holding the first ones all along)
        asm volatile("" ::: "memory");
        scores(x, off);
      }
      take_reference(x);
    } else {
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
      if (__ballot(!(mx <= st.m_thr)) != 0) take_reference(x);
    }
    const float s = probs(x, sl2, st.nms, p0, p1);
    finish(s, p0, p1);
  };
  auto step = [&](auto stage, int v) {
    constexpr int S = decltype(stage)::value;
    // this wave's loads of tile v have landed: the ones still allowed in
    // flight belong to the tiles after v that are already issued
    const int ahead = min(STAGES - 2, walk.n - 1 - v);
    if (STAGES >= 4 && ahead >= 2)
      wait_vmcnt<2 * kL>();
    else if (STAGES >= 3 && ahead >= 1)
      wait_vmcnt<kL>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // ... everyone's, and everyone is done with tile v - 1
    if (v + STAGES - 1 < walk.n) issue(v + STAGES - 1);  // into the stage tile v - 1 used
    off.refresh();
    const int jb = walk.at(v) * BKT;
    half(stage, std::integral_constant<int, 0>{}, jb);
    if constexpr (BKT == 64) half(stage, std::integral_constant<int, 1>{}, jb);
  };
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
  int v = 0;
  for (; v + STAGES <= walk.n; v += STAGES) {
    step(std::integral_constant<int, 0>{}, v);
    step(std::integral_constant<int, 1>{}, v + 1);
    if constexpr (STAGES >= 3) step(std::integral_constant<int, 2>{}, v + 2);
    if constexpr (STAGES >= 4) step(std::integral_constant<int, 3>{}, v + 3);
  }
  if (v < walk.n) step(std::integral_constant<int, 0>{}, v);
  if (v + 1 < walk.n) step(std::integral_constant<int, 1>{}, v + 1);
  if constexpr (STAGES >= 3)
    if (v + 2 < walk.n) step(std::integral_constant<int, 2>{}, v + 2);

  const float l_tot = pair_sum(st.l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (iq < N && g == 0) lb[iq] = l_tot > 0.f ? (st.m_ref * sl2 + fast_log2(l_tot)) * kLn2 : ninf;
  __syncthreads();  // every wave is done with the K / V ring: it becomes the output staging area
  if (wave_live) {
    // 32 x 64 floats per wave fit every ring here (d = 128: two passes)
    constexpr int kNC = D < 64 ? D : 64;
    static_assert(C::kWaves * 32 * kNC * 4 <= (int)sizeof(smem), "output staging fits the K / V ring");
    store_result<D, kNC>((float*)smem + wave * 32 * kNC, st.acc, inv, p.o, sh.row0 + iw0, min(32, N - iw0), false,
                         lane);
  }
}

}  // namespace

template <typename C>
static int launch_cfg(FwdArgs a, bool two, hipStream_t stream) {
  a.n_qt = (a.N + C::kBQ - 1) / C::kBQ;
  const long long total = work_grid(a.B, a.H, a.n_qt);
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  const dim3 grid((unsigned)total), block(C::kThreads);
  if (two)
    hipLaunchKernelGGL((fwd_bf16_kernel<C, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<C, false>), grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

int launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int N, int d, const Bands& bands, int local_window, float scale, const Packed& pk,
                    hipStream_t stream) {
  FwdArgs a;
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.o = (bf16*)o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  a.cu = pk.cu;
  a.T = pk.T;
  a.own_bdp = pk.own_bdp;
  a.local_window = local_window;
  a.scale_log2 = scale * kLog2e;
  a.bands = bands;
  const bool two = local_window > 0;
  if (d == 128) return launch_cfg<Fwd128>(a, two, stream);
  if (d == 64) return launch_cfg<Fwd64>(a, two, stream);
  return SPATTN_E_UNSUPPORTED;
}

WalkShape fwd_bf16_walk(int d);

void fwd_bf16_tiles(int d, int* BQ, int* BK) {
  const WalkShape w = fwd_bf16_walk(d);
  *BQ = w.own;
  *BK = w.tile;
}

WalkShape fwd_bf16_walk(int d) { return d == 64 ? Fwd64::walk : Fwd128::walk; }

}  // namespace spattn
