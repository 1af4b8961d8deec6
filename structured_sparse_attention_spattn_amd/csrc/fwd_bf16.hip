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
#include <type_traits>

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
  int B, H, N;  // sequences (B), heads, tokens per sequence (the longest, when packed)
  int n_qt;
  const int32_t* cu;  // packed sequence offsets [B + 1] (device), or null
  int T;              // packed: tokens per head
  int own_bdp;        // packed: each sequence's own BDP bands
  int local_window;  // shared local window width (0: exclusive bands)
  float scale_log2;
  Bands bands;
};

// Element mask of a tile for query iq against key block kb:
// base = iq - kb - 8 g - lo, width = hi - lo, and the same for the second
// distance range when there is one.
struct MaskArgs {
  int base, width, base2, width2;
};
template <bool TWO>
__device__ __forceinline__ void apply_mask(float* x, const MaskArgs& m, int shift) {
  if constexpr (TWO)
    band_mask2(x, m.base - shift, m.width, m.base2 - shift, m.width2);
  else
    band_mask(x, m.base - shift, m.width);
}

// Online-softmax state of one wave: O^T accumulator blocks, the reference
// maximum of every query column (raw score units) and this lane's share of
// the row sum, all relative to that reference.
template <int D>
struct OnlineState {
  f32x16 acc[D / 32];
  float m_ref;
  float l_run;
};

// A new reference maximum is taken only when some row's maximum has grown by
// more than 2^kRescaleLog2 over its reference (wave-uniform decision): until
// then probabilities are exp2 of at most kRescaleLog2, and numerator and
// denominator share the reference, so the result is the same softmax.  Most
// tiles then skip the rescale of the O accumulator entirely.
constexpr float kRescaleLog2 = 8.0f;

// Independent accumulator chains of the score product: one chain needs no
// adds afterwards, and the interleaved softmax work covers its latency.
constexpr int kChains = 1;

// Row maximum of one 32-key half, new reference, correction factor for the
// state accumulated so far (1 when the reference is kept) and the exponent
// offset -m_ref * scale_log2 of the probabilities.
__device__ __forceinline__ void reference_update(const float* x, float& m_ref, float sl2, float& alpha, bool& moved,
                                                 float& nms) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
  mx = pair_max(mx);
  const float m_new = fmaxf(m_ref, mx);
  moved = __ballot((m_new - m_ref) * sl2 > kRescaleLog2) != 0;  // -inf - -inf is NaN: false
  const float m_next = moved ? m_new : m_ref;
  alpha = m_next == m_ref ? 1.f : fast_exp2((m_ref - m_next) * sl2);
  m_ref = m_next;
  nms = -(m_ref == -__builtin_inff() ? 0.f : m_ref) * sl2;
}

// Probabilities of one half (in place), their sum, packed as the P^T operand.
__device__ __forceinline__ float probs(float* x, float sl2, float nms, bf16x8& p0, bf16x8& p1) {
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
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

// Both 32-key halves of a tile meet the wave's rows.  Software-pipelined so
// the exponentials of half 0 issue between the score MFMAs of half 1 and
// those of half 1 between the PV MFMAs of half 0.  When `masked` (a
// wave-uniform flag) the band mask is applied to both halves; the mask sits
// between phases, so its branch does not split an interleaved phase.
template <int D, bool TWO>
__device__ __forceinline__ void tile_pair(OnlineState<D>& st, const bf16* ks, const bf16* vs,
                                          const LaneOffsets<D>& off, const bf16x8* qreg, float sl2, bool masked,
                                          const MaskArgs& mk) {
  constexpr int kKK = D / 16, kDT = D / 32;
  // Phase boundaries are pinned (sched_barrier) so that operand reads of a
  // later phase are not hoisted into an earlier one, where they would only
  // lengthen register lifetimes.
  bf16x8 ka[kKK];
  load_ka<D>(ka, ks, off, 0);
  __builtin_amdgcn_sched_barrier(0);
  const f32x16 s0 = mfma_ksum<kKK, kChains>(ka, qreg);
  __builtin_amdgcn_sched_barrier(0);
  load_ka<D>(ka, ks, off, 32);
  float x0[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x0[i] = s0[i];
  if (masked) apply_mask<TWO>(x0, mk, 0);
  float alpha0, nms0;
  bool moved0;
  reference_update(x0, st.m_ref, sl2, alpha0, moved0, nms0);
  __builtin_amdgcn_sched_barrier(0);

  // scores of half 1 || probabilities of half 0
  const f32x16 s1 = mfma_ksum<kKK, kChains>(ka, qreg);
  bf16x8 pa0, pa1;
  st.l_run = st.l_run * alpha0 + probs(x0, sl2, nms0, pa0, pa1);
  keep_here(pa0);
  keep_here(pa1);
  interleave_mfma_valu<kKK, 16 / kKK, 48 / kKK>();
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 va[2 * kDT];
  load_va<D>(va, vs, off, 0);  // in flight during the half-1 row maximum

  float x1[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x1[i] = s1[i];
  if (masked) apply_mask<TWO>(x1, mk, 32);
  float alpha1, nms1;
  bool moved1;
  reference_update(x1, st.m_ref, sl2, alpha1, moved1, nms1);
  if (moved0) rescale<D>(st, alpha0);
  __builtin_amdgcn_sched_barrier(0);

  // PV of half 0 || probabilities of half 1
  pv<D>(st, va, pa0, pa1);
  bf16x8 pb0, pb1;
  st.l_run = st.l_run * alpha1 + probs(x1, sl2, nms1, pb0, pb1);
  keep_here(pb0);
  keep_here(pb1);
  interleave_mfma_valu<2 * kDT, 8 / kDT, 24 / kDT>();
  __builtin_amdgcn_sched_barrier(0);
  load_va<D>(va, vs, off, 32);
  if (moved1) rescale<D>(st, alpha1);
  __builtin_amdgcn_sched_barrier(0);
  pv<D>(st, va, pb0, pb1);
}

// Only half m of the tile meets the wave's rows (always masked).
template <int D, bool TWO>
__device__ __forceinline__ void tile_half(OnlineState<D>& st, const bf16* ks, const bf16* vs,
                                          const LaneOffsets<D>& off, const bf16x8* qreg, float sl2, int m,
                                          const MaskArgs& mk) {
  constexpr int kKK = D / 16, kDT = D / 32;
  bf16x8 ka[kKK];
  load_ka<D>(ka, ks, off, 32 * m);
  __builtin_amdgcn_sched_barrier(0);
  const f32x16 s = mfma_ksum<kKK, kChains>(ka, qreg);
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 va[2 * kDT];
  load_va<D>(va, vs, off, 32 * m);
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = s[i];
  apply_mask<TWO>(x, mk, 32 * m);
  float alpha, nms;
  bool moved;
  reference_update(x, st.m_ref, sl2, alpha, moved, nms);
  bf16x8 p0, p1;
  st.l_run = st.l_run * alpha + probs(x, sl2, nms, p0, p1);
  if (moved) rescale<D>(st, alpha);
  pv<D>(st, va, p0, p1);
}

template <int D, bool TWO>
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

  const WorkItem wi = work_item(blockIdx.x, p.B, p.H, p.n_qt);
  if (!wi.valid) return;  // padding pair
  const int t = wi.t;
  const int h = wi.h;
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, wi.b, h);
  const int N = sh.n;
  if (t * kBQ >= N) return;  // past the end of a packed sequence
  // the head's distance set: its band, joined with the local window if any
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
  const int i_tile1 = min(N - 1, i_tile0 + kBQ - 1);
  KeySpan span2{0, -1};
  if constexpr (TWO)
    if (has_second(dset)) span2 = band_key_span(i_tile0, i_tile1, dset.nlo, dset.nhi);
  TileWalk walk = tile_walk(band_key_span(i_tile0, i_tile1, lo, hi), span2, kBK);
  align_walk(walk, i_tile0 - hi, i_tile0 + kBQ - 1 - lo, kBK);
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

  // First K / V tile before the Q loads: the two round trips overlap (the
  // wait for Q covers both).
  Tile::load(smem, kb, walk.at(0) * kBK, N, wave, lane);
  Tile::load(smem + kTile, vb, walk.at(0) * kBK, N, wave, lane);

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
  st.l_run = 0.f;
  const float sl2 = p.scale_log2;

  // One tile from LDS stage S (a compile-time constant, so every LDS offset
  // is an immediate).
  auto step = [&](auto stage, int v) {
    constexpr int S = decltype(stage)::value;
    const int u = walk.at(v);
    wait_vmcnt<0>();  // this wave's part of tile u has landed
    __syncthreads();  // ... everyone's, and everyone is done with the previous tile
    if (v + 1 < walk.n) {
      bf16* nxt = smem + (S ^ 1) * 2 * kTile;
      const int un = walk.at(v + 1);
      Tile::load(nxt, kb, un * kBK, N, wave, lane);
      Tile::load(nxt + kTile, vb, un * kBK, N, wave, lane);
    }
    const bf16* ks = smem + S * 2 * kTile;
    const bf16* vs = ks + kTile;
    off.refresh();
    const int jb = u * kBK;
    bool a0, a1, full;
    if constexpr (TWO) {
      a0 = wave_live && set_meets(iw0, iw1, jb, jb + 31, dset);
      a1 = wave_live && set_meets(iw0, iw1, jb + 32, jb + 63, dset);
      full = set_full(iw0, iw1, jb, jb + 63, dset);
    } else {
      a0 = wave_live && tile_meets(iw0, iw1, jb, jb + 31, lo, hi);
      a1 = wave_live && tile_meets(iw0, iw1, jb + 32, jb + 63, lo, hi);
      full = tile_full(iw0, iw1, jb, jb + 63, lo, hi);
    }
    const int rb = iq - jb - 8 * g;
    const MaskArgs mk{rb - lo, hi - lo, rb - dset.nlo, dset.nhi - dset.nlo};
    if (a0 && a1) {
      tile_pair<D, TWO>(st, ks, vs, off, qreg, sl2, !full, mk);
    } else if (a0 || a1) {
      tile_half<D, TWO>(st, ks, vs, off, qreg, sl2, a0 ? 0 : 1, mk);
    }
  };
  for (int v = 0; v < walk.n; v += 2) {
    step(std::integral_constant<int, 0>{}, v);
    if (v + 1 < walk.n) step(std::integral_constant<int, 1>{}, v + 1);
  }

  // ---- epilogue: O = acc / l, LSE = scale * m + ln(sum)
  const float l_tot = pair_sum(st.l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (iq < N && g == 0) lb[iq] = l_tot > 0.f ? (st.m_ref * sl2 + fast_log2(l_tot)) * kLn2 : ninf;
  __syncthreads();  // every wave is done with the K / V ring: it becomes the output staging area
  if (wave_live) {
    float* stg = (float*)smem + wave * 32 * D;
    stage_transposed<D>(stg, st.acc, inv, lane);
    store_staged<D>(stg, p.o, sh.row0 + iw0, min(32, N - iw0), false, lane);
  }
}

}  // namespace

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
  a.n_qt = (N + kBQ - 1) / kBQ;
  a.cu = pk.cu;
  a.T = pk.T;
  a.own_bdp = pk.own_bdp;
  a.local_window = local_window;
  a.scale_log2 = scale * kLog2e;
  a.bands = bands;
  const long long total = work_grid(B, H, a.n_qt);
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  dim3 grid((unsigned)total), block(kThreads);
  const bool two = local_window > 0;
  if (d == 128 && !two)
    hipLaunchKernelGGL((fwd_bf16_kernel<128, false>), grid, block, 0, stream, a);
  else if (d == 128)
    hipLaunchKernelGGL((fwd_bf16_kernel<128, true>), grid, block, 0, stream, a);
  else if (d == 64 && !two)
    hipLaunchKernelGGL((fwd_bf16_kernel<64, false>), grid, block, 0, stream, a);
  else if (d == 64)
    hipLaunchKernelGGL((fwd_bf16_kernel<64, true>), grid, block, 0, stream, a);
  else
    return SPATTN_E_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

void fwd_bf16_tiles(int* BQ, int* BK) {
  *BQ = kBQ;
  *BK = kBK;
}

}  // namespace spattn
