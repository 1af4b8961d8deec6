// Single-query band attention over a key/value cache (the decode step).
//
// At position i = L_b - 1 of sequence b, head h attends the cached keys j
// with i - j in its band [lo_h, hi_h] ("Making Every Head Count", Figure 1
// caption), joined with the shared local window [0, w - 1] when w > 0
// (Figure 2 caption reading), through the masked-set softmax of "Sparse
// Attention, Then and Now", section 1.  The work is a gather of W key and
// value rows per (b, h) and is bound by HBM bandwidth, not by products.
//
// One workgroup (4 waves) per (b, h).  A head's key set is at most two
// contiguous runs of cache rows, walked as one virtual index t.  Each wave
// takes chunks of rows; D / 8 lanes share one row, every lane holding 8
// consecutive features (so K and V loads are whole-row, 16- or 32-byte
// pieces per lane), and a row's score is reduced over those lanes.  Online
// softmax across a wave's chunks; the four waves' (max, sum, output) are
// merged through LDS.
#include "common.h"

namespace spattn {
namespace {

struct DecodeArgs {
  const void* q;    // [B, H, d]
  const void* k;    // [B, H, Nmax, d]
  const void* v;    // [B, H, Nmax, d]
  void* o;          // [B, H, d]
  float* lse;       // [B, H]
  const int32_t* lengths;  // [B] valid cache rows, or null for Nmax
  int B, H, Nmax;
  int local_window;
  float scale_log2;
  Bands bands;
};

// 8 consecutive values of a row as loaded (raw) and widened to float.
template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  typedef bf16x8 Raw;
  __device__ __forceinline__ static Raw load(const bf16* p) { return *(const bf16x8*)p; }
  __device__ __forceinline__ static Raw zero() { return bf16x8{}; }
  __device__ __forceinline__ static float at(const Raw& v, int e) { return (float)v[e]; }
  __device__ __forceinline__ static void store(bf16* p, const float* x) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
    *(bf16x8*)p = v;
  }
};
template <>
struct Vec8<float> {
  struct Raw {
    f32x4 a, b;
  };
  __device__ __forceinline__ static Raw load(const float* p) { return Raw{*(const f32x4*)p, *(const f32x4*)(p + 4)}; }
  __device__ __forceinline__ static Raw zero() { return Raw{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }
  __device__ __forceinline__ static float at(const Raw& v, int e) { return e < 4 ? v.a[e] : v.b[e - 4]; }
  __device__ __forceinline__ static void store(float* p, const float* x) {
    *(f32x4*)p = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4*)(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
};

constexpr int kDecThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads, 4) void decode_kernel(DecodeArgs p) {
  constexpr int kLpr = D / 8;                       // lanes per cache row
  constexpr int kRpi = 64 / kLpr;                   // rows per wave step
  constexpr int kSteps = sizeof(T) == 2 ? 8 : 4;    // steps per chunk (register budget: 4 waves per SIMD)
  constexpr int kChunk = kSteps * kRpi;             // rows per chunk
  constexpr int kWaves = kDecThreads / 64;
  __shared__ float red_m[kWaves], red_l[kWaves];
  __shared__ float red_o[kWaves][D];

  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / kLpr, c = lane % kLpr;
  const float ninf = -__builtin_inff();

  int L = p.lengths != nullptr ? p.lengths[b] : p.Nmax;
  L = L < 0 ? 0 : (L > p.Nmax ? p.Nmax : L);

  float m = ninf, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  if (L > 0) {
    const int i = L - 1;
    const DistSet ds = dist_set(p.bands.lo[h], p.bands.hi[h], p.local_window);
    // run 1: the primary distance range [lo, hi] -> rows [i - hi, i - lo];
    // run 2: the second range (a window below the band) -> larger rows.
    const int a0 = max(0, i - ds.hi), a1 = i - ds.lo;
    const int n1 = (ds.hi >= ds.lo && a1 >= a0) ? a1 - a0 + 1 : 0;
    int b0 = 0, n2 = 0;
    if (has_second(ds)) {
      b0 = max(0, i - ds.nhi);
      const int b1 = i - ds.nlo;
      n2 = b1 >= b0 ? b1 - b0 + 1 : 0;
    }
    const int nk = n1 + n2;
    const size_t head = (size_t)bh * p.Nmax * D;
    const T* __restrict__ kb = (const T*)p.k + head;
    const T* __restrict__ vb = (const T*)p.v + head;
    float qf[8];
    {
      const typename Vec8<T>::Raw qr = Vec8<T>::load((const T*)p.q + (size_t)bh * D + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[e] = Vec8<T>::at(qr, e) * p.scale_log2;  // scores in log2 units
    }

    for (int t0 = wave * kChunk; t0 < nk; t0 += kWaves * kChunk) {
      typename Vec8<T>::Raw kx[kSteps], vx[kSteps];
      bool ok[kSteps];
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int t = t0 + s * kRpi + r;
        ok[s] = t < nk;
        const int j = t < n1 ? a0 + t : b0 + (t - n1);
        kx[s] = ok[s] ? Vec8<T>::load(kb + (size_t)j * D + 8 * c) : Vec8<T>::zero();
        vx[s] = ok[s] ? Vec8<T>::load(vb + (size_t)j * D + 8 * c) : Vec8<T>::zero();
      }
      float sc[kSteps];
      float mc = ninf;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf(qf[e], Vec8<T>::at(kx[s], e), part);
#pragma unroll
        for (int off = kLpr / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, kLpr);
        sc[s] = ok[s] ? part : ninf;
        mc = fmaxf(mc, sc[s]);
      }
#pragma unroll
      for (int off = kLpr; off < 64; off <<= 1) mc = fmaxf(mc, __shfl_xor(mc, off));
      const float mn = fmaxf(m, mc);  // wave-uniform; finite: the chunk has a valid row
      const float alpha = fast_exp2(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const float pr = fast_exp2(sc[s] - m);  // 0 for rows past the set
        l += pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(pr, Vec8<T>::at(vx[s], e), o[e]);
      }
    }
    // every lane holds its row group's sums (l over the group's rows, o over
    // its 8 features): add the groups, lanes of one feature slice c together
#pragma unroll
    for (int off = kLpr; off < 64; off <<= 1) {
      l += __shfl_xor(l, off);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], off);
    }
  }

  if (lane < kLpr) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red_o[wave][8 * lane + e] = o[e];
  }
  if (lane == 0) {
    red_m[wave] = m;
    red_l[wave] = l;
  }
  __syncthreads();
  if (wave == 0 && lane < kLpr) {
    float M = ninf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w]);
    float Lt = 0.f, out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = 0.f;
    if (M != ninf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = red_m[w] == ninf ? 0.f : fast_exp2(red_m[w] - M);
        Lt += red_l[w] * f;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] += red_o[w][8 * lane + e] * f;
      }
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] *= inv;
    Vec8<T>::store((T*)p.o + (size_t)bh * D + 8 * lane, out);
    if (lane == 0) p.lse[bh] = Lt > 0.f ? (M + fast_log2(Lt)) * kLn2 : ninf;
  }
}

}  // namespace

int launch_decode(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* lengths, int B,
                  int H, int Nmax, int d, int dtype, const Bands& bands, int local_window, float scale,
                  hipStream_t stream) {
  DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.lengths = lengths;
  a.B = B;
  a.H = H;
  a.Nmax = Nmax;
  a.local_window = local_window;
  a.scale_log2 = scale * kLog2e;
  a.bands = bands;
  const long long total = (long long)B * H;
  if (total > 0x7fffffffLL) return SPATTN_E_ARG;
  const dim3 grid((unsigned)total), block(kDecThreads);
  if (dtype == SPATTN_BF16 && d == 128)
    hipLaunchKernelGGL((decode_kernel<bf16, 128>), grid, block, 0, stream, a);
  else if (dtype == SPATTN_BF16)
    hipLaunchKernelGGL((decode_kernel<bf16, 64>), grid, block, 0, stream, a);
  else if (d == 128)
    hipLaunchKernelGGL((decode_kernel<float, 128>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<float, 64>), grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

}  // namespace spattn
