// Backward of band-partitioned attention (textbook derivative of the
// masked-set softmax of "Sparse Attention, Then and Now" section 1 over the
// distance bands of "Making Every Head Count" Figure 1; no page gives a
// backward pass).  With P recomputed from the saved LSE:
//     D_i = dO_i . O_i,  dP = dO V^T,  dS = P * (dP - D),
//     dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// This file holds the float32 path (one wave per row, wave reductions) and
// the dispatcher; the bfloat16 MFMA kernels are in bwd_bf16.hip.
//   bwd_pre      D_i = dO_i . O_i for every row (float32 path only).
//   bwd_f32_dq   one wave per query row:  dQ_i = scale sum_j dS_ij k_j.
//   bwd_f32_dkdv one wave per key row:    dK_j, dV_j over the queries reaching j.
#include "common.h"

namespace spattn {
namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------ preprocess
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                           float* __restrict__ dvec, long long rows) {
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
  }
#pragma unroll
  for (int off = kLanes / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && part == 0) dvec[row] = -s;  // the workspace holds -D
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
  int B, H, N;  // sequences (B), heads, tokens per sequence (the longest, when packed)
  int local_window;  // shared local window width (0: exclusive bands)
  float scale;
  const int32_t* cu;  // packed sequence offsets [B + 1] (device), or null
  int T;              // packed: tokens per head
  int own_bdp;        // packed: each sequence's own BDP bands
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
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, (int)(bh / p.H), h);
  if (i >= sh.n) return;  // past the end of a packed sequence
  const DistSet ds_ = dist_set(sh.lo, sh.hi, p.local_window);
  const size_t base = sh.row0 * D;
  float qi[kE], di[kE], acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    qi[e] = p.q[base + (size_t)i * D + lane + 64 * e];
    di[e] = p.dout[base + (size_t)i * D + lane + 64 * e];
    acc[e] = 0.f;
  }
  const float lse = p.lse[sh.row0 + i], nd = p.dvec[sh.row0 + i];  // nd = -D_i
  // keys of row i: the primary range, then the disjoint second range if any
  KeySpan spans[2] = {band_key_span(i, i, ds_.lo, ds_.hi), KeySpan{0, -1}};
  if (has_second(ds_)) spans[1] = band_key_span(i, i, ds_.nlo, ds_.nhi);
  for (int sp = 0; sp < 2; ++sp)
  for (int j = spans[sp].first; j <= spans[sp].last; ++j) {
    float kj[kE], vj[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      kj[e] = p.k[base + (size_t)j * D + lane + 64 * e];
      vj[e] = p.v[base + (size_t)j * D + lane + 64 * e];
    }
    const float s = wave_dot<D>(qi, kj, lane) * p.scale;
    const float pij = expf(s - lse);
    const float dp = wave_dot<D>(di, vj, lane);
    const float ds = pij * (dp + nd);
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
  const SeqHead sh = seq_head(p.cu, p.T, p.own_bdp, p.H, p.N, p.bands, (int)(bh / p.H), h);
  if (j >= sh.n) return;  // past the end of a packed sequence
  const DistSet ds_ = dist_set(sh.lo, sh.hi, p.local_window);
  const int N = sh.n;
  const size_t base = sh.row0 * D;
  const size_t lbase = sh.row0;
  float kj[kE], vj[kE], dk[kE], dv[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    kj[e] = p.k[base + (size_t)j * D + lane + 64 * e];
    vj[e] = p.v[base + (size_t)j * D + lane + 64 * e];
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  // queries reaching key j: the primary range, then the disjoint second range if any
  KeySpan spans[2] = {band_query_span(j, j, ds_.lo, ds_.hi, N), KeySpan{0, -1}};
  if (has_second(ds_)) spans[1] = band_query_span(j, j, ds_.nlo, ds_.nhi, N);
  for (int sp = 0; sp < 2; ++sp)
  for (int i = spans[sp].first; i <= spans[sp].last; ++i) {
    float qi[kE], di[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      qi[e] = p.q[base + (size_t)i * D + lane + 64 * e];
      di[e] = p.dout[base + (size_t)i * D + lane + 64 * e];
    }
    const float s = wave_dot<D>(qi, kj, lane) * p.scale;
    const float pij = expf(s - p.lse[lbase + i]);
    const float dp = wave_dot<D>(di, vj, lane);
    const float ds = pij * (dp + p.dvec[lbase + i]);  // dvec holds -D
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
  (void)d;
  (void)dtype;
  (void)grad_dtype;
  const size_t rows = (size_t)B * H * N;
  return 2 * ((rows * sizeof(float) + 255) / 256 * 256);  // -D, then -LSE * log2(e)
}

int launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                       void* dq, int B, int H, int N, int d, bool grad_f32, const Bands& bands, int local_window,
                       float scale, float* dvec, float* nl2, const Packed& pk, hipStream_t stream);
int launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                         void* dv, int B, int H, int N, int d, bool grad_f32, const Bands& bands, int local_window,
                         float scale, float* dvec, float* nl2, const Packed& pk, hipStream_t stream);

// The workspace holds two float vectors over the rows of the tensors, each
// starting on a 256-byte boundary: -D_i (so dP - D is dP plus a stored value,
// or an MFMA chain started from it), then -LSE_i * log2(e) (the bfloat16
// kernels' exponent offset, written by the dQ kernel for the dK/dV kernel).
static float* row_vector(void* workspace, int which, int B, int H, int N, const Packed& pk) {
  const size_t rows = pk.cu != nullptr ? (size_t)H * pk.T : (size_t)B * H * N;
  return (float*)workspace + which * ((rows + 63) / 64 * 64);
}

static BwdF32Args f32_args(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dq,
                           void* dk, void* dv, int B, int H, int N, const Bands& bands, int local_window,
                           float scale, float* dvec, const Packed& pk) {
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
  a.local_window = local_window;
  a.scale = scale;
  a.cu = pk.cu;
  a.T = pk.T;
  a.own_bdp = pk.own_bdp;
  a.bands = bands;
  return a;
}

// Stage 1: D_i = dO_i . O_i into the workspace, and dQ.
int launch_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, int B, int H, int N, int d, int dtype, int grad_dtype, const Bands& bands,
                  int local_window, float scale, const Packed& pk, void* workspace, hipStream_t stream) {
  float* dvec = row_vector(workspace, 0, B, H, N, pk);
  if (dtype == SPATTN_BF16)
    return launch_bwd_dq_bf16(q, k, v, o, lse, dout, dq, B, H, N, d, grad_dtype == SPATTN_F32, bands, local_window,
                              scale, dvec, row_vector(workspace, 1, B, H, N, pk), pk, stream);
  const long long rows = (long long)B * H * N;  // one wave per (sequence, head, row); packed: padded to N
  {
    const long long data_rows = pk.cu != nullptr ? (long long)H * pk.T : rows;  // rows held in the tensors
    const long long threads = data_rows * (d / 8);
    dim3 grid((unsigned)((threads + kThreads - 1) / kThreads)), block(kThreads);
    if (d == 128)
      hipLaunchKernelGGL((bwd_pre_kernel<float, 128>), grid, block, 0, stream, (const float*)o, (const float*)dout,
                         dvec, data_rows);
    else
      hipLaunchKernelGGL((bwd_pre_kernel<float, 64>), grid, block, 0, stream, (const float*)o, (const float*)dout,
                         dvec, data_rows);
    if (hipGetLastError() != hipSuccess) return SPATTN_E_HIP;
  }
  BwdF32Args a = f32_args(q, k, v, lse, dout, dq, nullptr, nullptr, B, H, N, bands, local_window, scale, dvec, pk);
  dim3 grid((unsigned)((rows + 3) / 4)), block(kThreads);
  if (d == 128)
    hipLaunchKernelGGL(bwd_f32_dq_kernel<128>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_f32_dq_kernel<64>, grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

// Stage 2: dK and dV, reading D from the workspace written by stage 1.
int launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                    void* dv, int B, int H, int N, int d, int dtype, int grad_dtype, const Bands& bands,
                    int local_window, float scale, const Packed& pk, void* workspace, hipStream_t stream) {
  float* dvec = row_vector(workspace, 0, B, H, N, pk);
  if (dtype == SPATTN_BF16)
    return launch_bwd_dkdv_bf16(q, k, v, lse, dout, dk, dv, B, H, N, d, grad_dtype == SPATTN_F32, bands,
                                local_window, scale, dvec, row_vector(workspace, 1, B, H, N, pk), pk, stream);
  const long long rows = (long long)B * H * N;  // one wave per (sequence, head, row); packed: padded to N
  BwdF32Args a = f32_args(q, k, v, lse, dout, nullptr, dk, dv, B, H, N, bands, local_window, scale, dvec, pk);
  dim3 grid((unsigned)((rows + 3) / 4)), block(kThreads);
  if (d == 128)
    hipLaunchKernelGGL(bwd_f32_dkdv_kernel<128>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_f32_dkdv_kernel<64>, grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

}  // namespace spattn
