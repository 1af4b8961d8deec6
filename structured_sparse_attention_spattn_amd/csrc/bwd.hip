// Backward of band-partitioned attention (textbook derivative of the
// masked-set softmax of "Sparse Attention, Then and Now" section 1 over the
// distance bands of "Making Every Head Count" Figure 1; no page gives a
// backward pass).  With P recomputed from the saved LSE:
//     D_i = dO_i . O_i,  dP = dO V^T,  dS = P * (dP - D),
//     dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// This file holds the preprocess of the float32 path and the dispatcher; the
// MFMA kernels are in bwd_bf16.hip and bwd_f32.hip.
//   bwd_pre      D_i = dO_i . O_i for every row (float32 path only; the
//                bfloat16 dQ kernel computes D from its own rows).
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
int launch_bwd_dq_f32(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dq,
                      int B, int H, int N, int d, const Bands& bands, int local_window, float scale,
                      const float* dvec, const Packed& pk, hipStream_t stream);
int launch_bwd_dkdv_f32(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                        void* dv, int B, int H, int N, int d, const Bands& bands, int local_window, float scale,
                        const float* dvec, const Packed& pk, hipStream_t stream);
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

// Stage 1: D_i = dO_i . O_i into the workspace, and dQ.
int launch_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, int B, int H, int N, int d, int dtype, int grad_dtype, const Bands& bands,
                  int local_window, float scale, const Packed& pk, void* workspace, hipStream_t stream) {
  float* dvec = row_vector(workspace, 0, B, H, N, pk);
  if (dtype == SPATTN_BF16)
    return launch_bwd_dq_bf16(q, k, v, o, lse, dout, dq, B, H, N, d, grad_dtype == SPATTN_F32, bands, local_window,
                              scale, dvec, row_vector(workspace, 1, B, H, N, pk), pk, stream);
  {
    const long long data_rows = pk.cu != nullptr ? (long long)H * pk.T : (long long)B * H * N;  // rows held in the tensors
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
  return launch_bwd_dq_f32(q, k, v, lse, dout, dq, B, H, N, d, bands, local_window, scale, dvec, pk, stream);
}

// Stage 2: dK and dV, reading D from the workspace written by stage 1.
int launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                    void* dv, int B, int H, int N, int d, int dtype, int grad_dtype, const Bands& bands,
                    int local_window, float scale, const Packed& pk, void* workspace, hipStream_t stream) {
  float* dvec = row_vector(workspace, 0, B, H, N, pk);
  if (dtype == SPATTN_BF16)
    return launch_bwd_dkdv_bf16(q, k, v, lse, dout, dk, dv, B, H, N, d, grad_dtype == SPATTN_F32, bands,
                                local_window, scale, dvec, row_vector(workspace, 1, B, H, N, pk), pk, stream);
  return launch_bwd_dkdv_f32(q, k, v, lse, dout, dk, dv, B, H, N, d, bands, local_window, scale, dvec, pk, stream);
}

}  // namespace spattn
