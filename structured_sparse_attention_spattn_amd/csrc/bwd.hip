// Backward of band-partitioned attention (textbook derivative of the
// masked-set softmax of "Sparse Attention, Then and Now" section 1 over the
// distance bands of "Making Every Head Count" Figure 1; no page gives a
// backward pass).  With P recomputed from the saved LSE:
//     D_i = dO_i . O_i,  dP = dO V^T,  dS = P * (dP - D),
//     dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// This file holds the workspace layout and the dispatch by dtype; the MFMA
// kernels are in bwd_bf16.hip and bwd_f32.hip.  In both paths the dQ kernel
// forms D_i for its own rows and stores -D_i for the dK/dV kernel.
#include "common.h"

namespace spattn {

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
int launch_bwd_dq_f32(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                      void* dq, int B, int H, int N, int d, const Bands& bands, int local_window, float scale,
                      float* dvec, const Packed& pk, hipStream_t stream);
int launch_bwd_dkdv_f32(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                        void* dv, int B, int H, int N, int d, const Bands& bands, int local_window, float scale,
                        float* dvec, const Packed& pk, hipStream_t stream);
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
  return launch_bwd_dq_f32(q, k, v, o, lse, dout, dq, B, H, N, d, bands, local_window, scale, dvec, pk, stream);
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
