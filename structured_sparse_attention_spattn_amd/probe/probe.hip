// Microbenchmarks for the measured denominators (declared in spattn_probe.h):
// matrix-core throughput of the two MFMA shapes the kernels use, the HBM
// read bandwidth of plain 16-byte loads, the LDS read bandwidth of the two
// LDS read forms the kernels use, and the throughput of float32 atomic adds
// into device memory (what a backward accumulating dQ with atomics needs).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spattn_probe.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Four independent accumulator chains per wave, operands from registers.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  if constexpr (KIND == 0) {
    bf16x8 a, b;
    for (int j = 0; j < 8; ++j) {
      a[j] = (__bf16)(1e-3f * (float)(lane + j));
      b[j] = (__bf16)(1e-3f * (float)(lane - j));
    }
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  } else {
    const float a = 1e-3f * (float)lane, b = 1e-3f * (float)(64 - lane);
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c3, 0, 0, 0);
    }
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_probe_kernel(const f32x4* __restrict__ src, size_t n, float* sink) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) acc += src[i];
  sink[blockIdx.x * 256 + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// LDS reads from a 32 KB workgroup buffer: every wave reads 8 KB per
// iteration, each read instruction a contiguous 1 KB (KIND 0: ds_read_b128)
// or 512 B (KIND 1: ds_read_b64_tr_b16) block, so no bank conflicts.  The
// block offset moves with the iteration so no read is loop-invariant.
template <int KIND>
__global__ __launch_bounds__(256) void lds_probe_kernel(int iters, float* sink) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[8192];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < 8192; i += 256) buf[i] = (uint32_t)(i * 2654435761u);
  __syncthreads();
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    const int base = ((it * 7 + wave * 3) & 3) * 8192;  // byte offset of an 8 KB quarter
    if constexpr (KIND == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const u32x4 v = *(const u32x4*)((const char*)buf + ((base + k * 1024 + lane * 16) & 32767));
        acc ^= v[0] + v[1] + v[2] + v[3];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const char* ptr = (const char*)buf + ((base + k * 512 + lane * 8) & 32767);
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)ptr);
        acc ^= (uint32_t)(v[0] + v[1] + v[2] + v[3]);
      }
    }
  }
  sink[blockIdx.x * 256 + tid] = (float)acc;
}

// float32 atomic adds without return (global_atomic_add_f32), each wave
// adding to 64 consecutive floats (256 B) per instruction, the lanes of the
// launch covering the buffer in a grid-stride pattern that wraps around.
// n is a power of two: the wrap is a mask.
__global__ __launch_bounds__(256) void atomic_probe_kernel(float* dst, size_t n, int iters) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int it = 0; it < iters; ++it) {
    unsafeAtomicAdd(dst + (i & (n - 1)), 1.0f);
    i += stride;
  }
}

}  // namespace

extern "C" {

int spattn_probe_mfma(int32_t kind, int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (blocks < 1 || iters < 1 || sink == nullptr || (kind != 0 && kind != 1)) return 1;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int spattn_probe_read(const void* src, size_t bytes, int32_t blocks, float* sink, void* stream) {
  if (src == nullptr || sink == nullptr || blocks < 1 || bytes % 16 != 0 || ((uintptr_t)src & 15u) != 0) return 1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const f32x4*)src,
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int spattn_probe_lds(int32_t kind, int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (blocks < 1 || iters < 1 || sink == nullptr || (kind != 0 && kind != 1)) return 1;
  if (kind == 0)
    hipLaunchKernelGGL(lds_probe_kernel<0>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  else
    hipLaunchKernelGGL(lds_probe_kernel<1>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int spattn_probe_atomic(float* dst, size_t n_floats, int32_t blocks, int32_t iters, void* stream) {
  if (dst == nullptr || n_floats < 256 || (n_floats & (n_floats - 1)) != 0 || blocks < 1 || iters < 1 ||
      ((uintptr_t)dst & 255u) != 0)
    return 1;
  hipLaunchKernelGGL(atomic_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, dst, n_floats, iters);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
