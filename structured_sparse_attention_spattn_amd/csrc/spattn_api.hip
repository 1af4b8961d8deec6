// C ABI of the band-partitioned attention library (declared in spattn.h):
// argument checks, the Balanced Distance Partitioning band table, kernel
// dispatch, and the tile-list export that runs the forward kernel's own
// scheduling code on the device.
#include <math.h>

#include <mutex>

#include "common.h"

namespace spattn {
int launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                    const Bands& bands, int local_window, float scale, const Packed& pk, hipStream_t stream);
int launch_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   const Bands& bands, int local_window, float scale, const Packed& pk, hipStream_t stream);
int launch_decode(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* lengths, int B,
                  int H, int Nmax, int d, int dtype, const Bands& bands, int local_window, float scale,
                  hipStream_t stream);
void fwd_bf16_tiles(int d, int* BQ, int* BK);
void fwd_f32_tiles(int* BQ, int* BK);
WalkShape fwd_bf16_walk(int d);
WalkShape bwd_bf16_dq_walk();
WalkShape bwd_bf16_dkdv_walk();
WalkShape fwd_f32_walk(int B, int H, int N);
WalkShape bwd_f32_dq_walk(int B, int H, int N);
WalkShape bwd_f32_dkdv_walk(int B, int H, int N);
size_t bwd_workspace_bytes(int B, int H, int N, int d, int dtype, int grad_dtype);
int launch_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, int B, int H, int N, int d, int dtype, int grad_dtype, const Bands& bands,
                  int local_window, float scale, const Packed& pk, void* workspace, hipStream_t stream);
int launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                    void* dv, int B, int H, int N, int d, int dtype, int grad_dtype, const Bands& bands,
                    int local_window, float scale, const Packed& pk, void* workspace, hipStream_t stream);

constexpr Packed kFixed{nullptr, 0, 0};  // fixed-length [B, H, N, d] layout

namespace {

// Balanced Distance Partitioning ("Making Every Head Count", Figure 1
// caption): contiguous bands from distance 0, widths floor(N/H) or ceil(N/H),
// the wider ones first; heads past the first N get the empty band (N, N-1).
void bdp_table(int N, int H, int32_t* lo, int32_t* hi) {
  const int base = N / H, extra = N % H;
  int start = 0;
  for (int h = 0; h < H; ++h) {
    const int w = base + (h < extra ? 1 : 0);
    lo[h] = start;
    hi[h] = start + w - 1;
    start += w;
  }
}

int make_bands(int N, int H, const int32_t* blo, const int32_t* bhi, Bands* out) {
  if ((blo == nullptr) != (bhi == nullptr)) return SPATTN_E_ARG;
  if (blo == nullptr) {
    bdp_table(N, H, out->lo, out->hi);
    return SPATTN_OK;
  }
  for (int h = 0; h < H; ++h) {
    const int l = blo[h], u = bhi[h];
    if (l < 0 || u > N - 1 || l > u + 1) return SPATTN_E_ARG;
    out->lo[h] = l;
    out->hi[h] = u;
  }
  return SPATTN_OK;
}

int check_sizes(int B, int H, int N, int d, int dtype) {
  if (B < 1 || H < 1 || N < 1 || H > SPATTN_MAX_HEADS) return SPATTN_E_ARG;
  if (dtype != SPATTN_F32 && dtype != SPATTN_BF16) return SPATTN_E_UNSUPPORTED;
  if (d != 64 && d != 128) return SPATTN_E_UNSUPPORTED;
  if ((long long)B * H * N * d > (1LL << 40)) return SPATTN_E_ARG;
  return SPATTN_OK;
}

float resolve_scale(float scale, int d) { return scale > 0.f ? scale : 1.0f / sqrtf((float)d); }

// The kernels move tensor rows in 16-byte pieces and row vectors / index
// arrays in 4-byte ones: a null or misaligned pointer is an argument error.
bool tensor_ptr(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
bool vec_ptr(const void* p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }

// Query-major tile list of one band, computed with the forward kernel's
// scheduler (band_key_span + tile_full) by a single workgroup.
__global__ __launch_bounds__(256) void tile_list_kernel(int N, int lo, int hi, int BQ, int BK, int32_t* row_ptr,
                                                         int32_t* tiles, uint8_t* kind, int cap, int32_t* n_out) {
  const int n_qt = (N + BQ - 1) / BQ;
  for (int t = threadIdx.x; t < n_qt; t += blockDim.x) {
    const int i_min = t * BQ, i_max = min(N - 1, i_min + BQ - 1);
    const KeySpan s = band_key_span(i_min, i_max, lo, hi);
    row_ptr[t + 1] = s.last < s.first ? 0 : s.last / BK - s.first / BK + 1;
  }
  __syncthreads();
  __threadfence_block();
  if (threadIdx.x == 0) {
    int run = 0;
    row_ptr[0] = 0;
    for (int t = 0; t < n_qt; ++t) {
      run += row_ptr[t + 1];
      row_ptr[t + 1] = run;
    }
    *n_out = run;
  }
  __syncthreads();
  __threadfence_block();
  for (int t = threadIdx.x; t < n_qt; t += blockDim.x) {
    const int i_min = t * BQ, i_max = min(N - 1, i_min + BQ - 1);
    const KeySpan s = band_key_span(i_min, i_max, lo, hi);
    if (s.last < s.first) continue;
    int pos = row_ptr[t];
    for (int u = s.first / BK; u <= s.last / BK; ++u, ++pos) {
      if (pos >= cap) break;
      const int j0 = u * BK, j1 = min(N - 1, j0 + BK - 1);
      tiles[pos] = u;
      kind[pos] = tile_full(i_min, i_max, j0, j1, lo, hi) ? 0 : 1;
    }
  }
}

// Visit order of one band's walk in the CSR form of spattn_tile_walk, with
// the kernels' own walk builder (kernel_walk) and tile tests (set_full), by a
// single workgroup: owned tile t lists the tiles it visits, in visit order.
__global__ __launch_bounds__(256) void walk_list_kernel(WalkShape ws, int N, DistSet ds, int32_t* ptr,
                                                         int32_t* tiles, uint8_t* kind, int cap, int32_t* n_out) {
  const int n_own = (N + ws.own - 1) / ws.own;
  for (int t = threadIdx.x; t < n_own; t += blockDim.x) ptr[t + 1] = kernel_walk(ws, t * ws.own, N, ds).n;
  __syncthreads();
  __threadfence_block();
  if (threadIdx.x == 0) {
    int run = 0;
    ptr[0] = 0;
    for (int t = 0; t < n_own; ++t) {
      run += ptr[t + 1];
      ptr[t + 1] = run;
    }
    *n_out = run;
  }
  __syncthreads();
  __threadfence_block();
  for (int t = threadIdx.x; t < n_own; t += blockDim.x) {
    const int r0 = t * ws.own, r1 = min(N - 1, r0 + ws.own - 1);
    const TileWalk w = kernel_walk(ws, r0, N, ds);
    int pos = ptr[t];
    for (int v = 0; v < w.n && pos < cap; ++v, ++pos) {
      const int u = w.at(v);
      const int a0 = u * ws.tile, a1 = min(N - 1, a0 + ws.tile - 1);
      const bool full = ws.key_major ? set_full(a0, a1, r0, r1, ds) : set_full(r0, r1, a0, a1, ds);
      tiles[pos] = u;
      kind[pos] = full ? 0 : 1;
    }
  }
}

// Table of one of the "Making Every Head Count" Figure 2 attention patterns.
int pattern_table(int N, int H, int kind, int width, int32_t* lo, int32_t* hi) {
  switch (kind) {
    case SPATTN_PATTERN_BDP:
      bdp_table(N, H, lo, hi);
      return SPATTN_OK;
    case SPATTN_PATTERN_SLIDING_WINDOW: {
      // every head sees the same distances [0, w - 1]; w = 0 leaves them empty
      if (width < 0) return SPATTN_E_ARG;
      const int w = width < N ? width : N;
      for (int h = 0; h < H; ++h) {
        lo[h] = w == 0 ? N : 0;
        hi[h] = w == 0 ? N - 1 : w - 1;
      }
      return SPATTN_OK;
    }
    case SPATTN_PATTERN_GAPPED_HALF: {
      // the first floor(W_h / 2) distances of each head's partition band
      bdp_table(N, H, lo, hi);
      for (int h = 0; h < H; ++h) {
        const int half = (hi[h] - lo[h] + 1) / 2;
        if (half == 0) {
          lo[h] = N;
          hi[h] = N - 1;
        } else {
          hi[h] = lo[h] + half - 1;
        }
      }
      return SPATTN_OK;
    }
    case SPATTN_PATTERN_DENSE:
      for (int h = 0; h < H; ++h) {
        lo[h] = 0;
        hi[h] = N - 1;
      }
      return SPATTN_OK;
    default:
      return SPATTN_E_ARG;
  }
}

// Workspace of the allocation-free backward (spattn_bwd_noalloc): a static
// device array, one per GPU the library runs on, held until the process
// ends.  Host code never uses the array's name as an address: its device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[SPATTN_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPATTN_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SPATTN_E_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SPATTN_OK;
}

}  // namespace
}  // namespace spattn

using namespace spattn;

extern "C" {

int spattn_band_table(int32_t N, int32_t H, int32_t* lo, int32_t* hi) {
  if (N < 1 || H < 1 || H > SPATTN_MAX_HEADS || lo == nullptr || hi == nullptr) return SPATTN_E_ARG;
  bdp_table(N, H, lo, hi);
  return SPATTN_OK;
}

int spattn_band_table_pattern(int32_t N, int32_t H, int32_t kind, int32_t width, int32_t* lo, int32_t* hi) {
  if (N < 1 || H < 1 || H > SPATTN_MAX_HEADS || lo == nullptr || hi == nullptr) return SPATTN_E_ARG;
  return pattern_table(N, H, kind, width, lo, hi);
}

static int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t H,
                    int32_t N, int32_t d, int32_t dtype, const int32_t* band_lo, const int32_t* band_hi,
                    int32_t local_window, float scale, void* stream) {
  int st = check_sizes(B, H, N, d, dtype);
  if (st != SPATTN_OK) return st;
  if (!tensor_ptr(q) || !tensor_ptr(k) || !tensor_ptr(v) || !tensor_ptr(o) || !vec_ptr(lse) || local_window < 0)
    return SPATTN_E_ARG;
  Bands bands;
  st = make_bands(N, H, band_lo, band_hi, &bands);
  if (st != SPATTN_OK) return st;
  const float sc = resolve_scale(scale, d);
  const int w = local_window < N ? local_window : N;
  if (dtype == SPATTN_BF16)
    return launch_fwd_bf16(q, k, v, o, lse, B, H, N, d, bands, w, sc, kFixed, (hipStream_t)stream);
  return launch_fwd_f32(q, k, v, o, lse, B, H, N, d, bands, w, sc, kFixed, (hipStream_t)stream);
}

int spattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t H, int32_t N,
               int32_t d, int32_t dtype, const int32_t* band_lo, const int32_t* band_hi, float scale, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, dtype, band_lo, band_hi, 0, scale, stream);
}

int spattn_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t H,
                     int32_t N, int32_t d, int32_t dtype, const int32_t* band_lo, const int32_t* band_hi,
                     int32_t local_window, float scale, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, dtype, band_lo, band_hi, local_window, scale, stream);
}

size_t spattn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype, int32_t grad_dtype) {
  if (check_sizes(B, H, N, d, dtype) != SPATTN_OK) return 0;
  if (grad_dtype != SPATTN_F32 && grad_dtype != dtype) return 0;
  return bwd_workspace_bytes(B, H, N, d, dtype, grad_dtype);
}

// Shared checks of the backward entry points.
static int bwd_check(int B, int H, int N, int d, int dtype, int grad_dtype, const int32_t* band_lo,
                     const int32_t* band_hi, void* workspace, size_t workspace_bytes, Bands* bands) {
  int st = check_sizes(B, H, N, d, dtype);
  if (st != SPATTN_OK) return st;
  if (grad_dtype != SPATTN_F32 && grad_dtype != dtype) return SPATTN_E_UNSUPPORTED;
  st = make_bands(N, H, band_lo, band_hi, bands);
  if (st != SPATTN_OK) return st;
  const size_t need = bwd_workspace_bytes(B, H, N, d, dtype, grad_dtype);
  if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return SPATTN_E_WORKSPACE;
  return SPATTN_OK;
}

int spattn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype, int32_t grad_dtype,
                  const int32_t* band_lo, const int32_t* band_hi, float scale, void* workspace,
                  size_t workspace_bytes, void* stream) {
  Bands bands;
  int st = bwd_check(B, H, N, d, dtype, grad_dtype, band_lo, band_hi, workspace, workspace_bytes, &bands);
  if (st != SPATTN_OK) return st;
  if (!tensor_ptr(q) || !tensor_ptr(k) || !tensor_ptr(v) || !tensor_ptr(o) || !vec_ptr(lse) || !tensor_ptr(dout) ||
      !tensor_ptr(dq))
    return SPATTN_E_ARG;
  return launch_bwd_dq(q, k, v, o, lse, dout, dq, B, H, N, d, dtype, grad_dtype, bands, 0,
                       resolve_scale(scale, d), kFixed, workspace, (hipStream_t)stream);
}

int spattn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                    void* dv, int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype, int32_t grad_dtype,
                    const int32_t* band_lo, const int32_t* band_hi, float scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
  Bands bands;
  int st = bwd_check(B, H, N, d, dtype, grad_dtype, band_lo, band_hi, workspace, workspace_bytes, &bands);
  if (st != SPATTN_OK) return st;
  if (!tensor_ptr(q) || !tensor_ptr(k) || !tensor_ptr(v) || !vec_ptr(lse) || !tensor_ptr(dout) || !tensor_ptr(dk) ||
      !tensor_ptr(dv))
    return SPATTN_E_ARG;
  return launch_bwd_dkdv(q, k, v, lse, dout, dk, dv, B, H, N, d, dtype, grad_dtype, bands, 0,
                         resolve_scale(scale, d), kFixed, workspace, (hipStream_t)stream);
}

static int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                    void* dq, void* dk, void* dv, int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype,
                    int32_t grad_dtype, const int32_t* band_lo, const int32_t* band_hi, int32_t local_window,
                    float scale, void* workspace, size_t workspace_bytes, void* stream) {
  Bands bands;
  int st = bwd_check(B, H, N, d, dtype, grad_dtype, band_lo, band_hi, workspace, workspace_bytes, &bands);
  if (st != SPATTN_OK) return st;
  if (!tensor_ptr(q) || !tensor_ptr(k) || !tensor_ptr(v) || !tensor_ptr(o) || !vec_ptr(lse) || !tensor_ptr(dout) ||
      !tensor_ptr(dq) || !tensor_ptr(dk) || !tensor_ptr(dv) || local_window < 0)
    return SPATTN_E_ARG;
  const float sc = resolve_scale(scale, d);
  const int w = local_window < N ? local_window : N;
  st = launch_bwd_dq(q, k, v, o, lse, dout, dq, B, H, N, d, dtype, grad_dtype, bands, w, sc, kFixed, workspace,
                     (hipStream_t)stream);
  if (st != SPATTN_OK) return st;
  return launch_bwd_dkdv(q, k, v, lse, dout, dk, dv, B, H, N, d, dtype, grad_dtype, bands, w, sc, kFixed,
                         workspace, (hipStream_t)stream);
}

int spattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype,
               int32_t grad_dtype, const int32_t* band_lo, const int32_t* band_hi, float scale, void* workspace,
               size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, dtype, grad_dtype, band_lo, band_hi, 0, scale,
                  workspace, workspace_bytes, stream);
}

int spattn_bwd_local(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype,
                     int32_t grad_dtype, const int32_t* band_lo, const int32_t* band_hi, int32_t local_window,
                     float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, dtype, grad_dtype, band_lo, band_hi, local_window,
                  scale, workspace, workspace_bytes, stream);
}

int spattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, int32_t B, int32_t H, int32_t N, int32_t d,
                       int32_t dtype, int32_t grad_dtype, const int32_t* band_lo, const int32_t* band_hi, float scale,
                       void* stream) {
  // everything that needs no device first, so a bad call fails before any HIP call
  int st = check_sizes(B, H, N, d, dtype);
  if (st != SPATTN_OK) return st;
  if (grad_dtype != SPATTN_F32 && grad_dtype != dtype) return SPATTN_E_UNSUPPORTED;
  if (bwd_workspace_bytes(B, H, N, d, dtype, grad_dtype) > (size_t)SPATTN_NOALLOC_SCRATCH_BYTES)
    return SPATTN_E_WORKSPACE;
  if (!tensor_ptr(q) || !tensor_ptr(k) || !tensor_ptr(v) || !tensor_ptr(o) || !vec_ptr(lse) || !tensor_ptr(dout) ||
      !tensor_ptr(dq) || !tensor_ptr(dk) || !tensor_ptr(dv))
    return SPATTN_E_ARG;
  Bands bands;
  st = make_bands(N, H, band_lo, band_hi, &bands);
  if (st != SPATTN_OK) return st;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st != SPATTN_OK) return st;
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, dtype, grad_dtype, band_lo, band_hi, 0, scale, ws,
                  SPATTN_NOALLOC_SCRATCH_BYTES, stream);
}

// Packed variable-length batches: n_seqs sequences in [H, total, d] tensors
// (LSE [H, total]), sequence s at tokens cu_seqlens[s] .. cu_seqlens[s+1] - 1.
static int varlen_check(const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen, int32_t total, int32_t H,
                        int32_t d, int32_t dtype, const int32_t* band_lo, const int32_t* band_hi,
                        int32_t local_window, Bands* bands, Packed* pk) {
  if (cu_seqlens == nullptr || n_seqs < 1 || max_seqlen < 1 || total < 1 || local_window < 0) return SPATTN_E_ARG;
  int st = check_sizes(1, H, total, d, dtype);
  if (st != SPATTN_OK) return st;
  st = make_bands(max_seqlen, H, band_lo, band_hi, bands);
  if (st != SPATTN_OK) return st;
  pk->cu = cu_seqlens;
  pk->T = total;
  pk->own_bdp = band_lo == nullptr ? 1 : 0;
  return SPATTN_OK;
}

int spattn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
                      int32_t n_seqs, int32_t max_seqlen, int32_t total, int32_t H, int32_t d, int32_t dtype,
                      const int32_t* band_lo, const int32_t* band_hi, int32_t local_window, float scale,
                      void* stream) {
  Bands bands;
  Packed pk;
  int st = varlen_check(cu_seqlens, n_seqs, max_seqlen, total, H, d, dtype, band_lo, band_hi, local_window, &bands,
                        &pk);
  if (st != SPATTN_OK) return st;
  if (!tensor_ptr(q) || !tensor_ptr(k) || !tensor_ptr(v) || !tensor_ptr(o) || !vec_ptr(lse) || !vec_ptr(cu_seqlens))
    return SPATTN_E_ARG;
  const float sc = resolve_scale(scale, d);
  const int w = local_window < max_seqlen ? local_window : max_seqlen;
  if (dtype == SPATTN_BF16)
    return launch_fwd_bf16(q, k, v, o, lse, n_seqs, H, max_seqlen, d, bands, w, sc, pk, (hipStream_t)stream);
  return launch_fwd_f32(q, k, v, o, lse, n_seqs, H, max_seqlen, d, bands, w, sc, pk, (hipStream_t)stream);
}

int spattn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, const int32_t* cu_seqlens, int32_t n_seqs,
                      int32_t max_seqlen, int32_t total, int32_t H, int32_t d, int32_t dtype, int32_t grad_dtype,
                      const int32_t* band_lo, const int32_t* band_hi, int32_t local_window, float scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  Bands bands;
  Packed pk;
  int st = varlen_check(cu_seqlens, n_seqs, max_seqlen, total, H, d, dtype, band_lo, band_hi, local_window, &bands,
                        &pk);
  if (st != SPATTN_OK) return st;
  if (grad_dtype != SPATTN_F32 && grad_dtype != dtype) return SPATTN_E_UNSUPPORTED;
  const size_t need = bwd_workspace_bytes(1, H, total, d, dtype, grad_dtype);
  if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return SPATTN_E_WORKSPACE;
  if (!tensor_ptr(q) || !tensor_ptr(k) || !tensor_ptr(v) || !tensor_ptr(o) || !vec_ptr(lse) || !tensor_ptr(dout) ||
      !tensor_ptr(dq) || !tensor_ptr(dk) || !tensor_ptr(dv) || !vec_ptr(cu_seqlens))
    return SPATTN_E_ARG;
  const float sc = resolve_scale(scale, d);
  const int w = local_window < max_seqlen ? local_window : max_seqlen;
  st = launch_bwd_dq(q, k, v, o, lse, dout, dq, n_seqs, H, max_seqlen, d, dtype, grad_dtype, bands, w, sc, pk,
                     workspace, (hipStream_t)stream);
  if (st != SPATTN_OK) return st;
  return launch_bwd_dkdv(q, k, v, lse, dout, dk, dv, n_seqs, H, max_seqlen, d, dtype, grad_dtype, bands, w, sc, pk,
                         workspace, (hipStream_t)stream);
}

int spattn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                  const int32_t* lengths, int32_t B, int32_t H, int32_t Nmax, int32_t d, int32_t dtype,
                  const int32_t* band_lo, const int32_t* band_hi, int32_t local_window, float scale, void* stream) {
  int st = check_sizes(B, H, Nmax, d, dtype);
  if (st != SPATTN_OK) return st;
  if (!tensor_ptr(q) || !tensor_ptr(k_cache) || !tensor_ptr(v_cache) || !tensor_ptr(o) || !vec_ptr(lse) ||
      (lengths != nullptr && !vec_ptr(lengths)) || local_window < 0)
    return SPATTN_E_ARG;
  Bands bands;
  st = make_bands(Nmax, H, band_lo, band_hi, &bands);
  if (st != SPATTN_OK) return st;
  const int w = local_window < Nmax ? local_window : Nmax;
  return launch_decode(q, k_cache, v_cache, o, lse, lengths, B, H, Nmax, d, dtype, bands, w,
                       resolve_scale(scale, d), (hipStream_t)stream);
}

int spattn_kernel_tiles(int32_t d, int32_t dtype, int32_t* BQ, int32_t* BK) {
  if (!BQ || !BK) return SPATTN_E_ARG;
  if (d != 64 && d != 128) return SPATTN_E_UNSUPPORTED;
  int bq, bk;
  if (dtype == SPATTN_BF16)
    fwd_bf16_tiles(d, &bq, &bk);
  else if (dtype == SPATTN_F32)
    fwd_f32_tiles(&bq, &bk);
  else
    return SPATTN_E_UNSUPPORTED;
  *BQ = bq;
  *BK = bk;
  return SPATTN_OK;
}

int spattn_tile_list(int32_t N, int32_t lo, int32_t hi, int32_t BQ, int32_t BK, int32_t* row_ptr, int32_t* tiles,
                     uint8_t* kind, int32_t cap, int32_t* n_out, void* stream) {
  if (N < 1 || BQ < 0 || BK < 0 || cap < 0 || !row_ptr || !n_out || (cap > 0 && (!tiles || !kind)))
    return SPATTN_E_ARG;
  if (lo < 0 || hi > N - 1 || lo > hi + 1) return SPATTN_E_ARG;
  if (BQ == 0 || BK == 0) {
    if (BQ != BK) return SPATTN_E_ARG;
    fwd_bf16_tiles(128, &BQ, &BK);
  }
  hipLaunchKernelGGL(tile_list_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, N, lo, hi, BQ, BK, row_ptr,
                     tiles, kind, cap, n_out);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

int spattn_tile_walk(int32_t kernel, int32_t d, int32_t dtype, int32_t B, int32_t H, int32_t N, int32_t lo,
                     int32_t hi, int32_t local_window, int32_t* ptr, int32_t* tiles, uint8_t* kind, int32_t cap,
                     int32_t* n_out, int32_t* own_rows, int32_t* tile_rows, void* stream) {
  if (B < 1 || H < 1 || N < 1 || cap < 0 || local_window < 0 || !ptr || !n_out ||
      (cap > 0 && (!tiles || !kind)))
    return SPATTN_E_ARG;
  if (d != 64 && d != 128) return SPATTN_E_UNSUPPORTED;
  if (lo < 0 || hi > N - 1 || lo > hi + 1) return SPATTN_E_ARG;
  WalkShape ws;
  if (dtype == SPATTN_BF16) {
    if (kernel == SPATTN_KERNEL_FWD)
      ws = fwd_bf16_walk(d);
    else if (kernel == SPATTN_KERNEL_BWD_DQ)
      ws = bwd_bf16_dq_walk();
    else if (kernel == SPATTN_KERNEL_BWD_DKDV)
      ws = bwd_bf16_dkdv_walk();
    else
      return SPATTN_E_ARG;
  } else if (dtype == SPATTN_F32) {
    if (kernel == SPATTN_KERNEL_FWD)
      ws = fwd_f32_walk(B, H, N);
    else if (kernel == SPATTN_KERNEL_BWD_DQ)
      ws = bwd_f32_dq_walk(B, H, N);
    else if (kernel == SPATTN_KERNEL_BWD_DKDV)
      ws = bwd_f32_dkdv_walk(B, H, N);
    else
      return SPATTN_E_ARG;
  } else {
    return SPATTN_E_UNSUPPORTED;
  }
  if (own_rows) *own_rows = ws.own;
  if (tile_rows) *tile_rows = ws.tile;
  const int w = local_window < N ? local_window : N;
  hipLaunchKernelGGL(walk_list_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, ws, N, dist_set(lo, hi, w), ptr,
                     tiles, kind, cap, n_out);
  return hipGetLastError() == hipSuccess ? SPATTN_OK : SPATTN_E_HIP;
}

const char* spattn_status_string(int status) {
  switch (status) {
    case SPATTN_OK:
      return "ok";
    case SPATTN_E_ARG:
      return "invalid argument";
    case SPATTN_E_UNSUPPORTED:
      return "unsupported head size or dtype";
    case SPATTN_E_HIP:
      return "HIP launch error";
    case SPATTN_E_WORKSPACE:
      return "workspace missing or too small";
    default:
      return "unknown status";
  }
}

}  // extern "C"
