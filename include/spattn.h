/*
 * spattn.h -- C ABI of the band-partitioned (SPAttention) attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method ("Making Every Head Count: Sparse Attention Without the
 * Speed-Performance Trade-off", abstract and Figure 1 caption): Balanced
 * Distance Partitioning cuts the causal distance spectrum d = i - j in
 * [0, N-1] into H contiguous, non-overlapping bands of width floor(N/H) or
 * ceil(N/H), head 0 nearest; head h runs ordinary softmax attention over only
 * the keys whose distance lies in its band.  The per-head rule is the
 * masked-set sparse-attention formula ("Story of Attention -- Part 4: Sparse
 * Attention, Then and Now", section 1): the attention formula is unchanged,
 * only the key set the softmax runs over is restricted.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every function returns an int status (enum spattn_status); nothing throws
 *   across this boundary.
 * - Tensors are caller-owned DEVICE pointers to contiguous row-major
 *   [B, H, N, d] arrays (batch, head, position, feature), 16-byte aligned
 *   (rows are moved in 16-byte pieces).  LSE is [B, H, N] float32; LSE,
 *   decode lengths and cu_seqlens are 4-byte aligned.  A null or misaligned
 *   pointer is SPATTN_E_ARG.  Band arrays are HOST pointers.
 * - dtype codes: SPATTN_F32 = 0 (float32 everywhere), SPATTN_BF16 = 1
 *   (bfloat16 storage, float32 accumulation).  Head size d must be 64 or 128.
 * - stream is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *   are asynchronous: the status covers argument checks and the launch only;
 *   faults during execution surface at the caller's next synchronisation.
 * - The library allocates no device memory.  Apart from the workspace array
 *   of spattn_bwd_noalloc (see there) it keeps no mutable global state, so
 *   calls on different streams may run concurrently.
 * - Score scale: scale <= 0 selects 1/sqrt(d).
 * - A query row whose key set is empty gets output 0 and LSE = -inf; it and
 *   any key no query reaches get zero gradients.
 */
#ifndef SPATTN_H
#define SPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum spattn_status {
  SPATTN_OK = 0,
  SPATTN_E_ARG = 1,          /* null or misaligned pointer, size out of range, bad band */
  SPATTN_E_UNSUPPORTED = 2,  /* head size / dtype combination not built */
  SPATTN_E_HIP = 3,          /* the HIP runtime refused the launch */
  SPATTN_E_WORKSPACE = 4     /* backward workspace too small */
};

enum spattn_dtype { SPATTN_F32 = 0, SPATTN_BF16 = 1 };

/* Largest head count a call accepts (band bounds travel in the kernel
 * argument block). */
#define SPATTN_MAX_HEADS 256

/* Attention patterns of spattn_band_table_pattern. */
enum spattn_pattern {
  SPATTN_PATTERN_BDP = 0,             /* Balanced Distance Partitioning (the method) */
  SPATTN_PATTERN_SLIDING_WINDOW = 1,  /* every head: distances [0, width - 1] */
  SPATTN_PATTERN_GAPPED_HALF = 2,     /* first half of each partition band */
  SPATTN_PATTERN_DENSE = 3            /* every head: [0, N - 1], dense causal */
};

/* Kernels whose tile walk spattn_tile_walk reports. */
enum spattn_kernel {
  SPATTN_KERNEL_FWD = 0,      /* forward: query-major */
  SPATTN_KERNEL_BWD_DQ = 1,   /* first backward stage (D and dQ): query-major */
  SPATTN_KERNEL_BWD_DKDV = 2  /* second backward stage (dK, dV): key-major */
};

/*
 * Band table of Balanced Distance Partitioning ("Making Every Head Count",
 * Figure 1 caption).  Host only, no GPU needed.
 *   N  sequence length (>= 1); H number of heads (1 .. SPATTN_MAX_HEADS).
 *   lo, hi  caller-owned host arrays of H int32; on return head h covers the
 *           distances lo[h] .. hi[h] inclusive.  Bands are contiguous from
 *           distance 0, the first N mod H heads get width ceil(N/H), the rest
 *           floor(N/H).  When H > N the heads beyond the first N get an empty
 *           band, written as lo = N, hi = N - 1.
 * Errors: SPATTN_E_ARG if N < 1, H < 1, H > SPATTN_MAX_HEADS or a pointer is
 * NULL (outputs untouched).
 */
int spattn_band_table(int32_t N, int32_t H, int32_t* lo, int32_t* hi);

/*
 * Band tables of the attention patterns that "Making Every Head Count"
 * compares in its Figure 2 caption, for use as band_lo / band_hi of the
 * other calls.  Host only.
 *   kind  SPATTN_PATTERN_BDP: the partition itself (as spattn_band_table).
 *         SPATTN_PATTERN_SLIDING_WINDOW: every head restricted to the same
 *           local window, distances [0, w - 1] with w = min(width, N); the
 *           page gives no width.  width = 0 gives every head an empty band.
 *         SPATTN_PATTERN_GAPPED_HALF: each head keeps only the first half of
 *           its partition band, floor(W_h / 2) distances from lo_h (the
 *           rounding is not on the page); a width-1 band becomes empty.
 *         SPATTN_PATTERN_DENSE: every head [0, N - 1], dense causal attention
 *           (the baseline the method is compared against).
 *   width used by SPATTN_PATTERN_SLIDING_WINDOW only (>= 0).
 *   lo, hi  caller-owned host arrays of H int32; an empty band is written
 *           lo = N, hi = N - 1.
 * Errors: SPATTN_E_ARG for N < 1, H outside 1 .. SPATTN_MAX_HEADS, a NULL
 * pointer, an unknown kind or a negative sliding-window width.
 */
int spattn_band_table_pattern(int32_t N, int32_t H, int32_t kind, int32_t width,
                              int32_t* lo, int32_t* hi);

/*
 * Forward pass: for every (b, h, i), with S = { j : lo_h <= i - j <= hi_h,
 * 0 <= j <= i },
 *     o[b,h,i,:] = sum_{j in S} softmax_j(scale * q_i . k_j) v_j
 *     lse[b,h,i] = ln sum_{j in S} exp(scale * q_i . k_j)
 * (the masked-set formula of "Sparse Attention, Then and Now", section 1,
 * over the band of "Making Every Head Count", Figure 1).
 *   q, k, v  device, [B,H,N,d] of dtype, read only.
 *   o        device, [B,H,N,d] of dtype, written (every row, empty rows = 0).
 *   lse      device, [B,H,N] float32, written (-inf for empty rows).
 *   band_lo, band_hi  host, H int32 each, or both NULL for the Balanced
 *            Distance Partitioning table of (N, H).  Any bands with
 *            0 <= lo <= hi + 1 and hi <= N - 1 are accepted (lo = hi + 1 is an
 *            empty band), so one band [0, N-1] per head is dense causal
 *            attention in the same kernels.
 * Errors: SPATTN_E_ARG (null tensor, B/H/N < 1, H > SPATTN_MAX_HEADS, bad
 * band), SPATTN_E_UNSUPPORTED (d not 64/128, unknown dtype), SPATTN_E_HIP.
 */
int spattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
               int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype,
               const int32_t* band_lo, const int32_t* band_hi, float scale,
               void* stream);

/*
 * Bytes of device workspace spattn_bwd needs for these sizes: two float32
 * row vectors [B,H,N], each rounded up to 256 bytes: -D_i = -dO_i . O_i,
 * then -LSE_i log2(e), the exponent offset the bfloat16 dK/dV kernel
 * recomputes P with (the float32 kernels leave the second vector unused).
 * grad_dtype (SPATTN_F32 or dtype, as in spattn_bwd) is part of the query so
 * that a gradient type needing more workspace can be added without a new
 * call; every current combination needs the same two vectors.
 * Returns 0 for invalid sizes or an unsupported grad_dtype.
 */
size_t spattn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d,
                                  int32_t dtype, int32_t grad_dtype);

/*
 * Backward pass of spattn_fwd (the textbook derivative of the masked-set
 * formula; no page gives one): with P the band-restricted softmax recomputed
 * from the saved lse, D_i = dO_i . O_i and dS = P * (dO V^T - D),
 *     dq = scale * dS K,   dk = scale * dS^T Q,   dv = P^T dO.
 *   q, k, v, o, dout  device [B,H,N,d] of dtype, read only (o and lse from
 *            spattn_fwd with the same bands).
 *   lse      device [B,H,N] float32.
 *   dq, dk, dv  device [B,H,N,d], written completely; element type float32
 *            if grad_dtype == SPATTN_F32, else dtype.
 *   grad_dtype  SPATTN_F32 or the input dtype.
 *   workspace   device, >= spattn_bwd_workspace_bytes(...) bytes, 256-byte
 *            aligned, caller-owned, contents need not be initialised.
 * The result is deterministic: dq is produced by a query-major pass and dk,
 * dv by a key-major pass, with no atomics.
 * Errors: as spattn_fwd, plus SPATTN_E_WORKSPACE if workspace is NULL or too
 * small.
 */
int spattn_bwd(const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dout, void* dq, void* dk, void* dv,
               int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype,
               int32_t grad_dtype, const int32_t* band_lo, const int32_t* band_hi,
               float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Band attention with a shared local window ("Making Every Head Count",
 * Figure 2 caption: its exclusive-band ablation is the method with the local
 * sharing removed; the page gives no window width).  Head h attends
 *     S = { j : 0 <= j <= i, lo_h <= i - j <= hi_h  or  i - j < local_window }
 * i.e. its band joined with the distances [0, local_window - 1] that every
 * head shares.  local_window = 0 is exactly spattn_fwd / spattn_bwd; widths
 * above N act as N.  Arguments, outputs and errors as spattn_fwd and
 * spattn_bwd, plus SPATTN_E_ARG for local_window < 0.  Both dtypes.
 */
int spattn_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                     int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype,
                     const int32_t* band_lo, const int32_t* band_hi,
                     int32_t local_window, float scale, void* stream);
int spattn_bwd_local(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype,
                     int32_t grad_dtype, const int32_t* band_lo, const int32_t* band_hi,
                     int32_t local_window, float scale, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Packed variable-length batches.  n_seqs sequences of different lengths are
 * stored back to back along the token axis: q, k, v, o, dout, dq, dk, dv are
 * [H, total, d] and lse is [H, total] (the [B, H, N, d] layout with B = 1 and
 * N = total).  Sequence s owns tokens cu_seqlens[s] .. cu_seqlens[s+1] - 1,
 * and positions restart at 0 in every sequence.  Attention never crosses a
 * sequence boundary: token i of sequence s attends the keys j of s with
 * i - j in its head's set, as in spattn_fwd_local.
 *   cu_seqlens  device int32 [n_seqs + 1], non-decreasing, cu_seqlens[0] = 0,
 *               cu_seqlens[n_seqs] = total.  Read by the kernels, not by the
 *               host, so a malformed array is not reported; the kernels clamp
 *               every sequence to tokens [0, total) and to max_seqlen, so they
 *               never index outside the tensors, but the rows of tokens that
 *               no valid sequence covers are then left unwritten.
 *   max_seqlen  an upper bound on every sequence's length.  It sizes the
 *               grid, and tokens past it in a longer sequence are not computed.
 *   band_lo, band_hi  host, H int32 each, validated against max_seqlen as in
 *               spattn_fwd and clipped to each sequence's length; or both
 *               NULL for each sequence's own Balanced Distance Partitioning
 *               table ("Making Every Head Count", Figure 1 caption: the bands
 *               partition the distances of that sequence).
 *   local_window  >= 0 as in spattn_fwd_local.
 * The backward workspace is spattn_bwd_workspace_bytes(1, H, total, d, dtype,
 * grad_dtype) bytes.  Both dtypes; d in {64, 128}.
 * Errors: SPATTN_E_ARG for NULL pointers, n_seqs, max_seqlen or total < 1, or
 * local_window < 0, and otherwise as spattn_fwd / spattn_bwd.
 */
int spattn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                      int32_t total, int32_t H, int32_t d, int32_t dtype,
                      const int32_t* band_lo, const int32_t* band_hi,
                      int32_t local_window, float scale, void* stream);
int spattn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                      int32_t total, int32_t H, int32_t d, int32_t dtype, int32_t grad_dtype,
                      const int32_t* band_lo, const int32_t* band_hi, int32_t local_window,
                      float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode step: one new query per sequence against a key/value cache.  For
 * sequence b with L_b valid cache rows the query sits at position
 * i = L_b - 1 and head h attends
 *     S = { j : 0 <= j <= i, lo_h <= i - j <= hi_h  or  i - j < local_window }
 * through the same masked-set softmax as spattn_fwd (the method's formula
 * evaluated for the newest query; the pages measure training only).
 *   q        device [B,H,d] of dtype; o device [B,H,d] of dtype, written.
 *   k_cache, v_cache  device [B,H,Nmax,d] of dtype, rows 0 .. L_b - 1 read.
 *   lse      device [B,H] float32, written (-inf for an empty set).
 *   lengths  device [B] int32 (values clamped to 0 .. Nmax; 0 gives o = 0,
 *            lse = -inf), or NULL for L_b = Nmax.
 *   band_lo, band_hi  host, H int32 each (validated against Nmax as in
 *            spattn_fwd), or both NULL for the Balanced Distance Partitioning
 *            table of (Nmax, H).
 *   local_window  >= 0, as in spattn_fwd_local; float32 and bfloat16 both.
 * Errors: as spattn_fwd, plus SPATTN_E_ARG for local_window < 0.
 */
int spattn_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                  float* lse, const int32_t* lengths, int32_t B, int32_t H, int32_t Nmax,
                  int32_t d, int32_t dtype, const int32_t* band_lo, const int32_t* band_hi,
                  int32_t local_window, float scale, void* stream);

/*
 * The two stages spattn_bwd runs, exported for callers that schedule them
 * separately (and for per-kernel timing).  Same arguments and checks as
 * spattn_bwd; together they compute exactly what spattn_bwd computes.
 *   spattn_bwd_dq    writes -D_i = -dO_i . O_i (and, for bfloat16 inputs,
 *                    -LSE_i log2(e)) into the workspace, and dq.
 *   spattn_bwd_dkdv  reads them from the workspace and writes dk, dv; it must run
 *                    after spattn_bwd_dq with the same workspace, bands and
 *                    inputs, on the same stream (or after a synchronisation).
 */
int spattn_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, void* dq,
                  int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype,
                  int32_t grad_dtype, const int32_t* band_lo, const int32_t* band_hi,
                  float scale, void* workspace, size_t workspace_bytes, void* stream);

int spattn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                    const void* dout, void* dk, void* dv,
                    int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype,
                    int32_t grad_dtype, const int32_t* band_lo, const int32_t* band_hi,
                    float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tile sizes the forward kernel schedules with for (d, dtype): BQ query rows
 * per workgroup and BK key rows per LDS stage.  Host only.  Float32 launches
 * with fewer than 512 tiles of 128 query rows (B * H * ceil(N / 128))
 * instead take 32-row tiles whose key tiles are split over the workgroup's
 * waves; the values returned here are those of the larger launches.
 * Errors: SPATTN_E_ARG for NULL outputs, SPATTN_E_UNSUPPORTED otherwise.
 */
int spattn_kernel_tiles(int32_t d, int32_t dtype, int32_t* BQ, int32_t* BK);

/*
 * Test export of the band-tile schedule: runs, on the device, the same
 * scheduling code the forward kernel uses, for one band [lo, hi] of a
 * length-N sequence, and writes the query-major tile list in CSR form:
 *   row_ptr  device int32 [ceil(N/BQ) + 1]
 *   tiles    device int32 [cap]   key-tile indices u, ascending per query tile
 *   kind     device uint8 [cap]   0 = FULL (every pair in band), 1 = PARTIAL
 *   n_out    device int32 [1]     total number of listed tiles
 * BQ = BK = 0 selects the forward kernel's own sizes for (d = 128, bf16).
 * If the list is longer than cap, n_out still holds the full count and only
 * the first cap entries are written.  A query tile t meets key tile u iff
 * some pair (i, j) in them has j <= i < N and lo <= i - j <= hi.
 * Errors: SPATTN_E_ARG (null pointers, N < 1, BQ or BK < 0, band outside
 * [0, N-1]), SPATTN_E_HIP.
 */
int spattn_tile_list(int32_t N, int32_t lo, int32_t hi, int32_t BQ, int32_t BK,
                     int32_t* row_ptr, int32_t* tiles, uint8_t* kind, int32_t cap,
                     int32_t* n_out, void* stream);

/*
 * Test export of a kernel's actual tile walk: for one band [lo, hi] (with
 * the shared local window as in spattn_fwd_local) of a length-N sequence,
 * runs on the device the walk builder and tile test the chosen kernel runs,
 * for the launch that B sequences of H heads with head size d would make (the
 * float32 kernels pick their tile shape by launch size, the bfloat16 forward
 * by head size).  Output in CSR form over the tiles
 * the kernel owns (query tiles for SPATTN_KERNEL_FWD and _BWD_DQ, key tiles
 * for SPATTN_KERNEL_BWD_DKDV):
 *   ptr    device int32 [ceil(N / own_rows) + 1]
 *   tiles  device int32 [cap]  indices of the visited tiles of the other
 *          operand, in the kernel's visit order (at most two ascending runs,
 *          a single run possibly rotated so that neighbouring workgroups read
 *          a shared tile at the same step)
 *   kind   device uint8 [cap]  0 = FULL (every pair of the two tiles is in
 *          the head's set), 1 = PARTIAL
 *   n_out  device int32 [1]    total number of visits
 *   own_rows, tile_rows  host int32, optional (NULL): rows of an owned tile
 *          and of a visited tile.
 * The visited tiles of an owned tile are exactly those in which some pair
 * (i, j), j <= i < N, has i - j in the head's set.  If the list is longer
 * than cap, n_out holds the full count and the first cap entries are written.
 * Errors: SPATTN_E_ARG (unknown kernel, null pointers, B, H or N < 1, band
 * outside [0, N-1], local_window < 0), SPATTN_E_UNSUPPORTED (dtype, d not
 * 64 / 128), SPATTN_E_HIP.
 */
int spattn_tile_walk(int32_t kernel, int32_t d, int32_t dtype, int32_t B, int32_t H, int32_t N,
                     int32_t lo, int32_t hi, int32_t local_window, int32_t* ptr,
                     int32_t* tiles, uint8_t* kind, int32_t cap, int32_t* n_out,
                     int32_t* own_rows, int32_t* tile_rows, void* stream);

/*
 * Size of the device array that spattn_bwd_noalloc uses as its workspace
 * (16 MiB per GPU): spattn_bwd_workspace_bytes(B, H, N, d, dtype, grad_dtype)
 * must not exceed it, i.e. B * H * N <= 2,097,152 rows (two float32 row
 * vectors, each rounded up to 256 bytes).
 */
#define SPATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * spattn_bwd for callers that cannot allocate device memory (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, same arguments minus the workspace, which
 * is a static array of SPATTN_NOALLOC_SCRATCH_BYTES in the library's device
 * code instead of a caller buffer.  Each GPU the library runs on holds its
 * own copy of that array until the process ends; its device address is
 * looked up on the first call on a device (with that device current) and
 * reused.  The call allocates nothing and needs no cleared memory (the first
 * stage writes every value the second reads).  All calls on one GPU share
 * its array: calls that overlap in time on one GPU (other streams, other host
 * threads) race on it and must be serialised by the caller.
 * Errors: as spattn_bwd; SPATTN_E_WORKSPACE when the sizes need more than
 * SPATTN_NOALLOC_SCRATCH_BYTES (checked before any device call);
 * SPATTN_E_HIP if the array's address cannot be obtained.
 */
int spattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype,
                       int32_t grad_dtype, const int32_t* band_lo, const int32_t* band_hi,
                       float scale, void* stream);

/* Static description of a status code (never NULL). */
const char* spattn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPATTN_H */
