/*
 * spattn_probe.h -- microbenchmarks that measure the MI355X denominators the
 * benchmark reports next to the published ones (libspattn_probe.so, separate
 * from the attention library).  Not part of the attention ABI.
 *
 * Every call launches one kernel on `stream` (a hipStream_t as void*, NULL =
 * the null stream) and returns 0 on success, 1 for bad arguments, 3 if the
 * launch failed.  Timing is the caller's (events around the call).
 */
#ifndef SPATTN_PROBE_H
#define SPATTN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Matrix-core throughput: `blocks` workgroups of 4 waves, each wave issuing
 * `iters` rounds of 4 independent 32x32 MFMA products (kind 0:
 * v_mfma_f32_32x32x16_bf16, 32768 FLOP each; kind 1: v_mfma_f32_32x32x2_f32,
 * 4096 FLOP each) from registers.  The accumulators are summed into
 * sink[blocks * 256] (device float32, written) so nothing is optimised away.
 * FLOP of the launch: blocks * 4 * iters * 4 * (32768 or 4096).
 */
int spattn_probe_mfma(int32_t kind, int32_t blocks, int32_t iters, float* sink, void* stream);

/*
 * HBM read bandwidth: `blocks` workgroups of 256 lanes read `bytes` bytes
 * (a multiple of 16) of the device buffer src with 16-byte loads in a
 * grid-stride loop and write one float32 per lane to sink[blocks * 256].
 */
int spattn_probe_read(const void* src, size_t bytes, int32_t blocks, float* sink, void* stream);

/*
 * LDS read bandwidth: `blocks` workgroups of 4 waves with a 32 KB LDS
 * buffer each; every wave reads 8 KB per iteration for `iters` iterations in
 * conflict-free 16-byte (kind 0: ds_read_b128) or 8-byte (kind 1: the
 * transposing ds_read_b64_tr_b16) lane reads, and one float32 per lane goes
 * to sink[blocks * 256].  Bytes of the launch: blocks * 4 * iters * 8192.
 */
int spattn_probe_lds(int32_t kind, int32_t blocks, int32_t iters, float* sink, void* stream);

/*
 * float32 atomic-add throughput: `blocks` workgroups of 256 lanes each issue
 * `iters` atomic adds of 1.0 without return (global_atomic_add_f32) into the
 * device buffer dst of n_floats floats (a power of two, at least 256; dst
 * 256-byte aligned), lane l of the launch at float (l + k * blocks * 256) mod
 * n_floats in its k-th add, so every wave instruction covers 256 contiguous
 * bytes.
 * dst is modified.  Bytes added by the launch: blocks * 256 * iters * 4.
 */
int spattn_probe_atomic(float* dst, size_t n_floats, int32_t blocks, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPATTN_PROBE_H */
