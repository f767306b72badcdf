/*
 * verify_probe.h -- measurement aids on MI355X (gfx950) that compute nothing
 * the method needs: a plain streaming read, used only to measure the
 * read-stream ceiling that the verification kernels' KV-read rate is quoted
 * against (the same byte counts, read from HBM with 16-byte loads by a full
 * grid), and the phase records of the trace build.
 */
#ifndef VERIFY_PROBE_H
#define VERIFY_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "verify_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads bytes [0, bytes) of src once (16-byte loads, 1,024 workgroups of
 * 256 threads striding over the buffer) and folds them into an XOR that is
 * stored to *sink only if it equals a fixed constant (so the loads stay).
 *   src    device memory, 16-byte aligned; bytes a multiple of 16.
 *   sink   device uint32_t, written at most once.
 * Errors: VA_ERR_INVALID (NULL, misaligned or a size not a multiple of 16),
 * VA_ERR_HIP. */
va_status va_read_probe(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Phase trace -- exported only by the trace build of the library
 * (lib/libverify_attn_trace.so, compiled with VA_PHASE_TRACE; the product
 * library has no trace code).  There, lane 0 of a fixed wave of every
 * workgroup of split_kernel and combine_kernel stores the 100 MHz
 * constant-rate GPU clock (s_memrealtime, common to all CUs) at phase
 * boundaries into a per-workgroup record (24 uint64 for split_kernel, 8 for
 * combine_kernel) in a static device array; each launch overwrites the
 * records of the workgroups it runs
 * (workgroup index blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y *
 * blockIdx.z), at most 8,192: for split_kernel split + S * KV head, for
 * combine_kernel h + Hq * (row * D/32 + d slice)).
 *   split_kernel:   0 kernel entry, 1 arguments in registers, 2 first
 *                   producer wave has issued the first chunks' DMA, 3 chunk
 *                   0 in LDS (consumer wave 0 leaves its first barrier),
 *                   4 last step issued, 5 wave 0's partials written,
 *                   6 wave 0's clock ticks at the later barriers (a
 *                   duration), 7 the workgroup's chunk count (a count);
 *                   slots 3-6 of a workgroup without live rows in wave 0
 *                   are not written.  Durations, each over the chunks
 *                   after chunk 0: 8 + w consumer wave w's clock ticks at
 *                   the barriers (w < W; 8 equals 6); the first producer
 *                   wave's ticks waiting for its DMA (14) and at the
 *                   barriers (15); the first decoder wave's ticks at the
 *                   barriers (16) and converting (17; quantised caches
 *                   only); 18-23 unused.  The role that waits least at the
 *                   barriers holds each chunk's step.
 *   combine_kernel: 0 entry, 1 arguments in registers, 2 first batch of
 *                   partials in registers, 3 every batch folded, 4 output
 *                   written (thread 0; padding rows and invalid states
 *                   return before slot 2).
 * which = 0 (split) or 1 (combine); copies n_wg records (192 or 64 bytes
 * each) to host memory dst.  Returns 0, 1 for bad arguments, 2 for a HIP error.  The
 * records are the last writer's: run one launch, or read after a sequence
 * whose last launch is the one of interest. */
int va_trace_read(int which, uint64_t *dst, int n_wg);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_PROBE_H */
