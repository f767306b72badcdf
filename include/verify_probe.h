/*
 * verify_probe.h -- a plain streaming read on MI355X (gfx950), used only to
 * measure the read-stream ceiling that the verification kernels' KV-read
 * rate is quoted against (the same byte counts, read from HBM with 16-byte
 * loads by a full grid).  It computes nothing the method needs.
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

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_PROBE_H */
