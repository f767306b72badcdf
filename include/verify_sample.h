/*
 * verify_sample.h -- C ABI for the step after verification on MI355X
 * (gfx950): top-k / top-p sampling of the verification rows and rejection
 * acceptance of the drafts.
 *
 * What is computed (IQuestRT report, section "Include sampling and acceptance
 * in the execution path"; the top-k search follows section "Parallelize the
 * Top-K vocabulary scan"):
 *
 *   Sampling, per row r of FP32 logits z (vocabulary V):
 *     candidates  the top_k token ids by logit, equal logits by lower id
 *                 first (top_k > V keeps all V);
 *     p_i         = e^{(z_i - z_0)/T} / sum_j e^{(z_j - z_0)/T} over the
 *                 candidates, z_0 the largest, T the temperature;
 *     top-p       candidate i is kept iff p_i > 0 and sum_{j<i} p_j < top_p
 *                 (the shortest prefix reaching top_p; at least one);
 *                 kept probabilities are renormalised;
 *     draw        u from the counter generator below at (first_position + r,
 *                 purpose); the token is the first kept candidate i with
 *                 u * sum(kept e) < e_0 + ... + e_i (the last kept one if
 *                 rounding leaves none).
 *
 *   Acceptance of n - 1 drafts d_1..d_{n-1} against the n sampled rows
 *   (row 0 is the committed token; row i draws the token at position
 *   first_position + i):
 *     draft d_{i+1} is accepted iff u * q_i(d) < p_i(d), u at (first_position
 *     + i, purpose 1), p_i the target row's kept list, q_i the draft's own
 *     kept list (the distribution it sampled from), both zero outside their
 *     lists;
 *     at the first rejection, at row i, the replacement is drawn from
 *     max(0, p_i(t) - q_i(t)) over row i's kept tokens, u at (first_position
 *     + i, purpose 2); a zero residual (rounding only) gives row i's own
 *     sample;
 *     with every draft accepted the bonus is row n-1's own sample.
 *     Output: the accepted count a (0..n-1) and a + 1 tokens d_1..d_a, then
 *     the replacement or the bonus.
 *
 *   Random numbers: Philox4x32-10 (Salmon et al., "Parallel random numbers:
 *   as easy as 1, 2, 3", SC'11) with key (seed low 32 bits, seed high 32
 *   bits) and counter (position low, position high, purpose, 0); the first
 *   output word x gives u = (x >> 8) * 2^-24.  Equal seeds and positions give
 *   equal draws on every GPU, so no draw needs to be broadcast.
 *
 * Conventions: as in verify_attn.h (caller-owned device memory, no
 * allocation or synchronisation, asynchronous on `stream`, a va_status
 * return).  Probabilities are computed in FP32; a kept count, a drawn index
 * or an accept bit whose deciding quantity lies within FP32 rounding of its
 * threshold may differ from an exact computation.  Logits must be finite or
 * -inf, with at least one finite logit per row (a NaN logit or an all -inf
 * row gives unspecified tokens, never an out-of-bounds access).
 */
#ifndef VERIFY_SAMPLE_H
#define VERIFY_SAMPLE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "verify_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define VA_SAMPLE_TILE 8192        /* logits per tile of the top-k scan        */
#define VA_SAMPLE_MAX_K 64         /* largest top_k                            */
#define VA_SAMPLE_MAX_VOCAB 262144 /* largest vocabulary (32 tiles)            */
#define VA_SAMPLE_MAX_ROWS 16      /* largest number of rows per call          */

#define VA_PURPOSE_TARGET 0u   /* the verification rows' own draws            */
#define VA_PURPOSE_ACCEPT 1u   /* acceptance tests (used by va_accept)        */
#define VA_PURPOSE_RESIDUAL 2u /* replacement draws (used by va_accept)       */

typedef struct {
  int32_t rows;           /* 1..VA_SAMPLE_MAX_ROWS                                 */
  int32_t top_k;          /* 1..VA_SAMPLE_MAX_K                                    */
  int64_t vocab;          /* 1..VA_SAMPLE_MAX_VOCAB                                */
  int64_t row_stride;     /* elements between rows of logits, >= vocab             */
  float temperature;      /* finite, > 0                                           */
  float top_p;            /* > 0; >= 1 keeps every nonzero candidate              */
  uint64_t seed;          /* request seed (the generator's key)                    */
  int64_t first_position; /* row r draws the token at first_position + r, >= 0     */
  uint32_t purpose;       /* counter word 2 of the rows' draws                     */
  int32_t reserved;       /* 0                                                     */
} va_sample_params;

/* Workspace bytes for va_sample / va_sample_accept with these parameters
 * (one sorted candidate list per (row, tile) after a 256-byte block of
 * counters), or 0 if the parameters are invalid.  The counters must be zero
 * before a workspace's first use (zero-fill it once); every call leaves them
 * zero again, so a workspace is reused without clearing.  Two calls in flight
 * at once must not share a workspace. */
size_t va_sample_workspace_bytes(const va_sample_params *params);

/* Sample every row (IQuestRT report, "Include sampling and acceptance in the
 * execution path"; top-k by tiles of 8,192 logits whose sorted candidate
 * lists are merged, "Parallelize the Top-K vocabulary scan").
 *   logits     [rows][row_stride] FP32, 4-byte aligned (rows that start on
 *              16 bytes -- an aligned pointer and row_stride % 4 == 0 -- are
 *              read with 16-byte loads).
 *   ids        [rows][top_k] int32: candidates in order, -1 past min(top_k, V).
 *   probs      [rows][top_k] FP32: renormalised kept probabilities, 0 past kept.
 *   kept       [rows] int32: number of kept candidates (>= 1).
 *   tokens     [rows] int32: the drawn token.
 *   workspace  >= va_sample_workspace_bytes, 16-byte aligned, counters
 *              zero (see above).
 * One launch, grid tiles x rows: each workgroup scans one tile; the last
 * workgroup of a row to finish merges the row's tile lists and draws (a
 * device-scope counter per row in the workspace hands over).
 * Errors: VA_ERR_INVALID (a parameter outside its range, a NULL or misaligned
 * pointer), VA_ERR_WORKSPACE, VA_ERR_HIP. */
va_status va_sample(const va_sample_params *params, const float *logits, int32_t *ids, float *probs,
                    int32_t *kept, int32_t *tokens, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Rejection acceptance of n - 1 drafts (same section), one wavefront.
 *   p_ids, p_probs   [n][p_stride] target lists (as written by va_sample).
 *   p_kept, p_tokens [n] target kept counts and own samples.
 *   q_ids, q_probs   [n-1][q_stride] the draft's kept lists; q_kept [n-1].
 *   drafts           [n-1] the draft tokens d_1..d_{n-1}.
 *   n                1..VA_SAMPLE_MAX_ROWS; strides 1..VA_SAMPLE_MAX_K.
 *   accepted         [1] int32 out; out_tokens [n] int32 out (entries past
 *                    a + 1 are written as -1).
 * Kept counts are read from device memory and clamped to the strides.
 * Errors: VA_ERR_INVALID, VA_ERR_HIP. */
va_status va_accept(const int32_t *p_ids, const float *p_probs, const int32_t *p_kept, const int32_t *p_tokens,
                    int32_t p_stride, const int32_t *q_ids, const float *q_probs, const int32_t *q_kept,
                    int32_t q_stride, const int32_t *drafts, int32_t n, uint64_t seed, int64_t first_position,
                    int32_t *accepted, int32_t *out_tokens, hipStream_t stream);

/* va_sample of the n = rows verification rows (purpose as given, normally
 * VA_PURPOSE_TARGET) followed by va_accept, in the one launch of va_sample:
 * the last row to finish its merge runs the acceptance (a second counter in
 * the workspace).  Outputs as the two calls'. */
va_status va_sample_accept(const va_sample_params *params, const float *logits, const int32_t *q_ids,
                           const float *q_probs, const int32_t *q_kept, int32_t q_stride, const int32_t *drafts,
                           int32_t *ids, float *probs, int32_t *kept, int32_t *tokens, int32_t *accepted,
                           int32_t *out_tokens, void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_SAMPLE_H */
