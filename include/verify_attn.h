/*
 * verify_attn.h -- C ABI for multi-row speculative-verification decode
 * attention on MI355X (gfx950).
 *
 * What the library computes (IQuestRT report, section "Read only the KV tiles
 * needed by the current positions"; section "Expose more parallelism in
 * attention"; "Qwen3.8-27B on one RTX 4090", sections "More tokens per round:
 * verify trees" and "A cheaper cache and state"):
 *
 *   A few query rows -- one committed token plus drafts, padded to a fixed
 *   width, or the nodes of a draft tree -- times the G query heads that share
 *   one KV head attend over a long KV cache.  For live row r and query head h,
 *   with KV head g = h / G and the sink logit sigma_h,
 *
 *     s_j = scale * <q_{r,h}, k_{g,j}>        for every key j row r sees
 *     o   = sum_j e^{s_j - M} v_{g,j} / (sum_j e^{s_j - M} + e^{sigma_h - M})
 *     lse = M + ln(sum_j e^{s_j - M} + e^{sigma_h - M}),  M = max(max_j s_j, sigma_h)
 *
 *   The sink has zero value: it adds to the denominator only.  The read stops
 *   at the live rows' positions (preallocated capacity adds no reads).  The
 *   keys are split along the sequence; verify_attn_split leaves one partial
 *   (max, sum, unnormalised output) per split and verify_attn_combine merges
 *   them by log-sum-exp and applies the sink.
 *
 * Which keys row r sees (all positions are absolute token positions):
 *   VA_MASK_CAUSAL  row r sits at t = first_pos + r and sees 0..t.
 *   VA_MASK_WINDOW  row r at t sees max(0, t-window+1)..t.  The keys live in
 *                   a ring of ring_slots slots (position p in slot
 *                   p mod ring_slots) or, with ring_slots = 0, in a linear
 *                   cache.  swa_ring_write (bf16) or verify_kv_write (any
 *                   format) stores the rows' own K/V first.
 *   VA_MASK_TREE    node i's key sits at position prefix_len + i; row i sees
 *                   0..prefix_len-1, its tree ancestors and itself.
 *   Rows live_rows..rows-1 are padding: they see nothing, never widen the
 *   read, and their outputs are written as 0 (lse -inf).
 *
 * Conventions shared by every entry point:
 *   - Device pointers are HIP device memory owned by the caller; the library
 *     never allocates, frees or synchronises, and keeps no global state.
 *   - Every call is asynchronous on `stream`; a fault inside a kernel shows
 *     up at the caller's next synchronisation, not in the returned status.
 *   - No function aborts or throws; each returns a va_status.  Launch errors
 *     are reported as VA_ERR_HIP.
 *   - Calls on one stream run in order: swa_ring_write (window mode) ->
 *     verify_attn_split -> verify_attn_combine.  The combine must follow the
 *     split that filled its workspace; a workspace must not be shared by two
 *     calls in flight at once.
 */
#ifndef VERIFY_ATTN_H
#define VERIFY_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VA_OK = 0,
  VA_ERR_INVALID = 1,      /* malformed problem or arguments                      */
  VA_ERR_UNSUPPORTED = 2,  /* well formed, but outside what the kernels implement  */
  VA_ERR_CAPACITY = 3,     /* a position the rows need lies beyond kv_capacity     */
  VA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the plan requires  */
  VA_ERR_HIP = 5           /* a HIP launch or query failed                         */
} va_status;

typedef enum { VA_MASK_CAUSAL = 0, VA_MASK_WINDOW = 1, VA_MASK_TREE = 2 } va_mask;

/* KV formats.
 * VA_KV_BF16: k and v are bf16.
 * VA_KV_K_E4M3_WHT_V_I8 ("Qwen3.8-27B on one RTX 4090", "A cheaper cache and
 *   state"): k holds OCP E4M3FN codes of the key after the normalised
 *   128-point Walsh-Hadamard rotation H/sqrt(128) (natural Sylvester order);
 *   v holds int8 codes, value = code * v_scale[token].  The library rotates q
 *   by the same matrix (in FP32, then rounds to bf16) before the scores, so
 *   scores equal <q, k> up to the key quantisation.  head_dim must be 128. */
typedef enum { VA_KV_BF16 = 0, VA_KV_K_E4M3_WHT_V_I8 = 1 } va_kv_fmt;

#define VA_MAX_ROWS 16
#define VA_MAX_MATRIX_ROWS 96   /* rows * (q_heads / kv_heads) */
#define VA_TILE 64              /* ring slots come in 64-slot tiles                      */
#define VA_SPLIT_KEYS 32        /* keys per split granule; split boundaries are 32-key aligned */

/* The problem, as plain host data.  Fields marked (w) are read in window mode
 * only, (t) in tree mode only. */
typedef struct {
  int32_t rows;          /* 1..16: kernel row width (chain rows, or tree nodes)            */
  int32_t live_rows;     /* 0..rows: rows [0, live_rows) are live, the rest padding        */
  int32_t q_heads;       /* Hq >= 1                                                        */
  int32_t kv_heads;      /* Hkv >= 1, Hq % Hkv == 0; G = Hq / Hkv, rows * G <= 96          */
  int32_t head_dim;      /* D: 64 or 128                                                   */
  int32_t mask;          /* va_mask                                                        */
  int32_t kv_fmt;        /* va_kv_fmt                                                      */
  int32_t window;        /* (w) W >= 1                                                     */
  int32_t ring_slots;    /* (w) 0 = linear cache; else C, C % 64 == 0, C >= W + rows - 1   */
  int32_t splits;        /* 0 = the plan chooses; > 0 forces that many splits              */
  int32_t num_cus;       /* compute units of the target GPU (used to choose splits)        */
  int32_t parent[VA_MAX_ROWS]; /* (t) -1 = child of the last committed token, else < i     */
  int64_t first_pos;     /* causal/window: position of row 0, >= 0                         */
  int64_t prefix_len;    /* (t) P >= 0: committed keys 0..P-1; node i's key at P + i       */
  int64_t kv_capacity;   /* linear cache: key slots allocated per KV head                  */
  float scale;           /* score scale, e.g. 1/sqrt(D); finite and > 0                    */
  int32_t reserved;      /* must be 0                                                      */
} va_problem;

/* A validated plan: opaque, plain host memory, immutable after
 * verify_attn_plan, freely copyable and reusable across calls and threads. */
typedef struct { uint64_t words[256]; } va_plan;

/* What the plan decided (for tests and diagnostics). */
typedef struct {
  int32_t splits;              /* S                                                        */
  int32_t matrix_rows;         /* rows * G                                                 */
  int64_t lo, hi;              /* union of the live rows' visible keys lies in [lo, hi)    */
  int64_t chunk_lo, chunks;    /* first granule floor(lo/32), count ceil(hi/32) - chunk_lo */
  int64_t row_lo[VA_MAX_ROWS]; /* row r sees [row_lo, row_hi) (tree: the prefix part)      */
  int64_t row_hi[VA_MAX_ROWS];
  uint32_t anc[VA_MAX_ROWS];   /* tree: bit j set iff node j is node r or its ancestor     */
  size_t workspace_bytes;
  int32_t row_groups;          /* workgroups per (split, KV head): 2 when the matrix rows
                                  fill more than four 16-row blocks and 2 * S * Hkv <=
                                  num_cus, each taking half the row blocks; else 1         */
} va_plan_info;

/* Validate *p and build *plan.  Writes the workspace size the split needs to
 * *workspace_bytes (may be NULL).  Pure host code: needs no GPU.
 * With splits = 0 the plan chooses from C, the number of 32-key granules:
 * s = round(sqrt(C * 47.61 * B_g / (B_p * Hkv))) (B_g the KV bytes of one
 * granule, 32*4*D or 32*(2*D+4) quantised; B_p = rows*G*(D+2)*4 partial
 * bytes per split and KV head); C itself (one granule per split) where
 * 4 * s >= 3 * C, else s rounded to the nearest multiple of 8 from 8 up;
 * then at most num_cus / Hkv (a multiple of 8 from 8 up) and at most C, at
 * least 1.
 * Errors: VA_ERR_INVALID (NULL pointers, counts out of range, parent[i] >= i
 * or < -1, C % 64 != 0, C < W + rows - 1 so that the rows' own writes would
 * evict history an earlier row needs, scale not finite and > 0, positions
 * negative, extent >= 2^31 keys), VA_ERR_UNSUPPORTED (D not 64/128,
 * rows * G > 96, quantised format with D != 128), VA_ERR_CAPACITY (linear
 * cache smaller than the highest key the live rows read). */
va_status verify_attn_plan(const va_problem *p, va_plan *plan, size_t *workspace_bytes);

/* Copy the plan's decisions into *info.  Host only. */
va_status verify_attn_plan_query(const va_plan *plan, va_plan_info *info);

/* Key range [*key_begin, *key_end) that split s covers (empty if begin ==
 * end).  With C granules of 32 keys, q = C / S and r = C % S, split s takes
 * q + 1 granules if s < r and q otherwise, contiguous from chunk_lo; keys are
 * clipped to [lo, hi).  Host only. */
va_status verify_attn_plan_split_range(const va_plan *plan, int32_t s,
                                       int64_t *key_begin, int64_t *key_end);

/* Run the split pass: for every split s, KV head g and matrix row
 * m = r*G + j (query head h = g*G + j) write
 *   m_s = max over the split's keys row r sees of s_j * log2(e)   (-inf if none)
 *   l_s = sum of 2^(s_j*log2(e) - m_s) over them
 *   O_s = the same weights times v_j, summed (FP32 [D], unnormalised)
 * into the workspace: first the {m, l} pairs as FP32 [S][Hkv][rows*G][2],
 * then, from the next multiple of 256 bytes, O as FP32 [S][Hkv][rows*G][D].
 * Padding rows' partials are not written (the combine never reads them).
 *   q        [rows, Hq, D] bf16, contiguous, 16-byte aligned.
 *   k, v     [Hkv, slots, D] with D contiguous: bf16 (VA_KV_BF16) or
 *            uint8 E4M3FN codes / int8 codes.  Slot of position p: p (linear)
 *            or p mod ring_slots (ring).  Element strides kv_head_stride and
 *            kv_row_stride (in elements of the stored type) apply to both;
 *            base pointers and row strides must give 16-byte aligned rows.
 *            Only slots of positions in [lo, hi) are read.
 *   v_scale  [Hkv][slots] FP32 with head stride v_scale_head_stride (in
 *            floats), for VA_KV_K_E4M3_WHT_V_I8; NULL otherwise.
 *   workspace, workspace_bytes: device memory of at least the plan's size.
 * Errors: VA_ERR_INVALID (bad plan, NULL or misaligned pointers, bad
 * strides), VA_ERR_WORKSPACE, VA_ERR_HIP. */
va_status verify_attn_split(const va_plan *plan, const void *q, const void *k, const void *v,
                            const float *v_scale, int64_t v_scale_head_stride,
                            int64_t kv_head_stride, int64_t kv_row_stride,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Merge the splits (IQuestRT report, "Read only the KV tiles needed by the
 * current positions": a separate combine kernel with four independent FP32
 * accumulation chains; "Expose more parallelism in attention": the merge is
 * by log-sum-exp and the combine applies the sink).
 *   sink  [Hq] FP32 logits in the units of s_j, or NULL for no sink.
 *   out   [rows, Hq, D] FP32; padding rows are written as 0.
 *   lse   [rows, Hq] FP32 natural-log LSE including the sink, or NULL;
 *         padding rows -inf; a live row that sees nothing, without sink, gets
 *         out = 0 and lse = -inf.
 * Errors: VA_ERR_INVALID, VA_ERR_WORKSPACE, VA_ERR_HIP. */
va_status verify_attn_combine(const va_plan *plan, const void *workspace, size_t workspace_bytes,
                              const float *sink, float *out, float *lse, hipStream_t stream);

/* verify_attn_split with the rows' own K/V written in the same launch, for
 * the step where the verification rows' keys and values enter the cache
 * right before the read (IQuestRT report, "IQuestRT execution": row 0's KV
 * is written before the attention that reads it; "Read only the KV tiles
 * needed by the current positions" and "Let correctness checks change the
 * design" for the ring; 4090 post, "More tokens per round: verify trees" for
 * the tree's node keys).  bf16 caches; static plans only.
 *   k_new, v_new  [rows, Hkv, D] bf16, contiguous, 16-byte aligned: every
 *                 row, padding included, is stored to slot (first_pos + r)
 *                 mod ring_slots (ring), first_pos + r (linear cache) or
 *                 prefix_len + r (tree), exactly as swa_ring_write /
 *                 verify_kv_write would.
 *   the rest as verify_attn_split; k and v are written.
 * The partials equal those of swa_ring_write (or verify_kv_write) followed by
 * verify_attn_split on the same stream: the live rows' keys and values are
 * taken from k_new / v_new for the split's own read, so no workgroup
 * depends on another's cache store.  The window ring's size guarantees that
 * no stored slot holds a key any row still sees.
 * Errors: as verify_attn_split, plus VA_ERR_UNSUPPORTED (a quantised cache),
 * VA_ERR_INVALID (NULL or misaligned k_new / v_new) and VA_ERR_CAPACITY
 * (linear cache or tree with the rows' last slot at or past kv_capacity). */
va_status verify_attn_split_append(const va_plan *plan, const void *q, const void *k_new, const void *v_new,
                                   void *k, void *v, int64_t kv_head_stride, int64_t kv_row_stride,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Per-call state in device memory, for calls whose positions and row count
 * are produced on the device (IQuestRT report, "IQuestRT execution": lengths
 * stay on the device and the step is launched from graphs).  A plan built for
 * a bucket -- the largest extent the state may describe -- fixes the grid and
 * the workspace; each call then reads this record, and the kernels derive the
 * row intervals, the read extent, the split table and the tree's ancestor
 * bits from it on the device.  Fields have the meaning of the va_problem
 * fields of the same name; the rest of the problem comes from the plan. */
typedef struct {
  int64_t first_pos;             /* causal/window: position of row 0                       */
  int64_t prefix_len;            /* tree: committed keys 0..P-1                              */
  int32_t live_rows;             /* 0..rows                                                  */
  int32_t reserved;              /* 0                                                        */
  int32_t parent[VA_MAX_ROWS];   /* tree: -1, or an index below the node's own               */
} va_state;

/* verify_attn_split and verify_attn_combine with the per-call state read from
 * device memory (`state`, 8-byte aligned, written before the call on the same
 * stream).  The plan's problem gives the bucket: the keys a state reads,
 * [lo, hi) as va_plan_info defines them for the state's own problem, must end
 * at or below the plan's hi (the plan has checked that key range against
 * kv_capacity, or against the ring, whose size covers any window state of at
 * most `rows` rows).  With C the state's 32-key granules, the split count is
 * min(S, C) for the plan's S (at least 1); the workgroups above it exit
 * without reading, so a short state in a long bucket reads only its own keys.
 * The launch configuration depends on the plan alone, so both calls can be
 * captured in a graph once and replayed for every state of the bucket.
 * A state outside the bucket, or with live_rows outside [0, rows], a
 * position outside [0, 2^61], reserved != 0 or (tree) a parent out of range,
 * reads no key: the combine writes NaN to every output element and lse.
 * Errors (returned): as verify_attn_split / verify_attn_combine, plus
 * VA_ERR_INVALID for a NULL or misaligned state. */
va_status verify_attn_split_state(const va_plan *plan, const va_state *state, const void *q, const void *k,
                                  const void *v, const float *v_scale, int64_t v_scale_head_stride,
                                  int64_t kv_head_stride, int64_t kv_row_stride, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);
va_status verify_attn_combine_state(const va_plan *plan, const va_state *state, const void *workspace,
                                    size_t workspace_bytes, const float *sink, float *out, float *lse,
                                    hipStream_t stream);
/* verify_attn_split_append with the per-call state read from device memory,
 * as verify_attn_split_state: the rows' own K/V stored (and read) in the
 * split launch of a device-driven step, so a captured step of one bucket
 * needs two launches.  Row r is stored to the slot of its own key under the
 * state's positions; in a linear cache, rows whose slot would be at or past
 * kv_capacity (padding rows of a state near the end of the bucket) are not
 * stored.  A state outside the bucket stores nothing.
 * Errors: as verify_attn_split_state and verify_attn_split_append (no host
 * capacity check: the state is on the device). */
va_status verify_attn_split_append_state(const va_plan *plan, const va_state *state, const void *q,
                                         const void *k_new, const void *v_new, void *k, void *v,
                                         int64_t kv_head_stride, int64_t kv_row_stride, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/* Store the verification rows' own K/V into the sliding-window ring before
 * the read (IQuestRT report, "Read only the KV tiles needed by the current
 * positions"; "Let correctness checks change the design"): row r's K/V, for
 * every KV head, goes to slot (first_pos + r) mod ring_slots.  All `rows` rows
 * are written, padding included.
 *   k_new, v_new   [rows, kv_heads, head_dim] bf16, contiguous.
 *   k_ring, v_ring [kv_heads, ring_slots, head_dim] bf16 with element strides
 *                  kv_head_stride, kv_row_stride; 16-byte aligned rows.
 * Errors: VA_ERR_INVALID (rows outside 0..16, ring_slots < rows, head_dim not
 * 64/128, negative first_pos, NULL or misaligned pointers), VA_ERR_HIP.
 * rows == 0 is a no-op. */
va_status swa_ring_write(const void *k_new, const void *v_new, int32_t rows, int64_t first_pos,
                         int32_t kv_heads, int32_t head_dim, void *k_ring, void *v_ring,
                         int32_t ring_slots, int64_t kv_head_stride, int64_t kv_row_stride,
                         hipStream_t stream);

/* Write the verification rows' own K/V into a KV cache before the read, in
 * the cache's storage format (4090 post, "A cheaper cache and state": keys in
 * FP8 after a Hadamard rotation, values in INT8 with one scale per token and
 * KV head; IQuestRT report, "Read only the KV tiles needed by the current
 * positions": the rows are written before the read).  Row r of KV head g
 * goes to slot first_pos + r of a linear cache (ring_slots = 0) or to slot
 * (first_pos + r) mod ring_slots of a ring.  All `rows` rows are written,
 * padding included.
 *   k_new, v_new  [rows, kv_heads, head_dim] bf16, contiguous.
 *   kv_fmt        VA_KV_BF16: the rows are copied.
 *                 VA_KV_K_E4M3_WHT_V_I8 (head_dim 128): k' = H k / sqrt(128)
 *                 is formed in FP32 by the fast transform (butterflies of
 *                 width 1, 2, ..., 64, each (a, b) -> (a + b, a - b), then a
 *                 multiply by FP32 1/sqrt(128)) and stored as the nearest
 *                 E4M3FN code (ties to even, saturating at 448, sign kept;
 *                 a NaN key element makes the row's codes 0x7F).  This is
 *                 the code of the exact rotation except where an E4M3
 *                 rounding midpoint lies within the FP32 rounding error of
 *                 the rotated value, where it may be the other neighbour.
 *                 s = max|v| / 127 in FP32 goes to v_scale and each value is
 *                 stored as the round-half-even of v / s (taken in FP64)
 *                 clamped to [-127, 127] (all codes 0 when s = 0, or when
 *                 the row holds NaN or an infinity, whose s is then NaN or
 *                 infinite).
 *   k_cache, v_cache  [kv_heads, slots, head_dim]: bf16, or uint8 (keys) and
 *                 int8 (values) codes, element strides kv_head_stride and
 *                 kv_row_stride, 16-byte aligned rows.
 *   v_scale       [kv_heads, slots] FP32 with head stride v_scale_head_stride
 *                 (quantised format), else ignored.
 *   kv_capacity   linear cache: slots per KV head; must hold first_pos + rows.
 * Errors: VA_ERR_INVALID (rows outside 0..4096, kv_heads < 1, head_dim not
 * 64/128, unknown kv_fmt, negative first_pos, ring_slots < rows or not a
 * multiple of 64, NULL or misaligned pointers, bad strides),
 * VA_ERR_UNSUPPORTED (quantised format with head_dim != 128),
 * VA_ERR_CAPACITY (linear cache smaller than first_pos + rows), VA_ERR_HIP.
 * rows == 0 is a no-op. */
va_status verify_kv_write(const void *k_new, const void *v_new, int32_t rows, int64_t first_pos,
                          int32_t kv_heads, int32_t head_dim, int32_t kv_fmt, void *k_cache,
                          void *v_cache, float *v_scale, int64_t v_scale_head_stride,
                          int64_t kv_capacity, int32_t ring_slots, int64_t kv_head_stride,
                          int64_t kv_row_stride, hipStream_t stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc:
 * verify_attn_split followed by verify_attn_combine on `stream`, with the
 * partials kept in a workspace that the library holds in a static device
 * array of VA_NOALLOC_WORKSPACE_BYTES per GPU (allocated when the library's
 * code object is loaded on that GPU, held until the process ends) instead of
 * a caller workspace.  No allocation, free or synchronisation happens in the
 * call.  The first call on a device (the device current at the call) looks
 * the array's address up on that device (not a stream operation); make it
 * outside a graph capture.
 * Arguments as verify_attn_split (q, k, v, v_scale, strides) and
 * verify_attn_combine (sink, out, lse).  The array needs no clearing: every
 * partial the combine reads is written by the split of the same call.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and must be ordered by the caller.
 * Errors: VA_ERR_WORKSPACE when the plan's workspace exceeds
 * VA_NOALLOC_WORKSPACE_BYTES; VA_ERR_HIP when the array's address cannot be
 * looked up; otherwise as verify_attn_split and verify_attn_combine. */
#define VA_NOALLOC_WORKSPACE_BYTES (16u << 20)
va_status verify_attn_noalloc(const va_plan *plan, const void *q, const void *k, const void *v,
                              const float *v_scale, int64_t v_scale_head_stride, int64_t kv_head_stride,
                              int64_t kv_row_stride, const float *sink, float *out, float *lse,
                              hipStream_t stream);

/* Static text for a status code. */
const char *va_status_string(va_status s);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_ATTN_H */
