// Host-side plan: validation, per-row visible intervals, tree ancestry, the
// split count and the workspace size.  Integer-only, no HIP calls.
//
// Row geometry follows the IQuestRT report ("IQuestRT execution": one
// committed token plus drafts padded to the kernel width; "Read only the KV
// tiles needed by the current positions": the read is bounded by the live
// positions, the ring is the window plus one 64-slot tile) and "Qwen3.8-27B
// on one RTX 4090" ("More tokens per round: verify trees": tree mask).
#include <math.h>
#include <string.h>

#include "plan_data.h"

static inline int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }
static inline int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// Splits: each workgroup streams a contiguous run of 32-key granules, one
// after another, and writes its live rows' partials (m, l, O: up to
// rows*G*(D+2)*4 bytes per KV head), which the combine reads back right
// after.  More splits shorten the longest walk; fewer shrink the partials
// that must be written back and read again.  Timed as split + combine pairs
// over cold caches on MI355X, the best count is near
// S = 6.9 * sqrt(C * B_granule / (B_partial * Hkv)), with B_partial counted
// over all rows: for the 48-row full-attention shape (ratio ~1.5) 64 splits
// at 4K keys, 128 at 16K (1.4 us per pair faster than 256), 176 at 32K; for
// the 96-row tree over four KV heads 16 / 32 / 64 at 2K / 8K / 32K.  The
// count is kept a multiple of 8 (one share per XCD) from 8 up and capped at
// one workgroup per CU over all KV heads.  Two workgroups of the 48-row
// kernel fit on a CU (124 VGPRs and 64 KiB of LDS each), but twice the
// splits write and read back twice the partials: pairs measured 9.7 / 14.9
// / 15.5 / 27.6 us at 16K / 32K / 64K / 192K keys against 8.9 / 11.1 / 13.2
// / 24.1 us at one workgroup per CU.  Where the fit comes within a quarter
// of one granule per split (short reads: 33 granules at 1K keys) every split
// takes one granule.
static const int64_t kWorkgroupsPerCU = 1;

// round(sqrt(chunks * k_num / k_den)) exactly: the largest s with
// (2s - 1)^2 * k_den <= 4 * chunks * k_num (a double estimate, then an
// integer check either way)
static int64_t round_sqrt_ratio(int64_t chunks, int64_t k_num, int64_t k_den) {
  const int64_t rhs = 4 * chunks * k_num;
  int64_t s = (int64_t)(sqrt((double)chunks * (double)k_num / (double)k_den) + 0.5);
  if (s > 65536) s = 65536;  // far above any cap; keeps the products below 2^63
  if (s > 0 && (2 * s - 1) * (2 * s - 1) * k_den > rhs) --s;
  if ((2 * s + 1) * (2 * s + 1) * k_den <= rhs) ++s;
  return s;
}

static int32_t choose_splits(int64_t chunks, int32_t kv_heads, int32_t num_cus, int64_t granule_bytes,
                             int64_t partial_bytes) {
  if (chunks <= 0) return 1;
  if (num_cus <= 0) num_cus = 256;
  int64_t cap = (kWorkgroupsPerCU * num_cus) / kv_heads;
  if (cap < 1) cap = 1;
  if (cap >= 8) cap = (cap / 8) * 8;  // whole rounds over the 8 XCDs
  // 6.9 * sqrt(chunks * granule_bytes / (partial_bytes * kv_heads)), 6.9^2 = 47.61
  int64_t s = round_sqrt_ratio(chunks, 4761 * granule_bytes, 100 * partial_bytes * kv_heads);
  if (4 * s >= 3 * chunks) {
    s = chunks;  // within a quarter of one granule per split: take one granule each
  } else if (s >= 8) {
    s = ((s + 4) / 8) * 8;
  }
  if (s > cap) s = cap;
  if (s > chunks) s = chunks;
  if (s < 1) s = 1;
  return (int32_t)s;
}

extern "C" va_status verify_attn_plan(const va_problem *p, va_plan *plan, size_t *workspace_bytes) {
  if (!p || !plan) return VA_ERR_INVALID;
  memset(plan, 0, sizeof(*plan));
  va_plan_data d;
  memset(&d, 0, sizeof(d));

  if (p->reserved != 0) return VA_ERR_INVALID;
  if (p->rows < 1 || p->rows > VA_MAX_ROWS) return VA_ERR_INVALID;
  if (p->live_rows < 0 || p->live_rows > p->rows) return VA_ERR_INVALID;
  if (p->q_heads < 1 || p->kv_heads < 1 || p->q_heads % p->kv_heads != 0) return VA_ERR_INVALID;
  if (p->mask < VA_MASK_CAUSAL || p->mask > VA_MASK_TREE) return VA_ERR_INVALID;
  if (p->kv_fmt < VA_KV_BF16 || p->kv_fmt > VA_KV_K_E4M3_WHT_V_I8) return VA_ERR_INVALID;
  if (!(isfinite(p->scale) && p->scale > 0.0f)) return VA_ERR_INVALID;
  if (p->splits < 0) return VA_ERR_INVALID;
  if (p->head_dim != 64 && p->head_dim != 128) return VA_ERR_UNSUPPORTED;
  if (p->kv_fmt == VA_KV_K_E4M3_WHT_V_I8 && p->head_dim != 128) return VA_ERR_UNSUPPORTED;
  const int32_t G = p->q_heads / p->kv_heads;
  if ((int64_t)p->rows * G > VA_MAX_MATRIX_ROWS) return VA_ERR_UNSUPPORTED;

  d.magic = VA_PLAN_MAGIC;
  d.rows = p->rows;
  d.live_rows = p->live_rows;
  d.q_heads = p->q_heads;
  d.kv_heads = p->kv_heads;
  d.head_dim = p->head_dim;
  d.group = G;
  d.matrix_rows = p->rows * G;
  d.mask = p->mask;
  d.kv_fmt = p->kv_fmt;
  d.scale = p->scale;
  d.kv_capacity = p->kv_capacity;

  const int R = p->rows;
  if (p->mask == VA_MASK_CAUSAL || p->mask == VA_MASK_WINDOW) {
    if (p->first_pos < 0) return VA_ERR_INVALID;
    if (p->first_pos > ((int64_t)1 << 61)) return VA_ERR_INVALID;
    d.first_pos = p->first_pos;
    if (p->mask == VA_MASK_WINDOW) {
      if (p->window < 1) return VA_ERR_INVALID;
      d.window = p->window;
    }
    for (int r = 0; r < R; ++r) {
      if (r < p->live_rows) {
        const int64_t t = p->first_pos + r;
        d.row_lo[r] = (p->mask == VA_MASK_WINDOW) ? imax64(0, t - p->window + 1) : 0;
        d.row_hi[r] = t + 1;
      }
    }
  } else {  // tree
    if (p->prefix_len < 0 || p->prefix_len > ((int64_t)1 << 61)) return VA_ERR_INVALID;
    d.prefix_len = p->prefix_len;
    for (int i = 0; i < R; ++i) {
      const int32_t pa = p->parent[i];
      if (pa < -1 || pa >= i) return VA_ERR_INVALID;
    }
    for (int i = 0; i < R; ++i) {
      uint32_t bits = 1u << i;
      for (int j = p->parent[i]; j >= 0; j = p->parent[j]) bits |= 1u << j;
      d.anc[i] = (i < p->live_rows) ? bits : 0u;
      if (i < p->live_rows) {
        d.row_lo[i] = 0;
        d.row_hi[i] = p->prefix_len;
      }
    }
  }

  // Ring storage (window mode only).
  if (p->ring_slots != 0) {
    if (p->mask != VA_MASK_WINDOW) return VA_ERR_INVALID;
    if (p->ring_slots < 0 || p->ring_slots % VA_TILE != 0) return VA_ERR_INVALID;
    // The rows' own writes must not evict a key an earlier row still needs.
    if ((int64_t)p->ring_slots < (int64_t)p->window + R - 1) return VA_ERR_INVALID;
    d.ring_slots = p->ring_slots;
  }

  // Union extent over live rows.
  int64_t lo = 0, hi = 0;
  if (p->live_rows > 0) {
    if (p->mask == VA_MASK_TREE) {
      lo = 0;
      hi = p->prefix_len + p->live_rows;
    } else {
      lo = d.row_lo[0];
      hi = d.row_hi[p->live_rows - 1];
    }
  }
  d.lo = lo;
  d.hi = hi;
  if (hi - lo >= ((int64_t)1 << 31) - 2 * VA_TILE) return VA_ERR_INVALID;
  if (d.ring_slots == 0 && p->live_rows > 0) {
    if (p->kv_capacity < hi) return VA_ERR_CAPACITY;
  }
  if (d.ring_slots == 0 && p->kv_capacity < 0) return VA_ERR_INVALID;

  d.chunk_lo = lo / VA_SPLIT_KEYS;
  d.chunks = (hi > lo) ? (hi + VA_SPLIT_KEYS - 1) / VA_SPLIT_KEYS - d.chunk_lo : 0;
  d.ring_base_slot = d.ring_slots ? (int32_t)((d.chunk_lo * VA_SPLIT_KEYS) % d.ring_slots) : 0;

  // Keys seen by every live row, where no per-key mask is needed.
  if (p->live_rows > 0) {
    int64_t flo = INT64_MIN, fhi = INT64_MAX;
    for (int r = 0; r < p->live_rows; ++r) {
      flo = imax64(flo, d.row_lo[r]);
      fhi = imin64(fhi, d.row_hi[r]);
    }
    if (fhi < flo) fhi = flo;
    d.full_lo = flo;
    d.full_hi = fhi;
  }

  const int64_t granule_bytes =
      (int64_t)VA_SPLIT_KEYS * (p->kv_fmt == VA_KV_K_E4M3_WHT_V_I8 ? 2 * d.head_dim + 4 : 4 * d.head_dim);
  const int64_t partial_bytes = (int64_t)d.matrix_rows * (d.head_dim + 2) * 4;
  d.splits = p->splits > 0 ? p->splits
                           : choose_splits(d.chunks, d.kv_heads, p->num_cus, granule_bytes, partial_bytes);

  // Row groups.  A consumer wave owns 16 matrix rows and one SIMD runs the
  // producers' and up to four consumers' work side by side; from five
  // 16-row blocks on (80 or 96 matrix rows: the 16-node tree at G = 6) two
  // consumers share a SIMD and each step takes about twice as long.  When
  // twice the workgroups still fit one per CU, each (split, KV head) is run
  // by two workgroups that stream the same keys and take half the row
  // blocks each (bf16 tree, ABBA on MI355X: calls 10.55 -> 9.12 us at 2K
  // keys and 14.2 -> 12.5 us at 8K).  Every row's partials are the same
  // either way: a row block's arithmetic does not depend on the workgroup
  // that runs it.
  {
    const int32_t blocks = (d.matrix_rows + 15) / 16;
    const int64_t cus = p->num_cus > 0 ? p->num_cus : 256;
    d.row_groups = (blocks >= 5 && (int64_t)d.splits * d.kv_heads * 2 <= cus) ? 2 : 1;
  }

  const uint64_t units = (uint64_t)d.splits * d.kv_heads * d.matrix_rows;
  d.ml_bytes = ((units * 2 * sizeof(float)) + 255) / 256 * 256;
  d.workspace_bytes = d.ml_bytes + units * d.head_dim * sizeof(float);

  memcpy(plan, &d, sizeof(d));
  if (workspace_bytes) *workspace_bytes = (size_t)d.workspace_bytes;
  return VA_OK;
}

static const va_plan_data *as_data(const va_plan *plan) {
  if (!plan) return nullptr;
  const va_plan_data *d = reinterpret_cast<const va_plan_data *>(plan);
  return d->magic == VA_PLAN_MAGIC ? d : nullptr;
}

extern "C" va_status verify_attn_plan_query(const va_plan *plan, va_plan_info *info) {
  const va_plan_data *d = as_data(plan);
  if (!d || !info) return VA_ERR_INVALID;
  memset(info, 0, sizeof(*info));
  info->splits = d->splits;
  info->matrix_rows = d->matrix_rows;
  info->lo = d->lo;
  info->hi = d->hi;
  info->chunk_lo = d->chunk_lo;
  info->chunks = d->chunks;
  for (int r = 0; r < VA_MAX_ROWS; ++r) {
    info->row_lo[r] = d->row_lo[r];
    info->row_hi[r] = d->row_hi[r];
    info->anc[r] = d->anc[r];
  }
  info->workspace_bytes = (size_t)d->workspace_bytes;
  info->row_groups = d->row_groups;
  return VA_OK;
}

extern "C" va_status verify_attn_plan_split_range(const va_plan *plan, int32_t s, int64_t *key_begin,
                                                  int64_t *key_end) {
  const va_plan_data *d = as_data(plan);
  if (!d || !key_begin || !key_end || s < 0 || s >= d->splits) return VA_ERR_INVALID;
  const int64_t C = d->chunks, S = d->splits;
  const int64_t q = C / S, r = C % S;
  const int64_t c0 = d->chunk_lo + s * q + (s < r ? s : r);
  const int64_t c1 = c0 + q + (s < r ? 1 : 0);
  int64_t a = imax64(d->lo, c0 * VA_SPLIT_KEYS);
  int64_t b = imin64(d->hi, c1 * VA_SPLIT_KEYS);
  if (b < a) b = a;
  *key_begin = a;
  *key_end = b;
  return VA_OK;
}

extern "C" const char *va_status_string(va_status s) {
  switch (s) {
    case VA_OK: return "ok";
    case VA_ERR_INVALID: return "invalid argument";
    case VA_ERR_UNSUPPORTED: return "unsupported problem";
    case VA_ERR_CAPACITY: return "position beyond kv capacity";
    case VA_ERR_WORKSPACE: return "workspace too small";
    case VA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}
