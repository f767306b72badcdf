// Internal layout of va_plan.  Shared by the host plan and the launchers only.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "verify_attn.h"

#define VA_PLAN_MAGIC 0x56415031u  // "VAP1"

struct va_plan_data {
  uint32_t magic;
  int32_t rows, live_rows, q_heads, kv_heads, head_dim;
  int32_t group;        // G = Hq / Hkv
  int32_t matrix_rows;  // rows * G
  int32_t mask, kv_fmt, window, ring_slots, splits;
  int32_t ring_base_slot;  // (chunk_lo * 32) mod ring_slots, 0 for a linear cache
  int32_t row_groups;      // workgroups per (split, KV head), each taking a share of the matrix rows
  int64_t first_pos, prefix_len, kv_capacity;
  int64_t lo, hi;          // union extent of the live rows' visible keys
  int64_t chunk_lo, chunks;  // 32-key granules [chunk_lo, chunk_lo + chunks) cover [lo, hi)
  int64_t full_lo, full_hi;  // keys every live row sees, outside the tree part
  int64_t row_lo[VA_MAX_ROWS], row_hi[VA_MAX_ROWS];
  uint32_t anc[VA_MAX_ROWS];
  float scale;
  uint64_t ml_bytes;         // size of the {m, l} block at the start of the workspace
  uint64_t workspace_bytes;  // total
};

static_assert(sizeof(va_plan_data) <= sizeof(va_plan), "plan record too large");
