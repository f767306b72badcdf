// Sampling of the verification rows and rejection acceptance of the drafts,
// for gfx950 (CDNA4, wave64).
//
// IQuestRT report, "Include sampling and acceptance in the execution path"
// (top-k, top-p and temperature of the target; the draft's saved proposal
// distribution; acceptance with probability min(1, p/q); replacement from
// max(0, p - q); bonus from the extra row; draws fixed by the request seed and
// the token position) and "Parallelize the Top-K vocabulary scan" (tiles of
// 8,192 logits scanned in parallel, then an ordered merge of their candidates
// in which the tile maxima bound what can still contribute).
//
// Kernels:
//   sample_kernel<ACCEPT>  grid (tiles, rows) x 256 threads: each workgroup
//                          writes one tile's exact top-k as a sorted list of
//                          64-bit composites; the last workgroup of a row to
//                          finish merges the row's lists and runs the softmax,
//                          top-p and the draw; with ACCEPT the last row to be
//                          merged also runs the acceptance.
//   accept_kernel          one wave: the acceptance alone.
//
// Every element of a row is ranked by a composite key: the FP32 logit mapped
// to an order-preserving uint32 in the high word and the complemented token id
// in the low word.  Composites are unique, so "the k largest composites" is
// exactly the top-k with equal logits taken by lower id, and 0 can mark an
// empty slot.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "verify_sample.h"

namespace va_sample_detail {

typedef unsigned long long u64;

constexpr int kTile = VA_SAMPLE_TILE;
constexpr int kTileThreads = 256;
constexpr int kPerThread = kTile / kTileThreads;               // 32 logits
constexpr int kMaxK = VA_SAMPLE_MAX_K;
constexpr int kMaxTiles = VA_SAMPLE_MAX_VOCAB / VA_SAMPLE_TILE;  // 32
constexpr int kMaxList = kMaxTiles * kMaxK;                     // 2,048 composites per row
constexpr int kListPerLane = kMaxList / 64;                     // 32
constexpr size_t kListOffset = 256;                             // after the counter

static_assert(kPerThread == 32 && kTile % (4 * kTileThreads) == 0, "tile layout");

// ---------------------------------------------------------------------------
// Keys and lane primitives.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  b = (b & 0x7fffffffu) ? b : 0u;  // -0 ranks with +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ u64 composite(float f, uint32_t id) {
  return ((u64)order_key(f) << 32) | (u64)(~id);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

__device__ __forceinline__ u64 umax64(u64 a, u64 b) { return a > b ? a : b; }

// Lane-to-lane moves on the DPP and permute paths (no LDS round trip).  They
// read other lanes' registers, so every lane of the wave must execute them.
__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ u64 readlane64(u64 v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((u64)hi << 32) | lo;
}

// Device-scope (agent) relaxed loads and stores: they bypass the per-XCD L2's
// non-coherent state (the sc1 bit), so data handed from a workgroup on one XCD
// to a workgroup on another needs no cache-wide write-back or invalidate --
// only the writer's wait for its stores before the hand-off counter moves.
template <typename T>
__device__ __forceinline__ void store_agent(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_agent(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Zero entries kept after the candidates of an LDS list: every rank loop
// below reads up to 8 steps of G past the end, and zeros rank below any entry.
constexpr int kRankPad = 128;

// The k-th largest of the wave's 64 values (1 <= k <= 64; values distinct
// unless 0), or 0 when fewer than k lanes hold a value above 0.  buf holds the
// 64 values in LDS (written by the caller, then a barrier); each lane counts
// the values above its own with broadcast reads.
__device__ __forceinline__ u64 wave_kth_largest(const u64 *buf, u64 v, int k) {
  int r = 0;
#pragma unroll
  for (int j = 0; j < 64; j += 16) {
    u64 w[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) w[q] = buf[j + q];
#pragma unroll
    for (int q = 0; q < 16; ++q) r += w[q] > v ? 1 : 0;
  }
  const u64 hit = __ballot(v != 0 && r == k - 1);
  return hit ? readlane64(v, __builtin_ctzll(hit)) : 0ull;
}

// Integer sum over groups of G consecutive lanes (G = 1, 2, 4, 8 or 16,
// uniform), every lane of a group getting the group's total.
__device__ __forceinline__ int group_sum(int x, int G) {
  if (G > 1) x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // lane ^ 1
  if (G > 2) x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // lane ^ 2
  if (G > 4) {                                                                // lane ^ 4
    const int y = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);   // 7 - i within 8
    x += __builtin_amdgcn_update_dpp(0, y, 0x1B, 0xF, 0xF, false);            // then i ^ 3 within 4
  }
  if (G > 8) x += __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);  // lane ^ 8
  return x;
}

// out[r] = c[i] for every entry i of c[0, C) whose rank r (number of larger
// entries) is below k.  NT threads (index t) share the work: G threads per
// entry, each counting over every G-th entry, then summing within the group.
// c needs kRankPad zeros after its C entries.
template <int NT, bool AGENT>
__device__ __forceinline__ void rank_and_place(const u64 *c, int C, int k, u64 *out, int t) {
  int G = 1;
  while (G < 16 && C * G * 2 <= NT) G <<= 1;
  const int lg = __builtin_ctz(G);
  for (int base = 0; base < C * G; base += NT) {
    const int slot = base + t, i = slot >> lg, q = slot & (G - 1);
    const bool ok = i < C;
    const u64 v = ok ? c[ok ? i : 0] : ~0ull;
    int r = 0;
    for (int j = q; j < C; j += 8 * G) {
      u64 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = c[j + u * G];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += w[u] > v ? 1 : 0;
    }
    r = group_sum(r, G);
    if (ok && q == 0 && r < k) {
      if constexpr (AGENT) store_agent(out + r, v);
      else out[r] = v;
    }
  }
}

// Inclusive prefix sum of integers over lanes (as wave_inclusive_scan).
__device__ __forceinline__ uint32_t wave_inclusive_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = lane_id() >> 4;
  if (row >= 1) x += r0;
  if (row >= 2) x += r1;
  if (row >= 3) x += r2;
  return x;
}

// Sum over the wave, the same value in every lane (lane 0's): rotations by
// 8, 4, 2, 1 inside each row of 16, then the row partners 16 and 32 apart.
__device__ __forceinline__ float wave_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Inclusive prefix sum over lanes: shifts by 1, 2, 4, 8 inside each row of
// 16 (lanes shifted in from outside the row add 0), then each row adds the
// totals of the rows before it.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  const int row = lane_id() >> 4;
  if (row >= 1) x += r0;
  if (row >= 2) x += r1;
  if (row >= 3) x += r2;
  return x;
}

// The value of lane i - 1 (0 in lane 0).
__device__ __forceinline__ float wave_shift_up1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x138, 0xF, 0xF, true));
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32
// multiplies, key bumped by the two Weyl constants between rounds.  Counter
// (position low, position high, purpose, 0), key (seed low, seed high); the
// first output word gives u = (x >> 8) * 2^-24 in [0, 1).
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t pos, uint32_t purpose) {
  uint32_t c0 = (uint32_t)pos, c1 = (uint32_t)(pos >> 32), c2 = purpose, c3 = 0u;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return (float)(c0 >> 8) * 0x1p-24f;
}

// ---------------------------------------------------------------------------
// The sampling kernel: tile scan, then (last tile of a row) merge and draw,
// then (last row, with ACCEPT) the acceptance.
// ---------------------------------------------------------------------------
struct SampleArgs {
  const float *logits;
  u64 *lists;           // [rows][tiles][k] sorted tile lists
  uint32_t *row_count;  // [rows] tiles finished; zero between calls
  uint32_t *done;       // rows finished; zero between calls
  int64_t row_stride, vocab;
  int32_t k, tiles, rows;
  int32_t vec;  // rows start 16-byte aligned: 16-byte loads
  int32_t *ids;
  float *probs;
  int32_t *kept, *tokens;
  float inv_temp, top_p;
  uint64_t seed;
  int64_t pos0;
  uint32_t purpose;
};

struct SampleShared {
  u64 cand[kTile + kRankPad];  // lane maxima, then candidates
  u64 top[kMaxK];
  u64 wbound[kTileThreads / 64];
  uint32_t ncand, flag;
};

// The exact top-k of x (kPerThread composites per thread, 0 = empty) over the
// workgroup, written in order to out[0, k) (zeros past the number of
// entries).  No sort of the whole set:
//   1. each wave takes B_w, the k-th largest of its 64 lanes' maxima: at
//      least k of the wave's entries reach B_w, so the k-th largest overall
//      does too, and so does B = max_w B_w;
//   2. the entries >= B (typically a few more than k) are gathered in LDS;
//   3. each gathered entry's rank is the number of larger ones; ranks below
//      k are written in order.
template <int E, bool AGENT>
__device__ __forceinline__ void block_topk(const u64 (&x)[E], int k, SampleShared &sh, u64 *out) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  u64 m = x[0];
#pragma unroll
  for (int e = 1; e < E; ++e) m = umax64(m, x[e]);
  if (t == 0) sh.ncand = 0u;
  sh.cand[t] = m;
  __syncthreads();
  const u64 bw = wave_kth_largest(sh.cand + 64 * wave, m, k);
  if (lane == 0) sh.wbound[wave] = bw;
  __syncthreads();
  u64 B = sh.wbound[0];
#pragma unroll
  for (int w = 1; w < kTileThreads / 64; ++w) B = umax64(B, sh.wbound[w]);
  // B = 0: no wave has k nonempty lanes; every entry is then a candidate
  const u64 lo = B > 0 ? B : 1ull;

  // each wave reserves room for its candidates (one LDS atomic), each lane
  // writes its own at its prefix offset
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) cnt += x[e] >= lo ? 1u : 0u;
  const uint32_t incl = wave_inclusive_scan_u32(cnt);
  const uint32_t wtotal = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  uint32_t wbase = 0u;
  if (lane == 0 && wtotal) wbase = atomicAdd(&sh.ncand, wtotal);
  uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane((int)wbase) + incl - cnt;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (x[e] >= lo) sh.cand[pos++] = x[e];
  __syncthreads();

  const int C = (int)sh.ncand;
  if (t < kRankPad) sh.cand[C + t] = 0ull;
  __syncthreads();
  rank_and_place<kTileThreads, AGENT>(sh.cand, C, k, out, t);
  for (int i = C + t; i < k; i += kTileThreads) {
    if constexpr (AGENT) store_agent(out + i, 0ull);
    else out[i] = 0ull;
  }
}

// Tile `tile` of row `row`: thread t holds logits 1024 j + 4 t + c (j < 8,
// c < 4).  Every load is issued before the first use: eight 16-byte loads
// for a full, aligned tile; otherwise 4-byte loads at indices clamped into
// the tile (always in bounds), the out-of-range ones masked after.
__device__ __forceinline__ void load_tile(const SampleArgs &a, int tile, int row, u64 (&x)[kPerThread]) {
  const int t = threadIdx.x;
  const int64_t first = (int64_t)tile * kTile;
  const int64_t left = a.vocab - first;
  const int nvalid = left < kTile ? (int)left : kTile;
  const float *src = a.logits + (int64_t)row * a.row_stride + first;
  if (a.vec && nvalid == kTile) {
    float4 v[kPerThread / 4];
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j) v[j] = *(const float4 *)(src + 1024 * j + 4 * t);
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j) {
      const uint32_t id = (uint32_t)(first + 1024 * j + 4 * t);
      x[4 * j + 0] = composite(v[j].x, id + 0);
      x[4 * j + 1] = composite(v[j].y, id + 1);
      x[4 * j + 2] = composite(v[j].z, id + 2);
      x[4 * j + 3] = composite(v[j].w, id + 3);
    }
  } else {
    float f[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int i = 1024 * (e >> 2) + 4 * t + (e & 3);
      f[e] = src[i < nvalid ? i : nvalid - 1];
    }
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int i = 1024 * (e >> 2) + 4 * t + (e & 3);
      x[e] = i < nvalid ? composite(f[e], (uint32_t)(first + i)) : 0ull;
    }
  }
}

// Row `row`'s merge (all tiles' lists, read with device-scope loads) and, in
// wave 0, the probabilities, the top-p cut and the draw.
__device__ __forceinline__ void merge_and_draw(const SampleArgs &a, int row, SampleShared &sh) {
  const int t = threadIdx.x, k = a.k, nl = a.tiles * k;
  const u64 *src = a.lists + (int64_t)row * nl;
  constexpr int E = kMaxList / kTileThreads;  // 8
  u64 x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = t + kTileThreads * e;
    x[e] = load_agent(src + (i < nl ? i : nl - 1));
  }
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = t + kTileThreads * e < nl ? x[e] : 0ull;
  block_topk<E, false>(x, k, sh, sh.top);
  __syncthreads();
  if (t >= 64) return;

  const int lane = t;
  const int kc = (int)(k < a.vocab ? k : a.vocab);  // candidates: min(k, V)
  const bool valid = lane < kc;
  const u64 v = valid ? sh.top[lane] : 0ull;
  const int id = (int)(~(uint32_t)v);
  const float z = key_value((uint32_t)(v >> 32));
  const float z0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(z)));
  const float e = valid ? expf((z - z0) * a.inv_temp) : 0.f;
  const float S = wave_sum(e);
  const float p = e / S;
  const float incl_p = wave_inclusive_scan(p);
  const float excl = wave_shift_up1(incl_p);
  const u64 km = __ballot(valid && p > 0.f && excl < a.top_p);
  const int mk = ~km ? __builtin_ctzll(~km) : 64;  // leading run of kept candidates
  const bool in = lane < mk;
  const float ek = in ? e : 0.f;
  const float Sm = wave_sum(ek);
  const float pk = in ? ek / Sm : 0.f;
  const float u = philox_uniform(a.seed, (uint64_t)(a.pos0 + row), a.purpose);
  const float target = u * Sm;
  const float incl_e = wave_inclusive_scan(ek);
  const u64 hit = __ballot(in && target < incl_e);
  const int token = __builtin_amdgcn_readlane(id, hit ? __builtin_ctzll(hit) : mk - 1);

  // agent-scope stores: the acceptance may read them from another XCD
  const int64_t o = (int64_t)row * k;
  if (lane < k) {
    store_agent(a.ids + o + lane, valid ? id : -1);
    store_agent(a.probs + o + lane, pk);
  }
  if (lane == 0) {
    store_agent(a.kept + row, mk);
    store_agent(a.tokens + row, token);
  }
}

// ---------------------------------------------------------------------------
// Acceptance (one wave).
// ---------------------------------------------------------------------------
struct AcceptArgs {
  const int32_t *p_ids;
  const float *p_probs;
  const int32_t *p_kept, *p_tokens;
  const int32_t *q_ids;
  const float *q_probs;
  const int32_t *q_kept, *drafts;
  int32_t *accepted, *out_tokens;
  uint64_t seed;
  int64_t pos0;
  int32_t p_stride, q_stride, n;
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Every load is issued before the first decision: lane i reads row i's kept
// counts, draft and own sample, and each draft row's two lists (the kept
// counts mask them afterwards), so the rows cost one memory round trip
// together instead of two each.  Indices are clamped into the arrays (rows
// past the last draft row reread it) rather than predicated or branched on,
// and nothing is computed from a loaded value until every load is issued.
// R (7 or 15) bounds the draft rows, so eight rows load eight lists.
template <int R>
__device__ void accept_rows(const AcceptArgs &a) {
  const int lane = lane_id();
  const int n = a.n;
  const int lr = lane < n ? lane : n - 1, ld = lane < n - 1 ? lane : n - 2;
  const int lp = lane < a.p_stride ? lane : 0, lq = lane < a.q_stride ? lane : 0;
  const int pk_raw = load_agent(a.p_kept + lr);
  const int tok_l = load_agent(a.p_tokens + lr);
  const int qk_raw = a.q_kept[ld];
  const int d_l = a.drafts[ld];
  int pid[R], qid[R];
  float pp[R], qp[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = i < n - 1 ? i : n - 2;
    pid[i] = load_agent(a.p_ids + (int64_t)row * a.p_stride + lp);
    pp[i] = load_agent(a.p_probs + (int64_t)row * a.p_stride + lp);
    qid[i] = a.q_ids[(int64_t)row * a.q_stride + lq];
    qp[i] = a.q_probs[(int64_t)row * a.q_stride + lq];
  }
  const int pk_l = lane < n ? clampi(pk_raw, 0, a.p_stride) : 0;
  const int qk_l = lane < n - 1 ? clampi(qk_raw, 0, a.q_stride) : 0;
  int acc = n - 1, tok = -1;
  bool done = false;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (done || i >= n - 1) break;
    const int d = __builtin_amdgcn_readlane(d_l, i);
    const int pk = __builtin_amdgcn_readlane(pk_l, i), qk = __builtin_amdgcn_readlane(qk_l, i);
    const bool pin = lane < pk, qin = lane < qk;  // kept counts are at most the strides
    const int pidv = pin ? pid[i] : -1, qidv = qin ? qid[i] : -1;
    const float ppv = pin ? pp[i] : 0.f, qpv = qin ? qp[i] : 0.f;
    const u64 ph = __ballot(pin && pidv == d), qh = __ballot(qin && qidv == d);
    const float pd = ph ? readlane_f(ppv, __builtin_ctzll(ph)) : 0.f;
    const float qd = qh ? readlane_f(qpv, __builtin_ctzll(qh)) : 0.f;
    const float u = philox_uniform(a.seed, (uint64_t)(a.pos0 + i), VA_PURPOSE_ACCEPT);
    if (u * qd < pd) continue;
    // rejected at row i: replacement from max(0, p - q) over the row's kept tokens
    float qt = 0.f;
    bool found = false;
    for (int j = 0; j < qk; ++j) {
      const int id2 = __builtin_amdgcn_readlane(qidv, j);
      const float pr2 = readlane_f(qpv, j);
      if (!found && pidv == id2) qt = pr2, found = true;
    }
    const float r = pin ? fmaxf(0.f, ppv - qt) : 0.f;
    const float Rsum = wave_sum(r);
    if (Rsum > 0.f) {
      const float u2 = philox_uniform(a.seed, (uint64_t)(a.pos0 + i), VA_PURPOSE_RESIDUAL);
      const float incl = wave_inclusive_scan(r);
      const u64 h = __ballot(pin && u2 * Rsum < incl);
      tok = __builtin_amdgcn_readlane(pidv, h ? __builtin_ctzll(h) : pk - 1);
    } else {
      tok = __builtin_amdgcn_readlane(tok_l, i);
    }
    acc = i;
    done = true;
  }
  if (acc == n - 1) tok = __builtin_amdgcn_readlane(tok_l, n - 1);
  for (int i = lane; i < n; i += 64) a.out_tokens[i] = i < acc ? a.drafts[i] : (i == acc ? tok : -1);
  if (lane == 0) *a.accepted = acc;
}

__device__ void accept_wave(const AcceptArgs &a) {
  if (a.n == 1) {  // no draft: the row's own sample
    const int tok = load_agent(a.p_tokens);
    if (lane_id() == 0) *a.out_tokens = tok, *a.accepted = 0;
  } else if (a.n <= 8) {
    accept_rows<7>(a);
  } else {
    accept_rows<VA_SAMPLE_MAX_ROWS - 1>(a);
  }
}

__global__ __launch_bounds__(64) void accept_kernel(const AcceptArgs a) { accept_wave(a); }

// One workgroup per (tile, row).  The last workgroup of a row to finish its
// tile merges the row; with ACCEPT the last row to be merged runs the
// acceptance.  Each hand-off: the writers store with device-scope stores and
// wait for them before a device-scope counter increment; the workgroup that
// sees the final count reads with device-scope loads and resets the counter
// for the next call.
// Naming a value in an empty asm statement forces it into a scalar register
// there: applied to every kernel argument at entry, all argument loads issue
// together in one round trip, not one per first use in a later phase.
__device__ __forceinline__ void pin(int32_t x) { asm volatile("" ::"s"(x)); }
__device__ __forceinline__ void pin(uint32_t x) { asm volatile("" ::"s"(x)); }
__device__ __forceinline__ void pin(int64_t x) { asm volatile("" ::"s"(x)); }
__device__ __forceinline__ void pin(uint64_t x) { asm volatile("" ::"s"(x)); }
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"s"(x)); }
__device__ __forceinline__ void pin(const void *x) { asm volatile("" ::"s"(x)); }

template <bool ACCEPT>
__global__ __launch_bounds__(kTileThreads) void sample_kernel(const SampleArgs ka, const AcceptArgs kacc) {
  SampleArgs a = ka;
  pin(a.logits), pin(a.lists), pin(a.row_count), pin(a.done), pin(a.row_stride), pin(a.vocab), pin(a.k);
  pin(a.tiles), pin(a.rows), pin(a.vec), pin(a.ids), pin(a.probs), pin(a.kept), pin(a.tokens);
  pin(a.inv_temp), pin(a.top_p), pin(a.seed), pin(a.pos0), pin(a.purpose);
  AcceptArgs acc = kacc;
  if constexpr (ACCEPT) {
    pin(acc.p_ids), pin(acc.p_probs), pin(acc.p_kept), pin(acc.p_tokens), pin(acc.q_ids), pin(acc.q_probs);
    pin(acc.q_kept), pin(acc.drafts), pin(acc.accepted), pin(acc.out_tokens), pin(acc.seed), pin(acc.pos0);
    pin(acc.p_stride), pin(acc.q_stride), pin(acc.n);
  }
  __shared__ SampleShared sh;
  const int tile = blockIdx.x, row = blockIdx.y, t = threadIdx.x;
  u64 x[kPerThread];
  load_tile(a, tile, row, x);
  block_topk<kPerThread, true>(x, a.k, sh, a.lists + ((int64_t)row * a.tiles + tile) * a.k);

  wait_stores();
  __syncthreads();
  if (t == 0) sh.flag = atomicAdd(&a.row_count[row], 1u);
  __syncthreads();
  if (sh.flag != (uint32_t)(a.tiles - 1)) return;
  merge_and_draw(a, row, sh);
  if (t == 0) store_agent(a.row_count + row, 0u);

  if constexpr (ACCEPT) {
    wait_stores();
    __syncthreads();
    if (t == 0) sh.flag = atomicAdd(a.done, 1u);
    __syncthreads();
    if (sh.flag != (uint32_t)(a.rows - 1)) return;
    if (t < 64) accept_wave(acc);
    if (t == 0) store_agent(a.done, 0u);
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
inline bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

bool params_ok(const va_sample_params *p) {
  if (!p || p->reserved != 0) return false;
  if (p->rows < 1 || p->rows > VA_SAMPLE_MAX_ROWS) return false;
  if (p->top_k < 1 || p->top_k > VA_SAMPLE_MAX_K) return false;
  if (p->vocab < 1 || p->vocab > VA_SAMPLE_MAX_VOCAB) return false;
  if (p->row_stride < p->vocab) return false;
  if (p->row_stride > ((int64_t)1 << 40)) return false;
  if (!(p->temperature > 0.f) || !isfinite(p->temperature)) return false;
  if (!(p->top_p > 0.f)) return false;  // rejects NaN
  if (p->first_position < 0 || p->first_position > ((int64_t)1 << 62)) return false;
  return true;
}

int tiles_of(const va_sample_params *p) { return (int)((p->vocab + kTile - 1) / kTile); }

size_t workspace_of(const va_sample_params *p) {
  return kListOffset + (size_t)p->rows * tiles_of(p) * p->top_k * sizeof(u64);
}

// Workspace layout: [0, 64) one arrival counter per row, [64, 68) the rows
// counter, lists from byte 256.  The counters are zero between calls.
va_status launch_sample(const va_sample_params *p, const float *logits, int32_t *ids, float *probs, int32_t *kept,
                        int32_t *tokens, void *workspace, size_t workspace_bytes, const AcceptArgs *acc,
                        hipStream_t stream) {
  if (!params_ok(p)) return VA_ERR_INVALID;
  if (!logits || !ids || !probs || !kept || !tokens) return VA_ERR_INVALID;
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(probs, 4) || !aligned(kept, 4) || !aligned(tokens, 4))
    return VA_ERR_INVALID;
  if (!workspace || !aligned(workspace, 16)) return VA_ERR_INVALID;
  if (workspace_bytes < workspace_of(p)) return VA_ERR_WORKSPACE;
  const int tiles = tiles_of(p);
  SampleArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.logits = logits;
  sa.lists = (u64 *)((uint8_t *)workspace + kListOffset);
  sa.row_count = (uint32_t *)workspace;
  sa.done = (uint32_t *)((uint8_t *)workspace + 64);
  sa.row_stride = p->row_stride;
  sa.vocab = p->vocab;
  sa.k = p->top_k;
  sa.tiles = tiles;
  sa.rows = p->rows;
  sa.vec = aligned(logits, 16) && (p->row_stride & 3) == 0;
  sa.ids = ids;
  sa.probs = probs;
  sa.kept = kept;
  sa.tokens = tokens;
  sa.inv_temp = 1.0f / p->temperature;
  sa.top_p = p->top_p;
  sa.seed = p->seed;
  sa.pos0 = p->first_position;
  sa.purpose = p->purpose;
  const dim3 grid(tiles, p->rows), block(kTileThreads);
  if (acc) {
    hipLaunchKernelGGL((sample_kernel<true>), grid, block, 0, stream, sa, *acc);
  } else {
    AcceptArgs none;
    memset(&none, 0, sizeof(none));
    hipLaunchKernelGGL((sample_kernel<false>), grid, block, 0, stream, sa, none);
  }
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

bool accept_ptrs_ok(const int32_t *q_ids, const float *q_probs, const int32_t *q_kept, int32_t q_stride,
                    const int32_t *drafts, int32_t n) {
  if (n < 1 || n > VA_SAMPLE_MAX_ROWS) return false;
  if (n > 1) {
    if (!q_ids || !q_probs || !q_kept || !drafts) return false;
    if (!aligned(q_ids, 4) || !aligned(q_probs, 4) || !aligned(q_kept, 4) || !aligned(drafts, 4)) return false;
    if (q_stride < 1 || q_stride > VA_SAMPLE_MAX_K) return false;
  }
  return true;
}

}  // namespace va_sample_detail
using namespace va_sample_detail;

extern "C" size_t va_sample_workspace_bytes(const va_sample_params *params) {
  return params_ok(params) ? workspace_of(params) : 0;
}

extern "C" va_status va_sample(const va_sample_params *params, const float *logits, int32_t *ids, float *probs,
                               int32_t *kept, int32_t *tokens, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return launch_sample(params, logits, ids, probs, kept, tokens, workspace, workspace_bytes, nullptr, stream);
}

extern "C" va_status va_accept(const int32_t *p_ids, const float *p_probs, const int32_t *p_kept,
                               const int32_t *p_tokens, int32_t p_stride, const int32_t *q_ids, const float *q_probs,
                               const int32_t *q_kept, int32_t q_stride, const int32_t *drafts, int32_t n,
                               uint64_t seed, int64_t first_position, int32_t *accepted, int32_t *out_tokens,
                               hipStream_t stream) {
  if (!accept_ptrs_ok(q_ids, q_probs, q_kept, q_stride, drafts, n)) return VA_ERR_INVALID;
  if (!p_ids || !p_probs || !p_kept || !p_tokens || !accepted || !out_tokens) return VA_ERR_INVALID;
  if (!aligned(p_ids, 4) || !aligned(p_probs, 4) || !aligned(p_kept, 4) || !aligned(p_tokens, 4) ||
      !aligned(accepted, 4) || !aligned(out_tokens, 4))
    return VA_ERR_INVALID;
  if (p_stride < 1 || p_stride > VA_SAMPLE_MAX_K) return VA_ERR_INVALID;
  if (first_position < 0 || first_position > ((int64_t)1 << 62)) return VA_ERR_INVALID;
  AcceptArgs a;
  a.p_ids = p_ids;
  a.p_probs = p_probs;
  a.p_kept = p_kept;
  a.p_tokens = p_tokens;
  a.q_ids = q_ids;
  a.q_probs = q_probs;
  a.q_kept = q_kept;
  a.drafts = drafts;
  a.accepted = accepted;
  a.out_tokens = out_tokens;
  a.seed = seed;
  a.pos0 = first_position;
  a.p_stride = p_stride;
  a.q_stride = n > 1 ? q_stride : 1;
  a.n = n;
  hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

extern "C" va_status va_sample_accept(const va_sample_params *params, const float *logits, const int32_t *q_ids,
                                      const float *q_probs, const int32_t *q_kept, int32_t q_stride,
                                      const int32_t *drafts, int32_t *ids, float *probs, int32_t *kept,
                                      int32_t *tokens, int32_t *accepted, int32_t *out_tokens, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (!params_ok(params)) return VA_ERR_INVALID;
  const int n = params->rows;
  if (!accept_ptrs_ok(q_ids, q_probs, q_kept, q_stride, drafts, n)) return VA_ERR_INVALID;
  if (!accepted || !out_tokens || !aligned(accepted, 4) || !aligned(out_tokens, 4)) return VA_ERR_INVALID;
  AcceptArgs a;
  a.p_ids = ids;
  a.p_probs = probs;
  a.p_kept = kept;
  a.p_tokens = tokens;
  a.q_ids = q_ids;
  a.q_probs = q_probs;
  a.q_kept = q_kept;
  a.drafts = drafts;
  a.accepted = accepted;
  a.out_tokens = out_tokens;
  a.seed = params->seed;
  a.pos0 = params->first_position;
  a.p_stride = params->top_k;
  a.q_stride = n > 1 ? q_stride : 1;
  a.n = n;
  return launch_sample(params, logits, ids, probs, kept, tokens, workspace, workspace_bytes, &a, stream);
}
