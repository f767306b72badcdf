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
//   topk_tile_kernel     grid (tiles, rows) x 256 threads: one tile's exact
//                        top-k as a sorted list of 64-bit composites.
//   sample_finish_kernel grid rows x 64: merge of a row's tile lists, softmax,
//                        top-p, the draw; with ACCEPT the last row to finish
//                        also runs the acceptance.
//   accept_kernel        one wave: the acceptance alone.
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

__device__ __forceinline__ int bits_below(u64 mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ u64 umax64(u64 a, u64 b) { return a > b ? a : b; }

// The k-th largest of the 64 lanes' values (1 <= k <= 64), or 0 when fewer
// than k lanes hold a value >= 1.  The count of lanes reaching c falls as c
// grows, so the largest c reached by k lanes -- the answer -- is built bit by
// bit from the top.
__device__ __forceinline__ u64 wave_kth_largest(u64 v, int k) {
  u64 t = 0;
#pragma unroll 8
  for (int b = 63; b >= 0; --b) {
    const u64 c = t | (1ull << b);
    if (__popcll(__ballot(v >= c)) >= k) t = c;
  }
  return t;
}

// Butterfly sum: every lane gets the same value in the same order.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// Inclusive prefix sum over lanes (Hillis-Steele).
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
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
// Tile scan.
// ---------------------------------------------------------------------------
struct TileArgs {
  const float *logits;
  u64 *lists;         // [rows][tiles][k]
  uint32_t *counter;  // zeroed here when the call accepts, else NULL
  int64_t row_stride, vocab;
  int32_t k, tiles;
  int32_t vec;  // rows start 16-byte aligned: 16-byte loads
};

// One workgroup per (tile, row).  Thread t holds logits 1024 j + 4 t + c
// (j < 8, c < 4): eight coalesced 16-byte loads (4-byte loads when rows do
// not start on 16 bytes).  The tile's top-k is found
// without sorting the tile:
//   1. each wave takes B_w, the k-th largest of its 64 lanes' maxima: at
//      least k of the wave's elements reach B_w, so the tile's k-th largest
//      does too, and so does B = max_w B_w;
//   2. the elements >= B (typically a few more than k) are gathered in LDS;
//   3. each candidate's rank is the number of larger candidates; ranks below
//      k are written in order.
__global__ __launch_bounds__(kTileThreads) void topk_tile_kernel(const TileArgs a) {
  __shared__ u64 cand[kTile];
  __shared__ u64 wbound[kTileThreads / 64];
  __shared__ uint32_t ncand;
  const int tile = blockIdx.x, row = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int k = a.k;
  if (t == 0) {
    ncand = 0u;
    if (a.counter && tile == 0 && row == 0) *a.counter = 0u;
  }
  const int64_t first = (int64_t)tile * kTile;
  const int64_t left = a.vocab - first;
  const int nvalid = left < kTile ? (int)left : kTile;
  const float *src = a.logits + (int64_t)row * a.row_stride + first;

  u64 x[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread / 4; ++j) {
    const int base = 1024 * j + 4 * t;
    float f[4];
    if (a.vec && base + 4 <= nvalid) {
      const float4 v = *(const float4 *)(src + base);
      f[0] = v.x, f[1] = v.y, f[2] = v.z, f[3] = v.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) f[c] = base + c < nvalid ? src[base + c] : 0.f;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      x[4 * j + c] = base + c < nvalid ? composite(f[c], (uint32_t)(first + base + c)) : 0ull;
  }

  u64 m = x[0];
#pragma unroll
  for (int e = 1; e < kPerThread; ++e) m = umax64(m, x[e]);
  const u64 bw = wave_kth_largest(m, k);
  if (lane == 0) wbound[wave] = bw;
  __syncthreads();
  u64 B = wbound[0];
#pragma unroll
  for (int w = 1; w < kTileThreads / 64; ++w) B = umax64(B, wbound[w]);
  // B = 0: no wave has k valid lanes; every valid element is then a candidate
  const u64 lo = B > 0 ? B : 1ull;

  int cnt = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) cnt += __popcll(__ballot(x[e] >= lo));
  uint32_t base = 0;
  if (lane == 0 && cnt) base = atomicAdd(&ncand, (uint32_t)cnt);
  base = __shfl(base, 0);
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool in = x[e] >= lo;
    const u64 msk = __ballot(in);
    if (in) cand[base + bits_below(msk)] = x[e];
    base += (uint32_t)__popcll(msk);
  }
  __syncthreads();

  const int C = (int)ncand;
  u64 *out = a.lists + ((int64_t)row * a.tiles + tile) * k;
  for (int i = t; i < C; i += kTileThreads) {
    const u64 v = cand[i];
    int r = 0;
    for (int j = 0; j < C; ++j) r += cand[j] > v ? 1 : 0;
    if (r < k) out[r] = v;
  }
  for (int i = C + t; i < k; i += kTileThreads) out[i] = 0ull;  // a tile with fewer than k logits
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

__device__ void accept_wave(const AcceptArgs &a) {
  const int lane = lane_id();
  const int n = a.n;
  int acc = n - 1, tok = -1;
  for (int i = 0; i < n - 1; ++i) {
    const int d = a.drafts[i];
    const int pk = clampi(a.p_kept[i], 0, a.p_stride), qk = clampi(a.q_kept[i], 0, a.q_stride);
    const int pid = lane < pk ? a.p_ids[(int64_t)i * a.p_stride + lane] : -1;
    const float pp = lane < pk ? a.p_probs[(int64_t)i * a.p_stride + lane] : 0.f;
    const int qid = lane < qk ? a.q_ids[(int64_t)i * a.q_stride + lane] : -1;
    const float qp = lane < qk ? a.q_probs[(int64_t)i * a.q_stride + lane] : 0.f;
    const u64 ph = __ballot(lane < pk && pid == d), qh = __ballot(lane < qk && qid == d);
    const float pd = ph ? __shfl(pp, __builtin_ctzll(ph)) : 0.f;
    const float qd = qh ? __shfl(qp, __builtin_ctzll(qh)) : 0.f;
    const float u = philox_uniform(a.seed, (uint64_t)(a.pos0 + i), VA_PURPOSE_ACCEPT);
    if (u * qd < pd) continue;
    // rejected at row i: replacement from max(0, p - q) over the row's kept tokens
    float qt = 0.f;
    bool found = false;
    for (int j = 0; j < qk; ++j) {
      const int id2 = __shfl(qid, j);
      const float pr2 = __shfl(qp, j);
      if (!found && pid == id2) qt = pr2, found = true;
    }
    const float r = lane < pk ? fmaxf(0.f, pp - qt) : 0.f;
    const float R = wave_sum(r);
    if (R > 0.f) {
      const float u2 = philox_uniform(a.seed, (uint64_t)(a.pos0 + i), VA_PURPOSE_RESIDUAL);
      const float incl = wave_inclusive_scan(r);
      const u64 h = __ballot(lane < pk && u2 * R < incl);
      tok = __shfl(pid, h ? __builtin_ctzll(h) : pk - 1);
    } else {
      tok = a.p_tokens[i];
    }
    acc = i;
    break;
  }
  if (acc == n - 1) tok = a.p_tokens[n - 1];
  for (int i = lane; i < n; i += 64) a.out_tokens[i] = i < acc ? a.drafts[i] : (i == acc ? tok : -1);
  if (lane == 0) *a.accepted = acc;
}

__global__ __launch_bounds__(64) void accept_kernel(const AcceptArgs a) { accept_wave(a); }

// ---------------------------------------------------------------------------
// Per-row merge, probabilities, top-p and the draw.
// ---------------------------------------------------------------------------
struct FinishArgs {
  const u64 *lists;
  uint32_t *counter;
  int32_t *ids;
  float *probs;
  int32_t *kept, *tokens;
  float inv_temp, top_p;
  uint64_t seed;
  int64_t pos0;
  uint32_t purpose;
  int32_t rows, k, tiles;
  AcceptArgs acc;  // ACCEPT only
};

// One wave per row.  The row's tile lists (tiles x k composites, each list
// sorted) are merged like a tile: B = the k-th largest of the lanes' maxima
// bounds the k-th largest overall, the entries >= B are ranked by counting.
template <bool ACCEPT>
__global__ __launch_bounds__(64) void sample_finish_kernel(const FinishArgs a) {
  __shared__ u64 cand[kMaxList];
  __shared__ u64 top[kMaxK];
  const int row = blockIdx.x, lane = threadIdx.x;
  const int k = a.k, nl = a.tiles * k;
  const u64 *src = a.lists + (int64_t)row * nl;

  u64 x[kListPerLane];
#pragma unroll
  for (int e = 0; e < kListPerLane; ++e) {
    const int i = lane + 64 * e;
    x[e] = i < nl ? src[i] : 0ull;
  }
  u64 m = x[0];
#pragma unroll
  for (int e = 1; e < kListPerLane; ++e) m = umax64(m, x[e]);
  const u64 B = wave_kth_largest(m, k);
  const u64 lo = B > 0 ? B : 1ull;
  int C = 0;
#pragma unroll
  for (int e = 0; e < kListPerLane; ++e) {
    const bool in = x[e] >= lo;
    const u64 msk = __ballot(in);
    if (in) cand[C + bits_below(msk)] = x[e];
    C += __popcll(msk);
  }
  __syncthreads();
  for (int i = lane; i < C; i += 64) {
    const u64 v = cand[i];
    int r = 0;
    for (int j = 0; j < C; ++j) r += cand[j] > v ? 1 : 0;
    if (r < k) top[r] = v;
  }
  __syncthreads();

  const int kc = C < k ? C : k;  // min(k, V) candidates
  const bool valid = lane < kc;
  const u64 v = valid ? top[lane] : 0ull;
  const int id = (int)(~(uint32_t)v);
  const float z = key_value((uint32_t)(v >> 32));
  const float z0 = __shfl(z, 0);
  const float e = valid ? expf((z - z0) * a.inv_temp) : 0.f;
  const float S = wave_sum(e);
  const float p = e / S;
  const float incl_p = wave_inclusive_scan(p);
  float excl = __shfl_up(incl_p, 1);
  excl = lane == 0 ? 0.f : excl;
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
  const int token = __shfl(id, hit ? __builtin_ctzll(hit) : mk - 1);

  const int64_t o = (int64_t)row * k;
  if (lane < k) {
    a.ids[o + lane] = valid ? id : -1;
    a.probs[o + lane] = pk;
  }
  if (lane == 0) {
    a.kept[row] = mk;
    a.tokens[row] = token;
  }

  if constexpr (ACCEPT) {
    // The last row to get here runs the acceptance over every row's outputs:
    // release this row's stores before counting, acquire the others' after.
    __threadfence();
    uint32_t prev = 0u;
    if (lane == 0) prev = atomicAdd(a.counter, 1u);
    prev = __shfl(prev, 0);
    if (prev != (uint32_t)(a.rows - 1)) return;
    __threadfence();
    accept_wave(a.acc);
    if (lane == 0) *a.counter = 0u;
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
  uint32_t *counter = (uint32_t *)workspace;
  u64 *lists = (u64 *)((uint8_t *)workspace + kListOffset);

  TileArgs ta;
  ta.logits = logits;
  ta.lists = lists;
  ta.counter = acc ? counter : nullptr;
  ta.row_stride = p->row_stride;
  ta.vocab = p->vocab;
  ta.k = p->top_k;
  ta.tiles = tiles;
  ta.vec = aligned(logits, 16) && (p->row_stride & 3) == 0;
  hipLaunchKernelGGL(topk_tile_kernel, dim3(tiles, p->rows), dim3(kTileThreads), 0, stream, ta);
  if (hipGetLastError() != hipSuccess) return VA_ERR_HIP;

  FinishArgs fa;
  memset(&fa, 0, sizeof(fa));
  fa.lists = lists;
  fa.counter = counter;
  fa.ids = ids;
  fa.probs = probs;
  fa.kept = kept;
  fa.tokens = tokens;
  fa.inv_temp = 1.0f / p->temperature;
  fa.top_p = p->top_p;
  fa.seed = p->seed;
  fa.pos0 = p->first_position;
  fa.purpose = p->purpose;
  fa.rows = p->rows;
  fa.k = p->top_k;
  fa.tiles = tiles;
  if (acc) {
    fa.acc = *acc;
    hipLaunchKernelGGL((sample_finish_kernel<true>), dim3(p->rows), dim3(64), 0, stream, fa);
  } else {
    hipLaunchKernelGGL((sample_finish_kernel<false>), dim3(p->rows), dim3(64), 0, stream, fa);
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
