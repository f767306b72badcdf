// Multi-row speculative-verification decode attention for gfx950 (CDNA4).
//
// Kernels:
//   split_kernel    one workgroup per (split, KV head); one wave64 per 16
//                   query matrix rows walks the split's 32-key chunks, which
//                   one or two producer waves stream into a ring of LDS
//                   stages by LDS DMA (for quantised caches two decoder
//                   waves convert each staged chunk to bf16 tiles); QK^T and PV
//                   run on MFMA 16x16x32 bf16 with FP32 accumulation; each
//                   wave writes its rows' partials (m, l, O) directly.
//   combine_kernel  one workgroup per (row, query head, 32-wide slice of D):
//                   LSE merge of the partials plus the sink, with the partial
//                   loads issued together into four independent FP32 chains
//                   per thread.
//   ring_write_kernel  copies the verification rows' K/V into the window ring.
//   kv_write_kernel    writes the rows' K/V into a linear cache or the ring,
//                      bf16 or encoded (rotated E4M3 keys, INT8 values with a
//                      per-token scale).
//
// The method is the one on the IQuestRT report's section "Read only the KV
// tiles needed by the current positions" (eight rows x six heads packed as
// 48 matrix rows against one KV head, sequence splits, causal mask only at
// the boundary, zero-value sink, separate combine with four FP32 chains,
// 4,096 + 64-slot ring written before the read) and on "Qwen3.8-27B on one
// RTX 4090" (tree mask; FP8 keys after a Hadamard rotation and INT8 values).
// The data movement below is designed for CDNA4, not taken from the pages.
//
// MFMA layout used throughout (v_mfma_f32_16x16x32_bf16, wave64, lane l,
// i = l % 16, g = l / 16):
//   A operand: row i, contraction elements 8g..8g+7
//   B operand: column i, contraction elements 8g..8g+7
//   C/D:       column i, rows 4g..4g+3
// Scores are computed transposed, S^T = K * Q^T (rows = keys, columns = query
// matrix rows), so the C layout of S^T is directly the B operand of
// O^T = V^T * P^T once each lane's keys are read in the order
// {4g..4g+3, 16+4g..16+4g+3}; the same key order is used for V^T.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "plan_data.h"
#include "verify_attn.h"

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
typedef float f32x2 __attribute__((__vector_size__(8)));

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f

namespace va_detail {

constexpr int kChunk = 32;  // keys per step
static_assert(kChunk == VA_SPLIT_KEYS, "a split is a whole number of chunks");
constexpr float kTau = 8.f;  // lazy-rescale threshold (log2 units)

struct SplitArgs {
  const uint8_t *q;  // bf16 [rows, Hq, D]
  const uint8_t *k;
  const uint8_t *v;
  const float *v_scale;
  float *ws_ml;
  float *ws_o;
  int64_t kv_head_stride_b;  // bytes
  int64_t kv_row_stride_b;   // bytes
  int64_t v_scale_head_stride;
  int64_t base;  // absolute position of relative key 0 (= chunk_lo * 32)
  int32_t rows, live_rows, group, mrows, q_heads, kv_heads;
  float inv_group;           // 1 / group (row of matrix row m: (m + 0.5) * inv_group)
  int32_t splits, chunks_q, chunks_r;  // chunks / splits, chunks % splits
  int32_t rel_lo, rel_hi;    // read extent, relative to base
  int32_t full_lo, full_hi;  // every live row sees these keys (relative)
  int32_t ring_slots, ring_base_slot;
  int32_t tree, tree_lo;     // tree mode: relative position of node 0's key
  float scale_log2;          // scale * log2(e)
  // Row geometry, relative to base.  Chain modes: row r sits at t0_rel + r and
  // sees [max(t0_rel + r - window + 1, 0), t0_rel + r] (window = 0: from 0).
  // Tree mode: every live row sees [0, tree_lo) plus the node keys whose
  // bits are set in anc[r].
  int32_t t0_rel, window;
  uint32_t anc[VA_MAX_ROWS];
  // Per-call state in device memory (the state entry points): the fields
  // above that depend on positions or rows are then derived from it.
  const va_state *state;
  int64_t bucket_hi;  // the plan's extent end: no state may read beyond it
  // Append (bf16): the rows' own K/V, [rows, Hkv, D] bf16 with
  // new_row_stride_b bytes between rows (NULL: no append).  Split 0 stores
  // every row to the slot of its own key (ring: mod ring_slots; a linear
  // cache: below kv_capacity only); the workgroups whose chunks hold the
  // live rows' keys put the new rows into their staged tiles.
  const uint8_t *k_new, *v_new;
  int64_t new_row_stride_b;
  int64_t kv_capacity;
  int64_t append_pos0;  // absolute position of row 0's key (first_pos, or prefix_len for a tree)
};

struct CombineArgs {
  const float *ws_ml;
  const float *ws_o;
  const float *sink;
  float *out;
  float *lse;
  int32_t rows, live_rows, group, mrows, q_heads, kv_heads, splits, head_dim;
  const va_state *state;  // as in SplitArgs
  int32_t tree, window, ring_slots;
  int64_t bucket_hi;
};

// Per-call geometry derived from a va_state on the device, with the same
// rules as the host plan (row intervals, read extent, 32-key split table,
// ancestor bits) and the split kernel's relative coordinates.
struct StateGeo {
  int64_t base;
  int64_t pos0;  // absolute position of row 0's key (first_pos, or prefix_len for a tree)
  int32_t rel_lo, rel_hi, full_lo, full_hi, cq, cr, splits, live_rows, ring_base, t0_rel, tree_lo;
  uint32_t anc[VA_MAX_ROWS];
  bool valid;
};

__device__ __forceinline__ StateGeo geo_from_state(const va_state *stp, int32_t rows, int32_t tree, int32_t window,
                                                   int32_t ring_slots, int32_t splits_plan, int64_t bucket_hi) {
  const va_state st = *stp;
  StateGeo g;
  const int32_t live = st.live_rows;
  const int64_t fp = st.first_pos, P = st.prefix_len;
  const int64_t kMaxPos = (int64_t)1 << 61;
  bool valid = st.reserved == 0 && live >= 0 && live <= rows;
  int64_t lo = 0, hi = 0, flo = 0, fhi = 0;
  uint32_t anc[VA_MAX_ROWS];
#pragma unroll
  for (int i = 0; i < VA_MAX_ROWS; ++i) anc[i] = 0u;
  if (tree) {
    valid = valid && P >= 0 && P <= kMaxPos;
#pragma unroll
    for (int i = 0; i < VA_MAX_ROWS; ++i) {
      const int32_t pa = st.parent[i];
      if (i < rows) valid = valid && pa >= -1 && pa < i;
      // parents precede their children, so anc[pa] is final here
      uint32_t bits = 1u << i;
#pragma unroll
      for (int j = 0; j < i; ++j) bits |= (pa == j) ? anc[j] : 0u;
      anc[i] = bits;
    }
#pragma unroll
    for (int i = 0; i < VA_MAX_ROWS; ++i) anc[i] = i < live ? anc[i] : 0u;
    lo = 0;
    hi = P + live;
    flo = 0;
    fhi = P;
  } else {
    valid = valid && fp >= 0 && fp <= kMaxPos;
    lo = window ? fp - window + 1 : 0;
    if (lo < 0) lo = 0;
    hi = fp + live;
    flo = window ? fp + live - 1 - window + 1 : 0;
    if (flo < 0) flo = 0;
    fhi = fp + 1;
  }
  if (live == 0) lo = hi = flo = fhi = 0;
  valid = valid && hi <= bucket_hi;
  const int64_t chunk_lo = lo >> 5;
  const int64_t chunks = live > 0 ? ((hi + 31) >> 5) - chunk_lo : 0;
  const int32_t S = (int32_t)(chunks < splits_plan ? (chunks > 0 ? chunks : 1) : splits_plan);
  g.base = chunk_lo << 5;
  g.splits = S;
  g.cq = (int32_t)(chunks / S);
  g.cr = (int32_t)(chunks % S);
  g.rel_lo = (int32_t)(lo - g.base);
  g.rel_hi = (int32_t)(hi - g.base);
  int32_t rflo = (int32_t)(flo - g.base), rfhi = (int32_t)(fhi - g.base);
  if (flo - g.base < g.rel_lo) rflo = g.rel_lo;
  if (fhi - g.base > g.rel_hi) rfhi = g.rel_hi;
  if (rfhi < rflo) rfhi = rflo;
  g.full_lo = rflo;
  g.full_hi = rfhi;
  g.ring_base = ring_slots ? (int32_t)(g.base % ring_slots) : 0;
  g.t0_rel = tree ? 0 : (int32_t)(fp - g.base);
  // tree: base is 0 and P < hi <= the bucket's hi < 2^31; unused otherwise
  g.tree_lo = tree ? (int32_t)P : 0;
  g.pos0 = tree ? P : fp;
  g.live_rows = live;
#pragma unroll
  for (int i = 0; i < VA_MAX_ROWS; ++i) g.anc[i] = anc[i];
  g.valid = valid;
  return g;
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Reductions over the four lanes l, l^16, l^32, l^48 (the lanes that share
// lane % 16), on the VALU: v_permlane32_swap pairs each lane with lane ^ 32,
// v_permlane16_swap with lane ^ 16 (each returns the lane's own value in one
// output and its partner's in the other).  Every lane gets the same result
// (IEEE max and + are commutative).
__device__ __forceinline__ float wave_max16x4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum16x4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Two E4M3FN codes (bytes 0-1, or 2-3 with hi) -> two bf16, exact (the gfx950
// scaled converter with scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// LDS DMA: lane l copies `bytes` from its global address to lds + bytes*l
// (the LDS base is wave-uniform, an LDS byte address).  Kept out of the
// kernel templates: the builtin exists only for the device.  The LDS
// address travels as an integer: a generic pointer cast to LDS at every
// call costs a null test and a select per instruction.
__device__ __forceinline__ uint32_t lds_addr(const void *shared_array) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)shared_array;
}
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(uintptr_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, uint32_t lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(uintptr_t)lds, 4, 0, 0);
}
// A 32-bit per-lane offset, opaque to the compiler at each use: added to a
// wave-uniform base it selects the DMA's scalar-base form (base in SGPRs,
// offset in one VGPR) instead of a 64-bit address add per instruction.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, output lane n, element e is the (n % 4)-th 16-bit value of the 8
// bytes addressed by lane 4e + n/4 of that group.  (Layout checked on the
// GPU with an in-bounds probe.)
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const void *p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)p);
  return __builtin_bit_cast(u32x2, r);
}

// ---------------------------------------------------------------------------
// Split kernel: one workgroup per (split, KV head) with W + NDW + NPW wave64s.
//   Consumers, waves 0..W-1: wave w owns query matrix rows [16w, 16w + 16)
//     for the whole split and keeps their online-softmax state in registers;
//     every consumer walks all of the split's 32-key chunks in order.
//   Decoders (quantised formats, NDW = 2), waves W..W+NDW-1: convert each
//     staged chunk to bf16 tiles one chunk ahead of the consumers, half of
//     it each.  Waves go to the four SIMDs in turn, so with six consumers
//     the two decoders share the two SIMDs that hold one consumer each, and
//     the conversion overlaps the consumers' steps.
//   Producers, waves W+NDW..W+NDW+NPW-1: fill a ring of NST LDS stages (chunk j in
//     stage j % NST) with the chunks' K and V tiles by LDS DMA, NST - 1
//     chunks ahead of the consumers; each producer issues its share of every
//     chunk's DMA instructions.
// One workgroup barrier per chunk both publishes chunk n (each producer waited
// for its share of the DMA just before) and frees the stage of chunk n - 1,
// which the producers refill right after.  No cross-wave merge: each
// consumer writes its own rows' partials.
//   D    head dim (64 or 128)
//   W    16-row blocks of query matrix rows (1..6)
//   FMT  0 = bf16 K/V; 1 = E4M3FN rotated K, INT8 V with per-key scale
//   NST  LDS stages
//   NPW  producer waves
// ---------------------------------------------------------------------------
template <int D, int FMT>
struct StageGeom {
  static constexpr int KROW = FMT == 0 ? D * 2 : D;      // bytes per key row
  static constexpr int PIECES = KROW / 16;               // 16-byte pieces per row
  static constexpr int RPI = 64 / PIECES;                // rows per DMA instruction (1 KiB)
  static constexpr int NDMA = kChunk / RPI;              // DMA instructions per tile
  static constexpr int kTileB = kChunk * KROW;
  static constexpr int kScaleB = FMT == 1 ? 256 : 0;
  static constexpr int kStageB = 2 * kTileB + kScaleB;
  static constexpr int kVm = 2 * NDMA + (FMT == 1 ? 1 : 0);  // DMA instructions per chunk
  // Piece swizzles of the staged tiles: piece P of row r sits at position
  // P ^ f(r).  K: f = r mod PIECES, so the 16 lanes reading one A operand
  // (16 keys, one piece) hit 16 different positions.  V (bf16): an even f,
  // so a pair of pieces {2k, 2k+1} stays a pair, the same for rows r and
  // r + 16, and spreading the 16 rows of one transpose read over all bank
  // groups: 2r mod PIECES for 256-byte rows; r mod 8 with its low bit
  // cleared for 128-byte rows, where two rows share a 256-byte bank window
  // and 2r mod 8 would put rows r and r + 4 on the same banks (a two-way
  // conflict on every transpose read).  V (INT8) is read bytewise,
  // unswizzled.  K codes (E4M3, eight pieces a row) are read only by the
  // decoders, a lane taking pieces 2k and 2k + 1 of one row: r mod 8 with
  // its low bit flipped when bit 1 of r is set puts each load's 16 lanes
  // (four rows) on 16 different bank groups.
  static __device__ constexpr int fk(int row) {
    return FMT != 0 ? ((row & 7) ^ ((row >> 1) & 1)) : row & (PIECES - 1);
  }
  static __device__ constexpr int fv(int row) {
    return FMT != 0 ? 0 : (PIECES == 8 ? row & 6 : (2 * row) & (PIECES - 2));
  }
};

// s_waitcnt vmcnt(KV * k) for a run-time k in [0, K] (the count is an
// immediate, so each value has its own instruction).
template <int KV, int K>
__device__ __forceinline__ void wait_chunks(int k) {
  if constexpr (K > 0) {
    if (k >= K) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KV * K) : "memory");
      return;
    }
    wait_chunks<KV, K - 1>(k);
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Kernel arguments live in memory and reach SGPRs through scalar loads; the
// compiler issues each load where the value is first needed, so arguments
// used in different places cost separate round trips.  Naming every argument
// in an empty asm statement at the kernel's entry makes all of those loads
// issue together, in one round trip.
__device__ __forceinline__ void pin(int32_t x) { asm volatile("" ::"s"(x)); }
__device__ __forceinline__ void pin(uint32_t x) { asm volatile("" ::"s"(x)); }
__device__ __forceinline__ void pin(int64_t x) { asm volatile("" ::"s"(x)); }
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"s"(x)); }
__device__ __forceinline__ void pin(const void *x) { asm volatile("" ::"s"(x)); }

// Phase trace (builds with VA_PHASE_TRACE only; see include/verify_probe.h):
// lane 0 of a chosen wave stores the 100 MHz constant-rate clock
// (s_memrealtime, the same on every CU) into slot `slot` of its workgroup's
// record.  Records: split_kernel 24 slots per workgroup (phases, then each
// role's waits), combine_kernel 8.
#ifdef VA_PHASE_TRACE
constexpr int kTraceWG = 8192;
constexpr int va_trace_split_len = 24, va_trace_comb_len = 8;
__device__ uint64_t va_trace_split[kTraceWG * va_trace_split_len];
__device__ uint64_t va_trace_comb[kTraceWG * va_trace_comb_len];
__device__ __forceinline__ uint64_t trace_now() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ void trace_put(uint64_t *rec, int len, int slot, uint64_t v, bool lane0) {
  const int wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  if (lane0 && wg < kTraceWG && slot < len) rec[wg * len + slot] = v;
}
#define VA_TRACE(rec, slot, lane0) trace_put(rec, rec##_len, slot, trace_now(), lane0)
#define VA_TRACE_VAL(rec, slot, v, lane0) trace_put(rec, rec##_len, slot, v, lane0)
#else
#define VA_TRACE(rec, slot, lane0) ((void)0)
#define VA_TRACE_VAL(rec, slot, v, lane0) ((void)0)
#endif

// Decoder waves of the quantised formats.
template <int FMT>
constexpr int decoders_for() { return FMT == 1 ? 2 : 0; }

template <int D, int W, int FMT, int NST, int NPW, bool STATE, bool APP, int RG>
__global__ __launch_bounds__(64 * (W + NPW + decoders_for<FMT>())) void split_kernel(const SplitArgs a) {
  static_assert(!APP || (FMT == 0 && NPW == 2), "append: bf16 tiles, one producer per tile kind");
#ifdef VA_PHASE_TRACE
  const uint64_t t_entry = trace_now();
#endif
  using G = StageGeom<D, FMT>;
  constexpr int KS = D / 32;  // QK contraction steps
  constexpr int MD = D / 16;  // O^T row blocks over d
  constexpr int KROW = G::KROW, PIECES = G::PIECES, RPI = G::RPI, NDMA = G::NDMA;
  constexpr int kTileB = G::kTileB, kStageB = G::kStageB, kVm = G::kVm;
  static_assert(NST >= 2, "a ring of at least two stages");
  constexpr int NDW = decoders_for<FMT>();
  constexpr int U = 2 * NDMA / NPW;           // DMA instructions per chunk and producer
  constexpr int kVmP = U + (FMT == 1 ? 1 : 0);  // the same, with the quantised scales
  static_assert(FMT == 0 || NPW == 1, "the scale DMA belongs to a single producer");
  static_assert((2 * NDMA) % NPW == 0, "producers share a chunk's DMA evenly");
  static_assert((NST - 2) * kVmP <= 63, "vmcnt counts at most 63 loads");
  static_assert(FMT == 0 || NST >= 3, "the quantised pipeline stages one chunk ahead of the decode");
  // Quantised formats: the decoder waves convert every chunk once into bf16
  // tiles (two buffers, [K | V]); each consumer then reads bf16 operands as
  // for bf16 caches instead of converting the whole chunk itself.
  constexpr int kDecRow = 2 * D;                         // bf16 bytes per key row
  constexpr int kDecTile = kChunk * kDecRow;             // one decoded K or V tile
  constexpr int kDecB = FMT == 1 ? 2 * 2 * kDecTile : 0;  // two buffers of K and V
  __shared__ __attribute__((aligned(16))) uint8_t smem[kDecB + NST * kStageB];
  // The decoded tiles sit at the start of LDS, below 64 KiB, so the
  // consumers' reads of them take their buffer offset as an instruction
  // immediate; the staged ring follows.
  uint8_t *const ring = smem + kDecB;
  const uint32_t ring_lds = lds_addr(smem) + kDecB;  // the ring as an LDS byte address

  const int lane = threadIdx.x & 63;
  // wave-uniform: keeps chunk indices and mask decisions in scalar registers
  // Roles by hardware wave: the producers first (a workgroup's waves start
  // in order, and the producers' first DMA is what every other wave waits
  // for), then the decoders, then the consumers; `wave` is the role index
  // (consumers 0 .. W-1, decoders W .. W+NDW-1, producers after).
  const int hw_wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = hw_wave < NPW ? W + NDW + hw_wave : (hw_wave < NPW + NDW ? W + hw_wave - NPW : hw_wave - NPW - NDW);
  const int i16 = lane & 15;
  const int g4 = lane >> 4;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;

  // ---------------- this split's chunk range ----------------
  // split s takes q + 1 chunks if s < r, else q (q = C / S, r = C % S)
  int32_t cq = a.chunks_q, cr = a.chunks_r, rel_lo = a.rel_lo, rel_hi = a.rel_hi;
  const int32_t ring_slots = a.ring_slots;
  int32_t ring_base = a.ring_base_slot;
  int64_t kv_base = a.base;
  int64_t append_pos0 = a.append_pos0;
  const int64_t row_stride = a.kv_row_stride_b, head_stride = a.kv_head_stride_b;
  const uint8_t *kptr = a.k, *vptr = a.v;
  const float *vsc = a.v_scale;
  const int64_t vsc_stride = a.v_scale_head_stride;
  const float inv_group = a.inv_group, scale_log2 = a.scale_log2;
  const int32_t mrows = a.mrows, group = a.group, q_heads = a.q_heads;
  int32_t live_rows = a.live_rows;
  const int32_t tree = a.tree, window = a.window;
  int32_t tree_lo = a.tree_lo, t0_rel = a.t0_rel;
  int32_t full_lo = a.full_lo, full_hi = a.full_hi;
  const int32_t kv_heads = a.kv_heads;
  const uint8_t *qptr = a.q;
  float *ws_ml = a.ws_ml, *ws_o = a.ws_o;
  uint32_t anc[VA_MAX_ROWS];
#pragma unroll
  for (int i = 0; i < VA_MAX_ROWS; ++i) anc[i] = a.anc[i];
  if constexpr (STATE) {
    const StateGeo g = geo_from_state(a.state, a.rows, tree, window, ring_slots, a.splits, a.bucket_hi);
    // workgroups above the state's split count, or any for a state outside
    // the bucket, read nothing (uniform over the workgroup, before any barrier)
    if (!g.valid || split >= g.splits) return;
    cq = g.cq, cr = g.cr, rel_lo = g.rel_lo, rel_hi = g.rel_hi, ring_base = g.ring_base, kv_base = g.base;
    append_pos0 = g.pos0;
    live_rows = g.live_rows, tree_lo = g.tree_lo, t0_rel = g.t0_rel, full_lo = g.full_lo, full_hi = g.full_hi;
#pragma unroll
    for (int i = 0; i < VA_MAX_ROWS; ++i) anc[i] = g.anc[i];
  }
  pin(cq), pin(cr), pin(rel_lo), pin(rel_hi), pin(ring_slots), pin(ring_base), pin(kv_base);
  pin(row_stride), pin(head_stride), pin(kptr), pin(vptr);
  if constexpr (FMT == 1) pin(vsc), pin(vsc_stride);
  pin(inv_group), pin(scale_log2), pin(mrows), pin(live_rows), pin(group), pin(q_heads), pin(tree);
  pin(tree_lo), pin(t0_rel), pin(window), pin(full_lo), pin(full_hi), pin(kv_heads), pin(qptr);
  pin(ws_ml), pin(ws_o);
#pragma unroll
  for (int i = 0; i < VA_MAX_ROWS; ++i) pin(anc[i]);
  const uint8_t *k_new = a.k_new, *v_new = a.v_new;
  if constexpr (APP) pin(k_new), pin(v_new);

  int32_t c_first = 0, nch = 0;
  auto chunk_range = [&]() {
    // in chunks relative to base (base is chunk aligned and the chunks cover
    // [rel_lo, rel_hi) exactly, so no clipping is needed)
    c_first = split * cq + (split < cr ? split : cr);
    nch = cq + (split < cr ? 1 : 0);
  };

  // Decoded tiles (quantised formats): buffer b holds K at dec + b*2*kDecTile
  // and V after it.  V is bf16 in the bf16 layout (piece P of a row at
  // 16*(P ^ fv0(row)), fv0 = 2*(row % 8)).  K is bf16 in the contraction
  // order of the rotated query: its 16-byte piece (k, g) holds d = 32k + 4g
  // + 0..3 and 32k + 16 + 4g + 0..3 (four codes from each of staged pieces
  // 2k and 2k + 1), at position (4k + g) ^ (row % 16), so that the 16 lanes
  // reading one operand hit 16 different positions.
  uint8_t *const dec = smem;
  auto fv0 = [](int row) { return (2 * row) & 14; };
  // Decoder d converts its share of chunk n.  Values: of the 8 * kChunk
  // units of 16 codes, the blocks of 64 consecutive units with index = d
  // (mod NDW), unit u on lane u % 64.  Keys: one unit of 32 codes per lane,
  // pieces 2k and 2k + 1 of row t / 4 (t = lane + 64 d, k = t % 4), which
  // become the four decoded pieces (k, 0..3).  All of a lane's code loads
  // are issued before it converts.
  constexpr int NUV = 8 * kChunk / 64 / (NDW > 0 ? NDW : 1);
  static_assert(FMT == 0 || (NDW == 2 && NUV * 64 * NDW == 8 * kChunk),
                "two decoders: two value units and one key unit per lane");
  auto decode = [&](int32_t n, int d) {
    if constexpr (FMT == 1) {
      const uint8_t *qs = ring + (n % NST) * kStageB;
      uint8_t *dk = dec + (n & 1) * 2 * kDecTile;
      uint8_t *dv = dk + kDecTile;
      u32x4 codes[NUV];
#pragma unroll
      for (int i = 0; i < NUV; ++i) {
        const int u = lane + 64 * (NDW * i + d);
        const int row = u >> 3, pc = u & 7;
        codes[i] = *(const u32x4 *)(qs + kTileB + row * KROW + 16 * pc);
      }
      const int t = lane + 64 * d;
      const int krow = t >> 2, kk = t & 3;
      const u32x4 ka = *(const u32x4 *)(qs + krow * KROW + 16 * ((2 * kk) ^ G::fk(krow)));
      const u32x4 kb = *(const u32x4 *)(qs + krow * KROW + 16 * ((2 * kk + 1) ^ G::fk(krow)));
#pragma unroll
      for (int i = 0; i < NUV; ++i) {
        const int u = lane + 64 * (NDW * i + d);
        const int row = u >> 3, pc = u & 7;
        // A unit's 16 codes become two 16-byte bf16 pieces, 2pc and 2pc + 1
        // of its row.  Lanes with pc >= 4 convert and store their second
        // piece first: one store instruction then puts a row's eight lanes
        // on eight different 16-byte bank groups, where storing every
        // lane's first piece together meets pc and pc ^ 4 in one group (a
        // two-way conflict on each store).  hf: the piece converted first.
        const int hf = pc >> 2;
        const u32x4 c0 = codes[i];
        const u32x4 c = hf ? (u32x4){c0[2], c0[3], c0[0], c0[1]} : c0;
        // INT8 values times the token's scale, rounded to bf16
        const float sc = ((const float *)(qs + 2 * kTileB))[row];
        u32x4 h[2];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = c[e];
          const float f0 = (float)((int32_t)(w << 24) >> 24) * sc, f1 = (float)((int32_t)(w << 16) >> 24) * sc;
          const float f2 = (float)((int32_t)(w << 8) >> 24) * sc, f3 = (float)((int32_t)w >> 24) * sc;
          h[e >> 1][2 * (e & 1)] = pack_bf16x2(f0, f1);
          h[e >> 1][2 * (e & 1) + 1] = pack_bf16x2(f2, f3);
        }
        uint8_t *dst = dv + row * kDecRow + 16 * ((2 * pc) ^ fv0(row));
        *(u32x4 *)(dst + 16 * hf) = h[0];
        *(u32x4 *)(dst + 16 * (hf ^ 1)) = h[1];
      }
      // E4M3 keys (exact in bf16): decoded piece (kk, g) is code word g of
      // staged piece 2kk, then code word g of piece 2kk + 1.  Lanes with kk
      // >= 2 take their pieces in the order g ^ 2: a store instruction's
      // eight lanes (two rows, kk = 0..3) then land on eight different
      // 16-byte bank groups of the 128-byte write window, where storing
      // piece g everywhere meets kk and kk ^ 2 in one group.
      const int sw = kk >> 1;
      const u32x4 a = sw ? (u32x4){ka[2], ka[3], ka[0], ka[1]} : ka;
      const u32x4 b = sw ? (u32x4){kb[2], kb[3], kb[0], kb[1]} : kb;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 h = {e4m3x2_to_bf16x2<false>(a[g]), e4m3x2_to_bf16x2<true>(a[g]),
                         e4m3x2_to_bf16x2<false>(b[g]), e4m3x2_to_bf16x2<true>(b[g])};
        *(u32x4 *)(dk + krow * kDecRow + 16 * ((4 * kk + (g ^ (2 * sw))) ^ (krow & 15))) = h;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tiles are whole at the next barrier
    }
  };

  if constexpr (NDW > 0) {
    if (wave >= W && wave < W + NDW) {
      // ================= decoders =================
      // Barrier n (in the loop) publishes decoded chunk n and staged chunk
      // n + 1 and frees decode buffer (n + 1) % 2 (last read in step n - 1),
      // which the decoders fill right after.
      chunk_range();
      wg_barrier();  // chunk 0 is staged
      if (nch > 0) decode(0, wave - W);
#ifdef VA_PHASE_TRACE
      uint64_t t_wait = 0, t_conv = 0;  // at the barriers after chunk 0's; converting the later chunks
#endif
      for (int32_t n = 0; n < nch; ++n) {
#ifdef VA_PHASE_TRACE
        const uint64_t tw0 = trace_now();
#endif
        wg_barrier();
#ifdef VA_PHASE_TRACE
        const uint64_t tw1 = trace_now();
        if (n > 0) t_wait += tw1 - tw0;
#endif
        if (n + 1 < nch) decode(n + 1, wave - W);
#ifdef VA_PHASE_TRACE
        t_conv += trace_now() - tw1;
#endif
      }
      VA_TRACE_VAL(va_trace_split, 16, t_wait, wave == W && lane == 0);
      VA_TRACE_VAL(va_trace_split, 17, t_conv, wave == W && lane == 0);
      return;
    }
  }

  if (wave >= W + NDW) {
    // ================= producers =================
    chunk_range();
    const uint8_t *kbase = kptr + (int64_t)kvh * head_stride;
    const uint8_t *vbase = vptr + (int64_t)kvh * head_stride;
    const uint32_t rs = (uint32_t)row_stride;
    // A chunk never straddles the ring's wrap (slots are 64-aligned), so every
    // key of chunk c0 lives at row_of(c0) + (j - c0): one scalar base per
    // chunk plus a 32-bit lane offset.  Keys outside [rel_lo, rel_hi) are
    // clamped to the extent's ends (read, then masked), so nothing outside it
    // is read.
    const uint32_t ring_div = ring_slots > 0 ? (uint32_t)ring_slots : 1u;
    auto chunk_row = [&](int32_t c0) -> int64_t {
      const int64_t ring_row = (int64_t)(((uint32_t)ring_base + (uint32_t)c0) % ring_div);
      return ring_slots ? ring_row : kv_base + c0;
    };
    auto clampx = [&](int32_t x, int32_t c0) -> int32_t {
      const int32_t lo = rel_lo - c0, hi = rel_hi - 1 - c0;
      return x < lo ? lo : (x > hi ? hi : x);
    };
    // Piece swizzles inside the staged tiles: G::fk, G::fv.
    // A chunk's DMA is 2*NDMA instructions: u < NDMA copies K rows
    // [u*RPI, u*RPI + RPI), the rest V; instruction u lands at stage + 1024*u
    // (the V tile starts NDMA KiB into the stage).  Producer wave PW issues
    // instructions [PW*U, PW*U + U) of every chunk; the producer index is a
    // template constant, so each producer's lane offsets are plain
    // arithmetic on constants.
    auto produce = [&](auto pw_const) {
      constexpr int PW = decltype(pw_const)::value;
      // Append: producer 0 owns the K tiles' DMA, producer 1 the V tiles'
      // (bf16: U = NDMA), so each takes the new rows of its tile kind, one
      // 16-byte piece per lane and pass, loaded before the first DMA issue.
      constexpr int APASS = (VA_MAX_ROWS * PIECES + 63) / 64;
      const uint8_t *knew = PW == 0 ? k_new : v_new;
      u32x4 nrow[APASS];
      if constexpr (APP) {
        const uint8_t *src = knew + (int64_t)kvh * D * 2;
#pragma unroll
        for (int i = 0; i < APASS; ++i) {
          const int rr = (64 * i + lane) / PIECES;
          if (rr < a.rows) nrow[i] = *(const u32x4 *)(src + rr * a.new_row_stride_b + 16 * (lane % PIECES));
        }
      }
      // the new live rows of chunk n into its staged tile (after its DMA
      // landed, before the barrier that publishes it)
      // relative key of row 0's own key: chain rows at t0_rel + r, tree
      // nodes at tree_lo + r
      const int32_t new0 = tree ? tree_lo : t0_rel;
      auto overlay = [&](int32_t n) {
        const int32_t c0 = (c_first + n) * kChunk;
        if (new0 >= c0 + kChunk || new0 + live_rows <= c0) return;
        uint8_t *tile = ring + (n % NST) * kStageB + (PW == 0 ? 0 : kTileB);
#pragma unroll
        for (int i = 0; i < APASS; ++i) {
          const int rr = (64 * i + lane) / PIECES;
          const int32_t x = new0 + rr;  // this row's key (relative)
          const int jx = x - c0;
          if (rr < live_rows && jx >= 0 && jx < kChunk) {
            const int f = PW == 0 ? G::fk(jx) : G::fv(jx);
            *(u32x4 *)(tile + jx * KROW + 16 * ((lane % PIECES) ^ f)) = nrow[i];
          }
        }
        if constexpr (PW == 1) {
          // Tile rows whose key is clamped into [rel_lo, rel_hi) (past rel_hi
          // - 1, or before rel_lo) were read from the slot of an edge key,
          // which this launch may be about to overwrite (stale contents, NaN
          // included).  Every row masks those keys (p = 0), and a stale K only
          // gives a score the mask replaces; a stale V would still give
          // 0 * NaN in P V.  So their V rows become zero, one 16-byte piece
          // per lane and pass.
          const int zlo = rel_lo - c0 > 0 ? rel_lo - c0 : 0;
          const int zhi = rel_hi - c0 < kChunk ? rel_hi - c0 : kChunk;
          if (zlo > 0 || zhi < kChunk) {
#pragma unroll
            for (int pz = 0; pz < kChunk * PIECES / 64; ++pz) {
              const int idx = 64 * pz + lane;
              const int j = idx / PIECES, pc = idx % PIECES;
              if (j < zlo || j >= zhi)
                *(u32x4 *)(tile + j * KROW + 16 * (pc ^ G::fv(j))) = (u32x4){0u, 0u, 0u, 0u};
            }
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      };
      uint32_t off[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int u = PW * U + i;
        const bool isv = u >= NDMA;
        const int t = isv ? u - NDMA : u;
        const int row = t * RPI + lane / PIECES;
        const int pos = lane % PIECES;
        const int f = isv ? G::fv(row) : G::fk(row);
        off[i] = (uint32_t)row * rs + 16u * (uint32_t)(pos ^ f);
      }
      // Chunk n into stage `st` (lane l of instruction u stores 16 bytes at
      // stage + 1024*u + 16*l), then (quantised values) the chunk's scales.
      auto issue = [&](int32_t n, int st) {
        const int32_t c0 = (c_first + n) * kChunk;
        const int64_t row0 = chunk_row(c0);
        const uint8_t *kc = kbase + row0 * row_stride;
        const uint8_t *vc = vbase + row0 * row_stride;
        const uint32_t stg = ring_lds + st * kStageB + 1024 * PW * U;
        if (c0 >= rel_lo && c0 + kChunk <= rel_hi) {
#pragma unroll
          for (int i = 0; i < U; ++i) dma16((PW * U + i >= NDMA ? vc : kc) + opaque(off[i]), stg + 1024 * i);
        } else {
#pragma unroll
          for (int i = 0; i < U; ++i) {
            const int u = PW * U + i;
            const int row = (u >= NDMA ? u - NDMA : u) * RPI + lane / PIECES;
            const uint32_t x = (uint32_t)clampx(row, c0) * rs;
            dma16((u >= NDMA ? vc : kc) + (x + (off[i] - (uint32_t)row * rs)), stg + 1024 * i);
          }
        }
        if constexpr (FMT == 1) {
          const float *sc = vsc + (int64_t)kvh * vsc_stride + row0;
          dma4(sc + clampx(lane & 31, c0), ring_lds + st * kStageB + 2 * kTileB);
        }
      };
#pragma unroll
      for (int j = 0; j < NST - 1; ++j)
        if (j < nch) issue(j, j);
      VA_TRACE(va_trace_split, 2, PW == 0 && lane == 0);  // first chunks' DMA issued
      if constexpr (FMT == 1) {
        // the decoders convert chunk n + 1 right after barrier n, so chunk 0
        // must have landed before an extra first barrier, and chunk n + 1
        // before barrier n
        const int32_t ahead = nch - 1;
        wait_chunks<kVmP, NST - 2>(ahead < NST - 2 ? (ahead > 0 ? ahead : 0) : NST - 2);
        wg_barrier();
      }
      int st_prev = NST - 1;  // stage of chunk n - 1
#ifdef VA_PHASE_TRACE
      uint64_t t_dma = 0, t_wait = 0;  // waiting for its DMA, at the barriers (after chunk 0's)
#endif
      for (int32_t n = 0; n < nch; ++n) {
#ifdef VA_PHASE_TRACE
        const uint64_t tw0 = trace_now();
#endif
        // chunks issued after n: n+1 .. min(n + NST - 2, nch - 1); DMA groups
        // complete in issue order, so this wait leaves exactly those in flight
        // (for the quantised formats, those after n + 1).
        const int32_t later = nch - 1 - n;
        if constexpr (FMT == 0) {
          wait_chunks<kVmP, NST - 2>(later < NST - 2 ? later : NST - 2);
          if constexpr (APP) overlay(n);
        } else {
          const int32_t after = later - 1;
          wait_chunks<kVmP, NST - 3>(after < NST - 3 ? (after > 0 ? after : 0) : NST - 3);
        }
#ifdef VA_PHASE_TRACE
        const uint64_t tw1 = trace_now();
#endif
        wg_barrier();
#ifdef VA_PHASE_TRACE
        if (n > 0) t_dma += tw1 - tw0, t_wait += trace_now() - tw1;
#endif
        if (n + NST - 1 < nch) issue(n + NST - 1, st_prev);
        st_prev = st_prev + 1 == NST ? 0 : st_prev + 1;
      }
      VA_TRACE_VAL(va_trace_split, 14, t_dma, PW == 0 && lane == 0);
      VA_TRACE_VAL(va_trace_split, 15, t_wait, PW == 0 && lane == 0);
      // split 0 stores every row (padding included) to the cache; nothing in
      // this launch reads those slots from memory: the live rows' keys were
      // put into the tiles above, and the padding rows' slots lie outside
      // every row's keys
      if (APP && split == 0 && (RG == 1 || blockIdx.z == 0)) {
        uint8_t *dst = (PW == 0 ? const_cast<uint8_t *>(kptr) : const_cast<uint8_t *>(vptr)) +
                       (int64_t)kvh * head_stride + 16 * (lane % PIECES);
#pragma unroll
        for (int i = 0; i < APASS; ++i) {
          const int rr = (64 * i + lane) / PIECES;
          // from the absolute position (64-bit: a state without live rows
          // may sit anywhere in [0, 2^61], where the relative coordinates
          // do not reach); positions are never negative
          const int64_t p = append_pos0 + rr;
          const int64_t slot = ring_slots ? (int64_t)((uint64_t)p % (uint64_t)ring_slots) : p;
          if (rr < a.rows && (ring_slots || slot < a.kv_capacity)) *(u32x4 *)(dst + slot * row_stride) = nrow[i];
        }
      }
    };
    static_assert(NPW == 1 || NPW == 2, "one or two producers");
    if constexpr (NPW == 1) {
      produce(std::integral_constant<int, 0>{});
    } else {
      if (wave == W + NDW) produce(std::integral_constant<int, 0>{});
      else produce(std::integral_constant<int, 1>{});
    }
    return;
  }

  // ================= consumers =================
  chunk_range();
  VA_TRACE_VAL(va_trace_split, 0, t_entry, wave == 0 && lane == 0);  // kernel entry
  VA_TRACE(va_trace_split, 1, wave == 0 && lane == 0);   // arguments in registers

  // lane column i16 of this wave is query matrix row m = 16*(wave + z*W) +
  // i16 = r*G + (h - kvh*G), z = blockIdx.z < RG the workgroup's row group;
  // live matrix rows are [0, live_rows * G).
  const int mb = 16 * (wave + (RG > 1 ? (int)blockIdx.z * W : 0));  // first matrix row of this wave
  const int m = mb + i16;
  const int r = (int)(((float)m + 0.5f) * inv_group);  // m / G: exact for every m < 96, G <= 96
  const bool row_ok = (m < mrows) && (r < live_rows);
  const bool active = mb < live_rows * group;  // wave-uniform
  const int rr = row_ok ? r : 0;
  const int h = kvh * group + (row_ok ? m - r * group : 0);
  const uint8_t *qrow = qptr + (int64_t)(rr * q_heads + h) * D * 2;

  // ---------------- Q^T operands (B operand of S^T = K Q^T) ----------------
  // lane (i16, g4) holds row m, contraction piece 4*ks + g4 of step ks.
  bf16x8 qop[KS];
  if constexpr (FMT == 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = *(const u32x4 *)(qrow + (32 * ks + 8 * g4) * 2);
      if (!row_ok) w = (u32x4){0u, 0u, 0u, 0u};
      qop[ks] = __builtin_bit_cast(bf16x8, w);
    }
  } else {
    // q' = H q / sqrt(128) (natural-order Walsh-Hadamard, H[i][j] =
    // (-1)^popcount(i & j)), summed in FP32 on the MFMA, then bf16.  Output
    // block nb (d = 16nb .. 16nb + 15) is the sum over the four 32-d steps
    // ks of H[16nb + m][32ks + k] times q[row][32ks + k]: the A operand (m
    // = i16, k = 8g4 + e) is that block of H, the B operand the raw query
    // as loaded (lane (i16, g4) holds row i16, d = 32ks + 8g4 + e).  With
    // the bits of both indices, popcount((16nb + m) & (32ks + 8g4 + e)) =
    // popcount(m & e & 7) + (m bit 3 & g4 bit 0) + (nb bit 0 & g4 bit 1) +
    // popcount((nb >> 1) & ks): the first two terms are this lane's, the
    // third picks one of two operands, and the last, uniform per product,
    // negates the query instead.  Every product is exact (+-1 times a bf16
    // value); the sums round in FP32.
    bf16x8 qb[KS], qn[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = *(const u32x4 *)(qrow + (32 * ks + 8 * g4) * 2);
      if (!row_ok) w = (u32x4){0u, 0u, 0u, 0u};
      qb[ks] = __builtin_bit_cast(bf16x8, w);
      qn[ks] = __builtin_bit_cast(bf16x8, w ^ 0x80008000u);
    }
    bf16x8 ha[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      u32x4 w;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        uint32_t h2 = 0u;
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
          const int e = 2 * e2 + hi;
          const uint32_t neg = (__builtin_popcount(i16 & e & 7) + ((i16 >> 3) & g4 & 1) + par * ((g4 >> 1) & 1)) & 1;
          h2 |= (0x3f80u | (neg << 15)) << (16 * hi);  // bf16 +1 or -1
        }
        w[e2] = h2;
      }
      ha[par] = __builtin_bit_cast(bf16x8, w);
    }
    f32x4 qr[8];  // lane (i16, g4): q'[row i16][16nb + 4g4 + i], i = 0..3
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = mfma16(ha[nb & 1], (__builtin_popcount((nb >> 1) & ks) & 1) ? qn[ks] : qb[ks], acc);
      qr[nb] = acc;
    }
    // 1/sqrt(128) and the softmax scale (log2 units) in one factor: the
    // rotated q is rounded to bf16 either way, and the scores then come
    // out of the MFMA already scaled.  Step ks contracts d = 32ks + 4g4 +
    // 0..3 (block 2ks) and 32ks + 16 + 4g4 + 0..3 (block 2ks + 1), the
    // order of the decoded key pieces.
    const float inv = 0.08838834764831845f * scale_log2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f32x4 a = qr[2 * ks] * inv, b = qr[2 * ks + 1] * inv;
      const u32x4 w = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                       pack_bf16x2(b[2], b[3])};
      qop[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---------------- row geometry for boundary masks ----------------
  // Chain modes: row r sits at t0_rel + r and sees [max(t0_rel + r - window
  // + 1, 0), t0_rel + r] (window 0: from 0).  Tree mode: [0, tree_lo) plus
  // the node keys whose bits are set in anc[r].
  int32_t rlo, rhi;
  uint32_t ranc = 0u;
  {
    int32_t lo_r, hi_r;
    if (tree) {
      lo_r = 0;
      hi_r = tree_lo;
#pragma unroll
      for (int i = 0; i < VA_MAX_ROWS; ++i) ranc = (r == i) ? anc[i] : ranc;
    } else {
      const int32_t t = t0_rel + r;
      hi_r = t + 1;
      lo_r = window ? t - window + 1 : 0;
      if (lo_r < 0) lo_r = 0;
    }
    rlo = row_ok ? lo_r : 0;
    rhi = row_ok ? hi_r : 0;
    ranc = row_ok ? ranc : 0u;
  }

  // ---------------- online-softmax state ----------------
  f32x4 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // mref: the row's reference maximum (log2 units, uniform over the row's
  // four lane groups); mlane: this lane's running maximum of its raw
  // scores; lrow: this lane's share of the row's sum of weights.
  float mref = -INFINITY, mlane = -INFINITY, lrow = 0.f;
  // scores times cs are in log2 units (quantised caches carry the scale in q)
  const float cs = FMT == 1 ? 1.f : scale_log2;

  // Swizzles of the staged tiles (must match the producer's).
  auto fk = [](int row) { return G::fk(row); };
  auto fv = [](int row) { return G::fv(row); };

  // Quantised formats: each lane's byte offsets of its decoded K and V
  // operands within a buffer, computed once; the buffer's own offset is a
  // constant of each unrolled step, so a read needs no address arithmetic.
  // (The empty asm keeps each sum in a register instead of letting the
  // compiler re-add its two parts at every read.)
  uint32_t dko[KS], dvo[MD];
  if constexpr (FMT == 1) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      dko[ks] = (uint32_t)(i16 * kDecRow + 16 * ((4 * ks + g4) ^ i16));
      asm volatile("" : "+v"(dko[ks]));
    }
    const int rowA = 4 * g4 + (i16 >> 2);
    const int F = fv0(rowA) >> 1;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      dvo[md] = (uint32_t)(rowA * kDecRow + 8 * (i16 & 3) + 32 * (md ^ F));
      asm volatile("" : "+v"(dvo[md]));
    }
  }

  // kt: the chunk's staged tiles; db: its decoded-tile buffer (quantised formats)
  auto step = [&](int32_t n, const uint8_t *kt, int db) {
    const uint8_t *vt = kt + kTileB;
    const int32_t c0 = (c_first + n) * kChunk;
    const uint8_t *dk = dec + db * 2 * kDecTile;  // decoded tiles (quantised formats)
    const uint8_t *dv = dk + kDecTile;

    // ---- K operands: A operand of block mb is keys 16*mb + i16 ----
    bf16x8 kop[2][KS];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int row = 16 * mb + i16;
      if constexpr (FMT == 0) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kop[mb][ks] = *(const bf16x8 *)(kt + row * KROW + 16 * ((4 * ks + g4) ^ fk(row)));
      } else {
        // decoded piece (ks, g4); rows 16 + i16 repeat row i16's swizzle 16
        // rows lower
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kop[mb][ks] = *(const bf16x8 *)(dk + 16 * mb * kDecRow + dko[ks]);
      }
    }
    // ---- V^T operands: lane (i16 = d within block md, g4) takes the keys
    //      {4g..4g+3, 16+4g..16+4g+3} of column d ----
    bf16x8 vop[MD];
    if constexpr (FMT == 0) {
      // Two transpose reads per block: lane s of group g4 addresses row
      // 4*g4 + s/4 (then +16), columns 16*md + 4*(s%4) .. +3, so output lane
      // i16 receives V[4*g4 + e][16*md + i16], e = 0..3.
      const int rowA = 4 * g4 + (i16 >> 2);
      const int F = fv(rowA) >> 1;  // same for rowA + 16
      const uint8_t *vb = vt + rowA * KROW + 8 * (i16 & 3);
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const uint8_t *pa = vb + 32 * (md ^ F);
        const u32x2 lo = lds_read_tr16(pa);
        const u32x2 hi = lds_read_tr16(pa + 16 * KROW);
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        vop[md] = __builtin_bit_cast(bf16x8, w);
      }
    } else {
      // the decoded bf16 tile, read as for bf16 caches
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const uint8_t *pa = dv + dvo[md];
        const u32x2 lo = lds_read_tr16(pa);
        const u32x2 hi = lds_read_tr16(pa + 16 * kDecRow);
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        vop[md] = __builtin_bit_cast(bf16x8, w);
      }
    }

    // ---- S^T = K Q^T ----
    f32x4 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16(kop[mb][ks], qop[ks], acc);
      s[mb] = acc;
    }

    // ---- boundary mask, this lane's maximum ----
    float x[8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * mb + e] = s[mb][e];
    if (!(c0 >= full_lo && c0 + kChunk <= full_hi)) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        // branch-free: row interval, or (tree) an ancestor-or-self node key
        const int32_t j = c0 + (t < 4 ? 4 * g4 + t : 16 + 4 * g4 + (t - 4));
        const uint32_t in_row = (uint32_t)(j - rlo) < (uint32_t)(rhi - rlo);
        const uint32_t ti = (uint32_t)(j - tree_lo);
        const uint32_t in_tree = (uint32_t)(ti < 16u) & (ranc >> (ti & 15u));
        x[t] = ((in_row | in_tree) & 1u) ? x[t] : -INFINITY;
      }
    }
    float lm = x[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) lm = fmaxf(lm, x[t]);
    mlane = fmaxf(mlane, lm);

    // ---- lazy reference maximum ----
    // Exponents are taken against mref, which moves only when a row's chunk
    // maximum exceeds it by more than kTau (so every p stays <= 2^kTau);
    // moving it rescales that row's O and l (a rare, wave-uniform branch).
    // The row maximum (across the row's lane groups) is formed only when
    // some lane's own maximum could move its row's reference, or a row has
    // none yet; otherwise no row's maximum exceeds mref + kTau either.
    // Rounding is monotone, so max(x) * cs is the maximum of the scaled x.
    if (__builtin_amdgcn_ballot_w64(mref == -INFINITY || lm * cs > mref + kTau) != 0) {
      const float mx = wave_max16x4(lm) * cs;
      const bool need = (mref != -INFINITY) && (mx > mref + kTau);
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float nref = need ? mx : mref;
        const float alpha = (mref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mref - nref);
        lrow *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md) o[md] *= alpha;
        mref = nref;
      }
      mref = (mref == -INFINITY) ? mx : mref;
    }

    // ---- P^T (B operand of PV) and l ----
    // One rounding per exponent: the product with the scale and the
    // subtraction in one FMA (quantised caches: cs = 1, so a row's largest
    // key gets p = 1 exactly).  The lane's eight weights are summed as a
    // tree (three dependent adds instead of eight).
    const float m_use = (mref == -INFINITY) ? 0.f : mref;
    float p[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) p[t] = __builtin_amdgcn_exp2f(fmaf(x[t], cs, -m_use));
    lrow += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    u32x4 pw;
#pragma unroll
    for (int e = 0; e < 4; ++e) pw[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int md = 0; md < MD; ++md) o[md] = mfma16(vop[md], pb, o[md]);
  };

  if constexpr (FMT == 1) wg_barrier();  // chunk 0 is staged (the decoders convert it)
  // Chunk n sits in stage n % NST (and decoded buffer n % 2): the loop is
  // unrolled over the stages, so each copy reads LDS at constant offsets
  // from lane bases computed once (no address arithmetic per chunk).
  static_assert(NST % 2 == 0, "decoded buffers alternate with the chunk index");
#ifdef VA_PHASE_TRACE
  uint64_t t_bar = 0;  // this wave's time at the barriers after its first chunk arrived
#endif
  for (int32_t n0 = 0; n0 < nch; n0 += NST) {
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      if (n0 + j < nch) {
#ifdef VA_PHASE_TRACE
        const uint64_t tb0 = trace_now();
#endif
        wg_barrier();  // chunk n0 + j is in LDS (decoded); every consumer has left the one before
#ifdef VA_PHASE_TRACE
        const uint64_t tb1 = trace_now();
        if (n0 + j == 0) VA_TRACE_VAL(va_trace_split, 3, tb1, wave == 0 && lane == 0);  // first chunk in LDS
        else t_bar += tb1 - tb0;
#endif
        if (active) step(n0 + j, ring + j * kStageB, j & 1);
      }
    }
  }
  VA_TRACE(va_trace_split, 4, wave == 0 && lane == 0);  // last step issued
  VA_TRACE_VAL(va_trace_split, 6, t_bar, wave == 0 && lane == 0);
  VA_TRACE_VAL(va_trace_split, 8 + wave, t_bar, lane == 0);
  VA_TRACE_VAL(va_trace_split, 7, (uint64_t)nch, wave == 0 && lane == 0);

  // ---------------- partials of this wave's live rows ----------------
  // Normalised to the true maximum M of the split: m = M, l = sum 2^(x - M),
  // O = sum 2^(x - M) v.  Padding rows store nothing: the combine never
  // reads them.
  if (!active) return;
  const float lt = wave_sum16x4(lrow);
  const float mtrue = wave_max16x4(mlane) * cs;
  const float f = (mref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mref - mtrue);
  if (row_ok) {
    const int64_t unit = ((int64_t)split * kv_heads + kvh) * mrows + m;
    if (g4 == 0) *(f32x2 *)(ws_ml + unit * 2) = (f32x2){mtrue, lt * f};
    float *op = ws_o + unit * D;
#pragma unroll
    for (int md = 0; md < MD; ++md) *(f32x4 *)(op + 16 * md + 4 * g4) = o[md] * f;
  }
#ifdef VA_PHASE_TRACE
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  VA_TRACE(va_trace_split, 5, wave == 0 && lane == 0);  // this wave's partials written
#endif
}

// ---------------------------------------------------------------------------
// Combine kernel: grid (G, Hkv, rows * D/32), WAVES wave64s; a workgroup
// merges 32 consecutive d of one (row, query head).  Thread t owns four of them
// (dq = t % 8) and the splits s = sg, sg + NSG, sg + 2*NSG, ... (sg = t / 8,
// NSG = 8 * WAVES split groups), which it folds into four FP32 chains (one
// per d) against a running maximum that moves only when a batch brings a
// larger m.  All loads of a batch (BATCH splits: their (m, l) and O) are
// issued together.  The chains of each d are then merged by lane exchanges
// inside each wave and, with four waves, once through LDS; then the sink.
// ---------------------------------------------------------------------------
constexpr int kMaxSplits = 4096;
constexpr int kCombD = 32;           // d per workgroup
constexpr int kCombDQ = kCombD / 4;  // threads per split group (four d each)
constexpr int kCombMaxBatch = 16;

// Lane l ^ 8 by DPP row_ror:8 (a rotation by 8 inside each 16-lane row).
__device__ __forceinline__ float lane_xor8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
}
// Reductions over the eight lanes l ^ {0, 8, 16, 24, 32, ...} that share
// l % 8, all on the VALU.
__device__ __forceinline__ float xor_max3(float x) {
  x = fmaxf(x, lane_xor8(x));
  return wave_max16x4(x);
}
__device__ __forceinline__ float xor_sum3(float x) {
  x += lane_xor8(x);
  return wave_sum16x4(x);
}

template <int BATCH, int WAVES, bool STATE>
__global__ __launch_bounds__(64 * WAVES) void combine_kernel(const CombineArgs a) {
#ifdef VA_PHASE_TRACE
  const uint64_t t_entry = trace_now();
#endif
  constexpr int kCombNSG = 8 * WAVES;  // split groups
  __shared__ f32x4 wacc[WAVES][kCombDQ];
  __shared__ float wm[WAVES], wden[WAVES];

  // every kernel argument loaded in one round trip (see pin())
  const float *ws_ml = a.ws_ml, *ws_o = a.ws_o, *sinkp = a.sink;
  float *outb = a.out, *lsep = a.lse;
  int32_t live_rows = a.live_rows, S = a.splits;
  const int32_t group = a.group, mrows = a.mrows, q_heads = a.q_heads;
  const int32_t kv_heads = a.kv_heads, D = a.head_dim;
  pin(ws_ml), pin(ws_o), pin(sinkp), pin(outb), pin(lsep), pin(live_rows), pin(group), pin(mrows);
  pin(q_heads), pin(kv_heads), pin(S), pin(D);
  if constexpr (STATE) {
    const StateGeo g = geo_from_state(a.state, a.rows, a.tree, a.window, a.ring_slots, a.splits, a.bucket_hi);
    if (!g.valid) {  // a state outside the bucket: every output is NaN
      const int t = threadIdx.x;
      if (t < kCombDQ) {
        const int sh = D == 128 ? 2 : 1;  // log2 of the 32-wide d slices
        const int rh = (blockIdx.z >> sh) * q_heads + blockIdx.y * group + blockIdx.x;
        const int ds = blockIdx.z & ((1 << sh) - 1);
        *(f32x4 *)(outb + (int64_t)rh * D + kCombD * ds + 4 * t) = (f32x4){NAN, NAN, NAN, NAN};
        if (lsep && ds == 0 && t == 0) lsep[rh] = NAN;
      }
      return;
    }
    live_rows = g.live_rows;
    S = g.splits;
  }

  // grid (G, Hkv, rows * D/32): query head h = g*G + j of KV head g, row r,
  // d slice ds (D/32 is 2 or 4, so no division on the way to the loads)
  const int sh = D == 128 ? 2 : 1;
  const int j = blockIdx.x, g = blockIdx.y;
  const int r = blockIdx.z >> sh, ds = blockIdx.z & ((1 << sh) - 1);
  const int h = g * group + j;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int dq = t % kCombDQ, sg = t / kCombDQ;
  const int d0 = kCombD * ds + 4 * dq;
  float *outp = outb + ((int64_t)r * q_heads + h) * D;

  if (r >= live_rows) {  // padding row: no read of the workspace
    if (sg == 0) *(f32x4 *)(outp + d0) = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (lsep && ds == 0 && t == 0) lsep[(int64_t)r * q_heads + h] = -INFINITY;
    return;
  }
  VA_TRACE_VAL(va_trace_comb, 0, t_entry, t == 0);
  VA_TRACE(va_trace_comb, 1, t == 0);  // arguments in registers (pin() waited for them)
  const int mrow = r * group + j;
  const int64_t stride_unit = (int64_t)kv_heads * mrows;  // units between splits
  const int64_t unit0 = (int64_t)g * mrows + mrow;
  // split s of this (row, head): (m, l) at mlb + s*ml_step, O at ob + s*o_step
  const uint8_t *mlb = (const uint8_t *)(ws_ml + unit0 * 2);
  const uint8_t *ob = (const uint8_t *)(ws_o + unit0 * D + d0);
  const uint64_t ml_step = (uint64_t)stride_unit * 2 * 4;
  const uint64_t o_step = (uint64_t)stride_unit * D * 4;

  float M = -INFINITY, den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // the sink logit (used by wave 0's merge lanes, whose split group is 0 and
  // so always runs the first batch) is loaded right after that batch's
  // partials and used only at the end: no round trip of its own
  float sink_raw = -INFINITY;
  for (int s0 = sg; s0 < S; s0 += kCombNSG * BATCH) {
    f32x2 mlv[BATCH];
    f32x4 ov[BATCH];
    // Loads are unconditional, so they issue back to back: a split past S
    // re-reads split S-1 and gets m + (-inf) = -inf, hence weight 0 (its
    // finite l and O then add nothing).
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int s = s0 + kCombNSG * j;
      const uint32_t se = (uint32_t)(s < S - 1 ? s : S - 1);
      mlv[j] = *(const f32x2 *)(mlb + se * ml_step);
      ov[j] = *(const f32x4 *)(ob + se * o_step);
      mlv[j][0] += s < S ? 0.f : -INFINITY;
    }
    if (s0 == sg && sinkp && t < kCombDQ) sink_raw = sinkp[h];
    asm volatile("" ::: "memory");  // keeps every load of the batch above the first use
    float bm = M;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) bm = fmaxf(bm, mlv[j][0]);
#ifdef VA_PHASE_TRACE
    if (s0 == sg) {
      asm volatile("" ::"v"(bm), "v"(ov[BATCH - 1][3]));  // the batch has arrived
      VA_TRACE(va_trace_comb, 2, t == 0);                // first batch in registers
    }
#endif
    if (bm > M) {
      const float alpha = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - bm);
      den *= alpha;
      acc *= alpha;
      M = bm;
    }
    const float Mu = (M == -INFINITY) ? 0.f : M;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const float w = __builtin_amdgcn_exp2f(mlv[j][0] - Mu);  // 0 for m = -inf
      den = fmaf(w, mlv[j][1], den);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = fmaf(w, ov[j][c], acc[c]);
    }
  }

  VA_TRACE(va_trace_comb, 3, t == 0);  // every batch folded
  // merge the eight split groups of this wave (lanes dq, dq + 8, ..., dq + 56)
  const float Mw = xor_max3(M);
  const float f = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mw);
  den = xor_sum3(den * f);
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = xor_sum3(acc[c] * f);
  if constexpr (WAVES > 1) {
    if (lane < kCombDQ) {
      wacc[wave][lane] = acc;
      if (lane == 0) {
        wm[wave] = Mw;
        wden[wave] = den;
      }
    }
    __syncthreads();
  }

  if (t < kCombDQ) {  // wave 0, one lane per dq: merge the waves and the sink
    const float sink2 = sinkp ? sink_raw * LOG2E_F : -INFINITY;
    float Mt = sink2;
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float dt = 0.f;
    if constexpr (WAVES > 1) {
#pragma unroll
      for (int i = 0; i < WAVES; ++i) Mt = fmaxf(Mt, wm[i]);
    } else {
      Mt = fmaxf(Mt, Mw);
    }
    const float Mu = (Mt == -INFINITY) ? 0.f : Mt;
#pragma unroll
    for (int i = 0; i < WAVES; ++i) {
      const float wmi = WAVES > 1 ? wm[i] : Mw;
      const float fi = (wmi == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(wmi - Mu);
      dt = fmaf(fi, WAVES > 1 ? wden[i] : den, dt);
      const f32x4 c = WAVES > 1 ? wacc[i][dq] : acc;
#pragma unroll
      for (int k = 0; k < 4; ++k) tot[k] = fmaf(fi, c[k], tot[k]);
    }
    dt += __builtin_amdgcn_exp2f(sink2 - Mu);  // 0 without a sink
    const bool lse_lane = lsep && ds == 0 && dq == 0;
    if (Mt == -INFINITY) {  // nothing visible and no sink
      *(f32x4 *)(outp + d0) = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (lse_lane) lsep[(int64_t)r * q_heads + h] = -INFINITY;
    } else {
      *(f32x4 *)(outp + d0) = tot / dt;
      if (lse_lane) lsep[(int64_t)r * q_heads + h] = (Mu + __log2f(dt)) * LN2_F;
    }
#ifdef VA_PHASE_TRACE
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    VA_TRACE(va_trace_comb, 4, t == 0);  // output written
#endif
  }
}

// One wave per workgroup while it covers the splits in one batch of at most
// kComb1WaveBatch (no LDS merge, no barrier); else four waves.  The batch is
// the smallest power of two that covers S in one round (fewer instructions
// for short reads); larger S loop over rounds of kCombMaxBatch.
constexpr int kComb1WaveBatch = 8;

template <int WAVES, bool STATE>
hipError_t launch_combine_w(const CombineArgs &a, dim3 grid, int per, hipStream_t stream) {
  const dim3 block(64 * WAVES);
  if (per <= 1) {
    hipLaunchKernelGGL((combine_kernel<1, WAVES, STATE>), grid, block, 0, stream, a);
  } else if (per <= 2) {
    hipLaunchKernelGGL((combine_kernel<2, WAVES, STATE>), grid, block, 0, stream, a);
  } else if (per <= 4) {
    hipLaunchKernelGGL((combine_kernel<4, WAVES, STATE>), grid, block, 0, stream, a);
  } else if (per <= 8) {
    hipLaunchKernelGGL((combine_kernel<8, WAVES, STATE>), grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((combine_kernel<kCombMaxBatch, WAVES, STATE>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

// S is the plan's split count: with a per-call state the kernel runs with at
// most that many, so the configuration covers every state of the bucket.
template <bool STATE>
hipError_t launch_combine(const CombineArgs &a, dim3 grid, int S, hipStream_t stream) {
  const int per1 = (S + 7) / 8;  // splits per thread with one wave (8 split groups)
  if (per1 <= kComb1WaveBatch) return launch_combine_w<1, STATE>(a, grid, per1, stream);
  return launch_combine_w<4, STATE>(a, grid, (S + 31) / 32, stream);
}

// ---------------------------------------------------------------------------
// Ring write: one thread per 16-byte piece of K and of V.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void ring_write_kernel(const uint8_t *k_new, const uint8_t *v_new, int rows,
                                                         int kv_heads, int head_dim, uint8_t *k_ring,
                                                         uint8_t *v_ring, int ring_slots, int slot0,
                                                         int64_t head_stride_b, int64_t row_stride_b) {
  const int pieces = head_dim / 8;
  const int total = rows * kv_heads * pieces;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int pc = idx % pieces;
  const int g = (idx / pieces) % kv_heads;
  const int r = idx / (pieces * kv_heads);
  const int slot = (int)(((uint32_t)slot0 + (uint32_t)r) % (uint32_t)ring_slots);
  const int64_t src = ((int64_t)(r * kv_heads + g) * head_dim + pc * 8) * 2;
  const int64_t dst = (int64_t)g * head_stride_b + (int64_t)slot * row_stride_b + pc * 16;
  *(u32x4 *)(k_ring + dst) = *(const u32x4 *)(k_new + src);
  *(u32x4 *)(v_ring + dst) = *(const u32x4 *)(v_new + src);
}

// ---------------------------------------------------------------------------
// KV write with the cache's codec: one wave per (row, KV head).
// ---------------------------------------------------------------------------
// E4M3FN code of y: nearest finite value, ties to the even code, saturating
// at 448, sign copied from y; NaN gives 0x7F.  Integer-exact: the mantissa is
// rounded as rint(|y| * 2^(3 - e)) in [8, 16] for |y| >= 2^-6 (e = floor(log2
// |y|); a carry to 16 moves to the next binade), and as rint(|y| * 2^9) for
// the subnormal step 2^-9 below; both scalings are exact powers of two.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  if (y != y) return 0x7Fu;
  const uint32_t sign = (__float_as_uint(y) >> 31) << 7;
  const float a = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);  // 0..8; 8 is the smallest normal 2^-6
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // a is a normal FP32 here
    uint32_t r = (uint32_t)rintf(a * __uint_as_float((uint32_t)(127 + 3 - e) << 23));
    if (r == 16u) {
      r = 8u;
      e += 1;
    }
    code = ((uint32_t)(e + 7) << 3) | (r - 8u);
  }
  return sign | code;
}

template <int FMT>
__global__ __launch_bounds__(64) void kv_write_kernel(const uint16_t *k_new, const uint16_t *v_new, int kv_heads,
                                                      int head_dim, uint8_t *k_cache, uint8_t *v_cache, float *v_scale,
                                                      int64_t v_scale_head_stride, int64_t first_pos, int ring_slots,
                                                      int64_t head_stride_b, int64_t row_stride_b) {
  const int r = blockIdx.x / kv_heads, g = blockIdx.x % kv_heads;
  const int lane = threadIdx.x;
  const int64_t pos = first_pos + r;
  const int64_t slot = ring_slots ? pos % ring_slots : pos;
  const int64_t src = ((int64_t)r * kv_heads + g) * head_dim;  // elements
  const int64_t dst = (int64_t)g * head_stride_b + slot * row_stride_b;  // bytes
  if constexpr (FMT == 0) {
    const int pieces = head_dim / 8;  // 16-byte pieces per row
    if (lane < pieces) {
      *(u32x4 *)(k_cache + dst + 16 * lane) = *(const u32x4 *)(k_new + src + 8 * lane);
      *(u32x4 *)(v_cache + dst + 16 * lane) = *(const u32x4 *)(v_new + src + 8 * lane);
    }
  } else {
    // head_dim 128: lane l holds elements 2l and 2l + 1.
    const uint32_t kw = *(const uint32_t *)(k_new + src + 2 * lane);
    const uint32_t vw = *(const uint32_t *)(v_new + src + 2 * lane);
    float x0 = __uint_as_float(kw << 16), x1 = __uint_as_float(kw & 0xffff0000u);
    // width 1 inside the lane, then widths 2..64 pair lane l with l ^ (width/2)
    float y0 = x0 + x1, y1 = x0 - x1;
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
      const float p0 = __shfl_xor(y0, h, 64), p1 = __shfl_xor(y1, h, 64);
      const bool upper = (lane & h) != 0;
      y0 = upper ? p0 - y0 : y0 + p0;
      y1 = upper ? p1 - y1 : y1 + p1;
    }
    const float inv = 0.08838834764831845f;  // 1/sqrt(128)
    const uint32_t kc = e4m3_code(y0 * inv) | (e4m3_code(y1 * inv) << 8);
    *(uint16_t *)(k_cache + dst + 2 * lane) = (uint16_t)kc;

    const float v0 = __uint_as_float(vw << 16), v1 = __uint_as_float(vw & 0xffff0000u);
    // maximum of |v| with NaN kept (fmaxf would drop it): a row holding NaN
    // or an infinity gets a non-finite scale and zero codes
    auto nmax = [](float a, float b) { return (a > b || a != a) ? a : b; };
    float amax = nmax(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) amax = nmax(amax, __shfl_xor(amax, h, 64));
    const float sc = amax / 127.f;  // IEEE division, correctly rounded
    int c0 = 0, c1 = 0;
    if (sc != 0.f && __builtin_isfinite(sc)) {
      c0 = (int)rint((double)v0 / (double)sc);
      c1 = (int)rint((double)v1 / (double)sc);
      c0 = c0 < -127 ? -127 : (c0 > 127 ? 127 : c0);
      c1 = c1 < -127 ? -127 : (c1 > 127 ? 127 : c1);
    }
    *(uint16_t *)(v_cache + dst + 2 * lane) = (uint16_t)((uint32_t)(c0 & 0xff) | ((uint32_t)(c1 & 0xff) << 8));
    if (lane == 0) v_scale[(int64_t)g * v_scale_head_stride + slot] = sc;
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
const va_plan_data *plan_of(const va_plan *plan) {
  if (!plan) return nullptr;
  const va_plan_data *d = reinterpret_cast<const va_plan_data *>(plan);
  return d->magic == VA_PLAN_MAGIC ? d : nullptr;
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Producer waves and LDS stages per format.  Measured on the full-attention
// sweep: one or two producers and three to five bf16 stages stream alike
// (the kernel runs at the chip's streaming rate once the ring has two or
// more chunks in flight); two producers halve each one's issue work.
template <int FMT>
constexpr int producers_for() { return FMT == 1 ? 1 : 2; }
template <int D, int FMT>
constexpr int stages_for() { return FMT == 1 ? 8 : (D == 64 ? 8 : 4); }

template <int D, int W, int FMT, bool STATE, bool APP, int RG = 1>
hipError_t launch_split(const SplitArgs &a, hipStream_t stream) {
  constexpr int NPW = producers_for<FMT>();
  constexpr int NST = stages_for<D, FMT>();
  dim3 grid(a.splits, a.kv_heads, RG);
  constexpr int NDW = decoders_for<FMT>();
  hipLaunchKernelGGL((split_kernel<D, W, FMT, NST, NPW, STATE, APP, RG>), grid, dim3(64 * (W + NDW + NPW)), 0, stream,
                     a);
  return hipGetLastError();
}

// nb_total: 16-row blocks per workgroup (the consumer waves W); rg: row
// groups, the workgroups per (split, KV head).  The plan makes two groups
// only from five blocks up (at most six), so a group then has three.
template <int D, int FMT, bool STATE, bool APP = false>
hipError_t dispatch_rows(const SplitArgs &a, int nb_total, int rg, hipStream_t stream) {
  if (rg == 2) return nb_total == 3 ? launch_split<D, 3, FMT, STATE, APP, 2>(a, stream) : hipErrorInvalidValue;
  if (rg != 1) return hipErrorInvalidValue;
  switch (nb_total) {
    case 1: return launch_split<D, 1, FMT, STATE, APP>(a, stream);
    case 2: return launch_split<D, 2, FMT, STATE, APP>(a, stream);
    case 3: return launch_split<D, 3, FMT, STATE, APP>(a, stream);
    case 4: return launch_split<D, 4, FMT, STATE, APP>(a, stream);
    case 5: return launch_split<D, 5, FMT, STATE, APP>(a, stream);
    case 6: return launch_split<D, 6, FMT, STATE, APP>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <bool STATE>
hipError_t dispatch_split(const SplitArgs &a, int nb_total, int rg, bool quant, int head_dim, hipStream_t stream) {
  if (quant) return dispatch_rows<128, 1, STATE>(a, nb_total, rg, stream);
  if (head_dim == 64) return dispatch_rows<64, 0, STATE>(a, nb_total, rg, stream);
  return dispatch_rows<128, 0, STATE>(a, nb_total, rg, stream);
}

va_status split_impl(const va_plan *plan, const va_state *state, const void *q, const void *k, const void *v,
                     const float *v_scale, int64_t v_scale_head_stride, int64_t kv_head_stride,
                     int64_t kv_row_stride, void *workspace, size_t workspace_bytes, hipStream_t stream,
                     const void *k_new = nullptr, const void *v_new = nullptr) {
  const va_plan_data *d = plan_of(plan);
  if (!d) return VA_ERR_INVALID;
  if (!workspace || workspace_bytes < d->workspace_bytes) return VA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return VA_ERR_INVALID;
  if (d->splits > kMaxSplits) return VA_ERR_UNSUPPORTED;
  const bool quant = d->kv_fmt == VA_KV_K_E4M3_WHT_V_I8;
  const int64_t esz = quant ? 1 : 2;
  // a per-call state may read anywhere in the bucket, and an append writes,
  // so their pointers are checked even when the plan's own extent is empty
  if (state || k_new || d->hi > d->lo) {
    if (!q || !k || !v) return VA_ERR_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return VA_ERR_INVALID;
    if (kv_head_stride < 0 || kv_row_stride < d->head_dim) return VA_ERR_INVALID;
    if (((kv_head_stride * esz) & 15) || ((kv_row_stride * esz) & 15)) return VA_ERR_INVALID;
    // a lane's offset inside a 32-key chunk is a 32-bit row * stride product
    if (kv_row_stride * esz > ((int64_t)1 << 26)) return VA_ERR_INVALID;
    if (quant && (!v_scale || v_scale_head_stride < 0)) return VA_ERR_INVALID;
  }
  SplitArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint8_t *)q;
  a.k = (const uint8_t *)k;
  a.v = (const uint8_t *)v;
  a.v_scale = v_scale;
  a.ws_ml = (float *)workspace;
  a.ws_o = (float *)((uint8_t *)workspace + d->ml_bytes);
  a.kv_head_stride_b = kv_head_stride * esz;
  a.kv_row_stride_b = kv_row_stride * esz;
  a.v_scale_head_stride = v_scale_head_stride;
  a.base = d->chunk_lo * VA_SPLIT_KEYS;
  a.rows = d->rows;
  a.live_rows = d->live_rows;
  a.group = d->group;
  a.inv_group = 1.0f / (float)d->group;
  a.mrows = d->matrix_rows;
  a.q_heads = d->q_heads;
  a.kv_heads = d->kv_heads;
  a.splits = d->splits;
  a.chunks_q = (int32_t)(d->chunks / d->splits);
  a.chunks_r = (int32_t)(d->chunks % d->splits);
  a.rel_lo = (int32_t)(d->lo - a.base);
  a.rel_hi = (int32_t)(d->hi - a.base);
  a.full_lo = (int32_t)(d->full_lo - a.base);
  a.full_hi = (int32_t)(d->full_hi - a.base);
  if (a.full_lo < a.rel_lo) a.full_lo = a.rel_lo;
  if (a.full_hi > a.rel_hi) a.full_hi = a.rel_hi;
  if (a.full_hi < a.full_lo) a.full_hi = a.full_lo;
  a.ring_slots = d->ring_slots;
  a.ring_base_slot = d->ring_base_slot;
  a.tree = d->mask == VA_MASK_TREE;
  // tree mode: base is 0 (the extent starts at key 0) and the plan keeps
  // prefix_len + live_rows below 2^31; chain modes never read it
  a.tree_lo = a.tree ? (int32_t)d->prefix_len : 0;
  a.scale_log2 = d->scale * LOG2E_F;
  a.t0_rel = (d->mask == VA_MASK_TREE) ? 0 : (int32_t)(d->first_pos - a.base);
  a.window = (d->mask == VA_MASK_WINDOW) ? d->window : 0;
  for (int r = 0; r < VA_MAX_ROWS; ++r) a.anc[r] = d->anc[r];
  a.state = state;
  a.bucket_hi = d->hi;
  if (k_new) {
    a.k_new = (const uint8_t *)k_new;
    a.v_new = (const uint8_t *)v_new;
    a.new_row_stride_b = (int64_t)d->kv_heads * d->head_dim * 2;
    a.kv_capacity = d->kv_capacity;
    a.append_pos0 = d->mask == VA_MASK_TREE ? d->prefix_len : d->first_pos;
  }
  // 16-row blocks per workgroup (the consumer waves W)
  const int rg = d->row_groups;
  const int nb_total = (d->matrix_rows + 16 * rg - 1) / (16 * rg);
  hipError_t e;
  if (k_new && state) {  // bf16 only (checked by the entry points)
    e = d->head_dim == 64 ? dispatch_rows<64, 0, true, true>(a, nb_total, rg, stream)
                          : dispatch_rows<128, 0, true, true>(a, nb_total, rg, stream);
  } else if (k_new) {
    e = d->head_dim == 64 ? dispatch_rows<64, 0, false, true>(a, nb_total, rg, stream)
                          : dispatch_rows<128, 0, false, true>(a, nb_total, rg, stream);
  } else {
    e = state ? dispatch_split<true>(a, nb_total, rg, quant, d->head_dim, stream)
              : dispatch_split<false>(a, nb_total, rg, quant, d->head_dim, stream);
  }
  return e == hipSuccess ? VA_OK : VA_ERR_HIP;
}

va_status combine_impl(const va_plan *plan, const va_state *state, const void *workspace, size_t workspace_bytes,
                       const float *sink, float *out, float *lse, hipStream_t stream) {
  const va_plan_data *d = plan_of(plan);
  if (!d || !out) return VA_ERR_INVALID;
  if (!workspace || workspace_bytes < d->workspace_bytes) return VA_ERR_WORKSPACE;
  if (d->splits > kMaxSplits) return VA_ERR_UNSUPPORTED;
  CombineArgs a;
  a.ws_ml = (const float *)workspace;
  a.ws_o = (const float *)((const uint8_t *)workspace + d->ml_bytes);
  a.sink = sink;
  a.out = out;
  a.lse = lse;
  a.rows = d->rows;
  a.live_rows = d->live_rows;
  a.group = d->group;
  a.mrows = d->matrix_rows;
  a.q_heads = d->q_heads;
  a.kv_heads = d->kv_heads;
  a.splits = d->splits;
  a.head_dim = d->head_dim;
  a.state = state;
  a.tree = d->mask == VA_MASK_TREE;
  a.window = (d->mask == VA_MASK_WINDOW) ? d->window : 0;
  a.ring_slots = d->ring_slots;
  a.bucket_hi = d->hi;
  dim3 grid(d->group, d->kv_heads, d->rows * (d->head_dim / kCombD));
  const hipError_t e = state ? launch_combine<true>(a, grid, d->splits, stream)
                             : launch_combine<false>(a, grid, d->splits, stream);
  return e == hipSuccess ? VA_OK : VA_ERR_HIP;
}

inline bool aligned8(const void *p) { return ((uintptr_t)p & 7u) == 0; }

}  // namespace va_detail
using namespace va_detail;

#ifdef VA_PHASE_TRACE
// Copies the phase records of the last launches: which = 0 for split_kernel
// (24 uint64 per workgroup), 1 for combine_kernel (8); n_wg workgroups to
// host memory.
extern "C" int va_trace_read(int which, uint64_t *dst, int n_wg) {
  if (!dst || n_wg < 0 || n_wg > va_detail::kTraceWG || (which != 0 && which != 1)) return 1;
  const hipError_t e = which == 0
                           ? hipMemcpyFromSymbol(dst, HIP_SYMBOL(va_detail::va_trace_split),
                                                 (size_t)n_wg * 8 * va_detail::va_trace_split_len, 0,
                                                 hipMemcpyDeviceToHost)
                           : hipMemcpyFromSymbol(dst, HIP_SYMBOL(va_detail::va_trace_comb),
                                                 (size_t)n_wg * 8 * va_detail::va_trace_comb_len, 0,
                                                 hipMemcpyDeviceToHost);
  return e == hipSuccess ? 0 : 2;
}
#endif

extern "C" va_status verify_attn_split(const va_plan *plan, const void *q, const void *k, const void *v,
                                       const float *v_scale, int64_t v_scale_head_stride,
                                       int64_t kv_head_stride, int64_t kv_row_stride, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  return split_impl(plan, nullptr, q, k, v, v_scale, v_scale_head_stride, kv_head_stride, kv_row_stride,
                    workspace, workspace_bytes, stream);
}

extern "C" va_status verify_attn_split_append(const va_plan *plan, const void *q, const void *k_new,
                                              const void *v_new, void *k, void *v, int64_t kv_head_stride,
                                              int64_t kv_row_stride, void *workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
  const va_plan_data *d = plan_of(plan);
  if (!d) return VA_ERR_INVALID;
  if (d->kv_fmt != VA_KV_BF16) return VA_ERR_UNSUPPORTED;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return VA_ERR_INVALID;
  const int64_t first = d->mask == VA_MASK_TREE ? d->prefix_len : d->first_pos;
  if (!d->ring_slots && first + d->rows > d->kv_capacity) return VA_ERR_CAPACITY;
  return split_impl(plan, nullptr, q, k, v, nullptr, 0, kv_head_stride, kv_row_stride, workspace, workspace_bytes,
                    stream, k_new, v_new);
}

extern "C" va_status verify_attn_split_append_state(const va_plan *plan, const va_state *state, const void *q,
                                                    const void *k_new, const void *v_new, void *k, void *v,
                                                    int64_t kv_head_stride, int64_t kv_row_stride,
                                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  const va_plan_data *d = plan_of(plan);
  if (!d) return VA_ERR_INVALID;
  if (!state || !aligned8(state)) return VA_ERR_INVALID;
  if (d->kv_fmt != VA_KV_BF16) return VA_ERR_UNSUPPORTED;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return VA_ERR_INVALID;
  return split_impl(plan, state, q, k, v, nullptr, 0, kv_head_stride, kv_row_stride, workspace, workspace_bytes,
                    stream, k_new, v_new);
}

extern "C" va_status verify_attn_combine(const va_plan *plan, const void *workspace, size_t workspace_bytes,
                                         const float *sink, float *out, float *lse, hipStream_t stream) {
  return combine_impl(plan, nullptr, workspace, workspace_bytes, sink, out, lse, stream);
}

extern "C" va_status verify_attn_split_state(const va_plan *plan, const va_state *state, const void *q,
                                             const void *k, const void *v, const float *v_scale,
                                             int64_t v_scale_head_stride, int64_t kv_head_stride,
                                             int64_t kv_row_stride, void *workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
  if (!state || !aligned8(state)) return VA_ERR_INVALID;
  return split_impl(plan, state, q, k, v, v_scale, v_scale_head_stride, kv_head_stride, kv_row_stride,
                    workspace, workspace_bytes, stream);
}

extern "C" va_status verify_attn_combine_state(const va_plan *plan, const va_state *state, const void *workspace,
                                               size_t workspace_bytes, const float *sink, float *out, float *lse,
                                               hipStream_t stream) {
  if (!state || !aligned8(state)) return VA_ERR_INVALID;
  return combine_impl(plan, state, workspace, workspace_bytes, sink, out, lse, stream);
}

// Workspace of verify_attn_noalloc: one copy per GPU, at a per-GPU address
// looked up once per device with hipGetSymbolAddress (host code never passes
// the array's name itself to a kernel or a copy: that is a host-side stand-in,
// not a device address).
static __device__ __align__(256) uint8_t scratch[VA_NOALLOC_WORKSPACE_BYTES];

namespace va_detail {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The array's address on the current device, or nullptr.
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    p = addr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}
}  // namespace va_detail

extern "C" va_status verify_attn_noalloc(const va_plan *plan, const void *q, const void *k, const void *v,
                                         const float *v_scale, int64_t v_scale_head_stride,
                                         int64_t kv_head_stride, int64_t kv_row_stride, const float *sink,
                                         float *out, float *lse, hipStream_t stream) {
  const va_plan_data *d = plan_of(plan);
  if (!d) return VA_ERR_INVALID;
  if (d->workspace_bytes > VA_NOALLOC_WORKSPACE_BYTES) return VA_ERR_WORKSPACE;
  void *ws = scratch_on_current_device();
  if (!ws) return VA_ERR_HIP;
  const va_status st = split_impl(plan, nullptr, q, k, v, v_scale, v_scale_head_stride, kv_head_stride,
                                  kv_row_stride, ws, VA_NOALLOC_WORKSPACE_BYTES, stream);
  if (st != VA_OK) return st;
  return combine_impl(plan, nullptr, ws, VA_NOALLOC_WORKSPACE_BYTES, sink, out, lse, stream);
}

extern "C" va_status swa_ring_write(const void *k_new, const void *v_new, int32_t rows, int64_t first_pos,
                                    int32_t kv_heads, int32_t head_dim, void *k_ring, void *v_ring,
                                    int32_t ring_slots, int64_t kv_head_stride, int64_t kv_row_stride,
                                    hipStream_t stream) {
  if (rows < 0 || rows > VA_MAX_ROWS) return VA_ERR_INVALID;
  if (rows == 0) return VA_OK;
  if (first_pos < 0 || kv_heads < 1 || ring_slots < rows) return VA_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128) return VA_ERR_INVALID;
  if (!k_new || !v_new || !k_ring || !v_ring) return VA_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_ring) || !aligned16(v_ring)) return VA_ERR_INVALID;
  if (kv_head_stride < 0 || kv_row_stride < head_dim) return VA_ERR_INVALID;
  if (((kv_head_stride * 2) & 15) || ((kv_row_stride * 2) & 15)) return VA_ERR_INVALID;
  const int slot0 = (int)(first_pos % ring_slots);
  const int total = rows * kv_heads * (head_dim / 8);
  hipLaunchKernelGGL(ring_write_kernel, dim3((total + 255) / 256), dim3(256), 0, stream,
                     (const uint8_t *)k_new, (const uint8_t *)v_new, rows, kv_heads, head_dim,
                     (uint8_t *)k_ring, (uint8_t *)v_ring, ring_slots, slot0, kv_head_stride * 2,
                     kv_row_stride * 2);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

extern "C" va_status verify_kv_write(const void *k_new, const void *v_new, int32_t rows, int64_t first_pos,
                                     int32_t kv_heads, int32_t head_dim, int32_t kv_fmt, void *k_cache,
                                     void *v_cache, float *v_scale, int64_t v_scale_head_stride,
                                     int64_t kv_capacity, int32_t ring_slots, int64_t kv_head_stride,
                                     int64_t kv_row_stride, hipStream_t stream) {
  if (rows < 0 || rows > 4096) return VA_ERR_INVALID;
  if (kv_heads < 1 || first_pos < 0) return VA_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128) return VA_ERR_INVALID;
  if (kv_fmt != VA_KV_BF16 && kv_fmt != VA_KV_K_E4M3_WHT_V_I8) return VA_ERR_INVALID;
  const bool quant = kv_fmt == VA_KV_K_E4M3_WHT_V_I8;
  if (quant && head_dim != 128) return VA_ERR_UNSUPPORTED;
  if (ring_slots < 0 || (ring_slots > 0 && (ring_slots < rows || ring_slots % VA_TILE != 0))) return VA_ERR_INVALID;
  if (rows == 0) return VA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache) return VA_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)) return VA_ERR_INVALID;
  const int64_t esz = quant ? 1 : 2;
  if (kv_head_stride < 0 || kv_row_stride < head_dim) return VA_ERR_INVALID;
  if (((kv_head_stride * esz) & 15) || ((kv_row_stride * esz) & 15)) return VA_ERR_INVALID;
  if (quant && (!v_scale || v_scale_head_stride < 0)) return VA_ERR_INVALID;
  if (ring_slots == 0 && kv_capacity < first_pos + rows) return VA_ERR_CAPACITY;
  const dim3 grid((unsigned)rows * (unsigned)kv_heads);
  if (quant) {
    hipLaunchKernelGGL(kv_write_kernel<1>, grid, dim3(64), 0, stream, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, kv_heads, head_dim, (uint8_t *)k_cache, (uint8_t *)v_cache,
                       v_scale, v_scale_head_stride, first_pos, ring_slots, kv_head_stride, kv_row_stride);
  } else {
    hipLaunchKernelGGL(kv_write_kernel<0>, grid, dim3(64), 0, stream, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, kv_heads, head_dim, (uint8_t *)k_cache, (uint8_t *)v_cache,
                       v_scale, v_scale_head_stride, first_pos, ring_slots, kv_head_stride * 2,
                       kv_row_stride * 2);
  }
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}
