// Multi-row speculative-verification decode attention for gfx950 (CDNA4).
//
// Kernels:
//   split_kernel    one workgroup per (split, KV head); four wave64s stream the
//                   split's 32-key chunks, each wave keeping its own online
//                   softmax state; QK^T and PV run on MFMA 16x16x32 bf16 with
//                   FP32 accumulation; the waves merge through LDS and write
//                   one partial (m, l, O) per matrix row.
//   combine_kernel  one workgroup per (row, query head, 64-wide slice of D):
//                   LSE merge of the partials plus the sink, with the partial
//                   loads issued together into four independent FP32 chains.
//   ring_write_kernel  copies the verification rows' K/V into the window ring.
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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 32;  // keys per wave step
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
  int64_t base;  // absolute position of relative key 0 (= tile_lo * 64)
  int32_t rows, live_rows, group, mrows, q_heads, kv_heads;
  int32_t splits, tiles, tiles_q, tiles_r;  // tiles_q = tiles / splits, tiles_r = tiles % splits
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
};

struct CombineArgs {
  const float *ws_ml;
  const float *ws_o;
  const float *sink;
  float *out;
  float *lse;
  int32_t rows, live_rows, group, mrows, q_heads, kv_heads, splits, head_dim;
};

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max16x4(float x) {
  // max over the four lanes that share lane % 16
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ float wave_sum16x4(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// E4M3FN pair -> two floats (exact), via the gfx950 OCP converter.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float out[4]) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  out[0] = a[0];
  out[1] = a[1];
  out[2] = b[0];
  out[3] = b[1];
}

// LDS DMA: lane l copies `bytes` from its global address to lds + bytes*l
// (the LDS base is wave-uniform).  Kept out of the kernel templates: the
// builtin exists only for the device.
__device__ __forceinline__ void dma16(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 4, 0, 0);
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
// Split kernel.
//   D     head dim (64 or 128)
//   NBW   16-row blocks of query matrix rows per wave (1..3)
//   RG    row groups per workgroup (1: all four waves hold every row and
//         stream different chunks; 2: wave pairs share a chunk, each wave
//         holding half of the rows)
//   FMT   0 = bf16 K/V; 1 = E4M3FN rotated K, INT8 V with per-key scale
// ---------------------------------------------------------------------------
template <int D, int NBW, int RG, int FMT>
__global__ __launch_bounds__(kThreads) void split_kernel(const SplitArgs a) {
  constexpr int KS = D / 32;       // QK contraction steps
  constexpr int MD = D / 16;       // O^T row blocks over d
  constexpr int STREAMS = kWaves / RG;
  constexpr int ROWS_W = NBW * 16;
  // Per-wave staging of one 32-key chunk, filled by LDS DMA: the K tile and
  // the V tile, each 32 rows of KROW bytes made of 16-byte pieces, plus (INT8
  // values) the chunk's scales.  Two such buffers per wave: the next chunk
  // streams in while the current one is computed.
  constexpr int KROW = FMT == 0 ? D * 2 : D;    // bytes per key row
  constexpr int PIECES = KROW / 16;             // 16-byte pieces per row
  constexpr int RPI = 64 / PIECES;              // rows per DMA instruction (1 KiB)
  constexpr int NDMA = kChunk / RPI;            // DMA instructions per tile
  constexpr int kTileB = kChunk * KROW;
  constexpr int kScaleB = FMT == 1 ? 256 : 0;
  constexpr int kBufB = 2 * kTileB + kScaleB;
  constexpr int kStageBytes = kWaves * 2 * kBufB;

  // LDS layout: [Q tile | staging | FP32 WHT scratch (quantised keys only)];
  // the cross-wave merge overlays the Q tile and staging after the loop.
  constexpr int QROWS = 16 * NBW * RG;               // padded query matrix rows
  constexpr int kQT = QROWS * D * 2;                 // bf16 Q tile
  constexpr int kWHT = FMT == 1 ? VA_MAX_MATRIX_ROWS * 128 * 4 : 0;
  constexpr int kMergeBytes = kWaves * ROWS_W * D * 4;  // every wave's O^T tile
  constexpr int kLoop = kQT + kStageBytes + kWHT;    // WHT scratch may not overlay early DMA
  constexpr int kBig = kLoop > kMergeBytes ? kLoop : kMergeBytes;
  constexpr int kML = kWaves * ROWS_W * 3 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kBig + kML];
  uint16_t *qt = (uint16_t *)smem;  // [QROWS][D], 16-byte pieces XOR-swizzled by (row & 15)

  const int lane = threadIdx.x & 63;
  // wave-uniform: keeps chunk indices and mask decisions in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15;
  const int g4 = lane >> 4;
  const int rg = wave % RG;
  const int stream = wave / RG;

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;

  // ---------------- this split's chunk range ----------------
  // Everything the first DMA needs is read here, in straight-line code, so
  // the kernel-argument loads issue together.
  const int32_t tq = a.tiles_q, tr = a.tiles_r, rel_lo = a.rel_lo, rel_hi = a.rel_hi;
  const int32_t ring_slots = a.ring_slots, ring_base = a.ring_base_slot;
  const int64_t kv_base = a.base, row_stride = a.kv_row_stride_b, head_stride = a.kv_head_stride_b;
  const uint8_t *kbase = a.k + (int64_t)kvh * head_stride;
  const uint8_t *vbase = a.v + (int64_t)kvh * head_stride;
  // split s takes q + 1 tiles if s < r, else q (q = T / S, r = T % S)
  const int32_t t0 = split * tq + (split < tr ? split : tr);
  const int32_t t1 = t0 + tq + (split < tr ? 1 : 0);
  int32_t c_first = 2 * t0, c_last = 2 * t1;  // in 32-key chunks, relative
  if (c_first < rel_lo / kChunk) c_first = rel_lo / kChunk;
  const int32_t c_end_ext = (rel_hi + kChunk - 1) / kChunk;
  if (c_last > c_end_ext) c_last = c_end_ext;
  const int32_t nchunks = c_last > c_first ? c_last - c_first : 0;
  // chunks handled by this wave: c_first + stream + STREAMS * n
  const int32_t my_n = nchunks > stream ? (nchunks - stream + STREAMS - 1) / STREAMS : 0;

  uint8_t *stage = smem + kQT + wave * 2 * kBufB;

  // A chunk never straddles the ring's wrap (slots are 64-aligned), so every
  // key of chunk c0 lives at row_of(c0) + (j - c0): one scalar base per chunk
  // plus a 32-bit lane offset.  Keys outside [rel_lo, rel_hi) are clamped to
  // the extent's ends (read, then masked), so nothing outside it is read.
  const uint32_t ring_div = ring_slots > 0 ? (uint32_t)ring_slots : 1u;
  auto chunk_row = [&](int32_t c0) -> int64_t {
    const int64_t ring_row = (int64_t)(((uint32_t)ring_base + (uint32_t)c0) % ring_div);
    return ring_slots ? ring_row : kv_base + c0;
  };
  auto clampx = [&](int32_t x, int32_t c0) -> int32_t {
    const int32_t lo = rel_lo - c0, hi = rel_hi - 1 - c0;
    return x < lo ? lo : (x > hi ? hi : x);
  };
  const uint32_t rs = (uint32_t)row_stride;

  // Piece swizzles inside the staged tiles (position = piece ^ f(row)):
  //   K: f = row % PIECES -> the 16 lanes reading one A operand (16 keys,
  //      same piece) hit 16 different positions.
  //   V (bf16): f = 2 * (row % (PIECES/2)), an even value, so a pair of
  //      pieces {2k, 2k+1} stays a pair; the 16 rows of one transpose read
  //      spread over all bank groups.  V (INT8) is read bytewise, unswizzled.
  auto fk = [](int row) { return row & (PIECES - 1); };
  auto fv = [](int row) { return FMT == 0 ? (2 * row) & (PIECES - 2) : 0; };

  // Issue the LDS DMA of chunk n into buffer `buf` (lane l of instruction t
  // stores 16 bytes at tile + 1024*t + 16*l).  Interior chunks use per-lane
  // byte offsets computed once (row * stride + swizzled piece) on top of the
  // chunk's scalar base; only a chunk that crosses the extent's ends clamps
  // its rows.
  uint32_t koff[NDMA], voff[NDMA];
#pragma unroll
  for (int t = 0; t < NDMA; ++t) {
    const int row = t * RPI + lane / PIECES;
    const int pos = lane % PIECES;
    koff[t] = (uint32_t)row * rs + 16u * (uint32_t)(pos ^ fk(row));
    voff[t] = (uint32_t)row * rs + 16u * (uint32_t)(pos ^ fv(row));
  }
  auto chunk_ptrs = [&](int32_t n, const uint8_t *base) -> const uint8_t * {
    const int32_t c0 = (c_first + stream + STREAMS * n) * kChunk;
    return base + chunk_row(c0) * row_stride;
  };
  // K group of chunk n: NDMA instructions into K buffer `buf`.
  auto issueK = [&](int32_t n, int buf) {
    const int32_t c0 = (c_first + stream + STREAMS * n) * kChunk;
    const uint8_t *kc = chunk_ptrs(n, kbase);
    uint8_t *kt = stage + buf * kBufB;
    if (c0 >= rel_lo && c0 + kChunk <= rel_hi) {
#pragma unroll
      for (int t = 0; t < NDMA; ++t) dma16(kc + koff[t], kt + 1024 * t);
    } else {
#pragma unroll
      for (int t = 0; t < NDMA; ++t) {
        const int row = t * RPI + lane / PIECES;
        const int pos = lane % PIECES;
        dma16(kc + (uint32_t)clampx(row, c0) * rs + 16 * (pos ^ fk(row)), kt + 1024 * t);
      }
    }
  };
  // V group of chunk n: NDMA instructions (+1 for the INT8 scales) into V buffer `buf`.
  auto issueV = [&](int32_t n, int buf) {
    const int32_t c0 = (c_first + stream + STREAMS * n) * kChunk;
    const uint8_t *vc = chunk_ptrs(n, vbase);
    uint8_t *vt = stage + buf * kBufB + kTileB;
    if (c0 >= rel_lo && c0 + kChunk <= rel_hi) {
#pragma unroll
      for (int t = 0; t < NDMA; ++t) dma16(vc + voff[t], vt + 1024 * t);
    } else {
#pragma unroll
      for (int t = 0; t < NDMA; ++t) {
        const int row = t * RPI + lane / PIECES;
        const int pos = lane % PIECES;
        dma16(vc + (uint32_t)clampx(row, c0) * rs + 16 * (pos ^ fv(row)), vt + 1024 * t);
      }
    }
    if constexpr (FMT == 1) {
      const float *sc = a.v_scale + (int64_t)kvh * a.v_scale_head_stride + chunk_row(c0);
      dma4(sc + clampx(lane & 31, c0), vt + kTileB);
    }
  };

  // The first two chunks start streaming before anything else is set up
  // (issue order K0 V0 K1 V1; later groups follow the per-step order below).
  if (my_n > 0) {
    issueK(0, 0);
    issueV(0, 0);
  }
  if (my_n > 1) {
    issueK(1, 1);
    issueV(1, 1);
  }

  // ---------------- Q tile in LDS (B operand of S^T = K Q^T) ----------------
  // Piece p (8 contraction elements) of matrix row m is stored at position
  // p ^ (m % QP), so the lanes reading one operand spread over the banks.
  // Loads are unconditional (padded rows read row 0 and are zeroed), so they
  // all issue before the first wait.
  constexpr int QP = D / 8;  // pieces per row
  if constexpr (FMT == 0) {
    constexpr int kIt = (QROWS * QP + kThreads - 1) / kThreads;
    u32x4 qv[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int idx = threadIdx.x + it * kThreads;
      const int m = idx / QP, pc = idx % QP;
      const int r = m / a.group;
      const bool ok = (idx < QROWS * QP) && (m < a.mrows) && (r < a.live_rows);
      const int rr = ok ? r : 0, h = ok ? kvh * a.group + (m - r * a.group) : 0;
      qv[it] = *(const u32x4 *)(a.q + ((int64_t)(rr * a.q_heads + h) * D + 8 * (ok ? pc : 0)) * 2);
      if (!ok) qv[it] = (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int idx = threadIdx.x + it * kThreads;
      const int m = idx / QP, pc = idx % QP;
      if (idx < QROWS * QP) *(u32x4 *)(qt + m * D + 8 * (pc ^ (m & (QP - 1)))) = qv[it];
    }
    __syncthreads();
  } else {
    // q' = H q / sqrt(128) in FP32 (natural-order Walsh-Hadamard), then bf16.
    float *qs = (float *)(smem + kQT + kStageBytes);
    const int nrows = a.mrows;
    for (int idx = threadIdx.x; idx < nrows * 128; idx += kThreads) {
      const int m = idx >> 7, d = idx & 127;
      const int r = m / a.group;
      const bool ok = r < a.live_rows;
      const int rr = ok ? r : 0, h = ok ? kvh * a.group + (m - r * a.group) : 0;
      const uint16_t u = *(const uint16_t *)(a.q + ((int64_t)(rr * a.q_heads + h) * 128 + d) * 2);
      qs[idx] = ok ? __uint_as_float((uint32_t)u << 16) : 0.f;
    }
    __syncthreads();
#pragma unroll 1
    for (int hstep = 1; hstep < 128; hstep <<= 1) {
      for (int idx = threadIdx.x; idx < nrows * 64; idx += kThreads) {
        const int m = idx >> 6, kk = idx & 63;
        const int i0 = (kk / hstep) * 2 * hstep + (kk % hstep);
        float *row = qs + m * 128;
        const float x0 = row[i0], x1 = row[i0 + hstep];
        row[i0] = x0 + x1;
        row[i0 + hstep] = x0 - x1;
      }
      __syncthreads();
    }
    const float inv = 0.08838834764831845f;  // 1/sqrt(128)
    // Quantised keys use the contraction order: contraction piece p (8
    // elements) holds d = 64*(p/8) + 16*(p%4) + 8*((p/4)%2) + e, so that one
    // 16-byte load of E4M3 codes (d0..d0+15) serves two contraction steps.
    for (int idx = threadIdx.x; idx < QROWS * QP; idx += kThreads) {
      const int m = idx / QP, pc = idx % QP;
      const int d0 = 64 * (pc >> 3) + 16 * (pc & 3) + 8 * ((pc >> 2) & 1);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x0 = 0.f, x1 = 0.f;
        if (m < nrows) {
          x0 = qs[m * 128 + d0 + 2 * e] * inv;
          x1 = qs[m * 128 + d0 + 2 * e + 1] * inv;
        }
        w[e] = pack_bf16x2(x0, x1);
      }
      u32x4 wv = {w[0], w[1], w[2], w[3]};
      *(u32x4 *)(qt + m * D + 8 * (pc ^ (m & (QP - 1)))) = wv;
    }
    __syncthreads();
  }
  // B operand for 16-row block nb of this wave, contraction step ks: lane
  // (i16, g4) holds row 16*(rg*NBW+nb)+i16, contraction piece 4*ks+g4.
  auto qop = [&](int nb, int ks) -> bf16x8 {
    const int m = 16 * (rg * NBW + nb) + i16;
    return __builtin_bit_cast(bf16x8, *(const u32x4 *)(qt + m * D + 8 * ((4 * ks + g4) ^ (m & (QP - 1)))));
  };

  // ---------------- per-lane row geometry for boundary masks ----------------
  // Computed from scalars (no per-lane loads): causal/window rows from their
  // position, tree ancestor bits selected from the sixteen kernel arguments.
  int32_t rlo[NBW], rhi[NBW];
  uint32_t ranc[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int m = 16 * (rg * NBW + nb) + i16;
    const int r = m / a.group;
    const bool ok = (m < a.mrows) && (r < a.live_rows);
    int32_t lo_r, hi_r;
    uint32_t an = 0u;
    if (a.tree) {
      lo_r = 0;
      hi_r = a.tree_lo;
#pragma unroll
      for (int i = 0; i < VA_MAX_ROWS; ++i) an = (r == i) ? a.anc[i] : an;
    } else {
      const int32_t t = a.t0_rel + r;
      hi_r = t + 1;
      lo_r = a.window ? t - a.window + 1 : INT32_MIN;
      if (lo_r < 0) lo_r = 0;
    }
    rlo[nb] = ok ? lo_r : 0;
    rhi[nb] = ok ? hi_r : 0;
    ranc[nb] = ok ? an : 0u;
  }

  // ---------------- online-softmax state ----------------
  f32x4 o[MD][NBW];
  float mref[NBW], mtrue[NBW], lrow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    mref[nb] = -INFINITY;
    mtrue[nb] = -INFINITY;
    lrow[nb] = 0.f;
#pragma unroll
    for (int md = 0; md < MD; ++md) o[md][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // DMA groups complete in issue order (vector-memory operations return in
  // order and only this wave's DMA is in flight), so a wait leaves exactly
  // the groups issued after the one needed.  Per step n the issue order is:
  // [wait K(n)] K(n+2) [wait V(n)] V(n+2).  The compiler does not track LDS
  // written by DMA across loop iterations, hence the explicit waits; their
  // memory clobber keeps the LDS reads below them.
  constexpr int kVmK = NDMA;
  constexpr int kVmV = NDMA + (FMT == 1 ? 1 : 0);

  auto step = [&](int32_t n) {
    const int buf = n & 1;
    const int32_t c0 = (c_first + stream + STREAMS * n) * kChunk;
    const uint8_t *kt = stage + buf * kBufB;
    const uint8_t *vt = kt + kTileB;
    const bool more1 = n + 1 < my_n, more2 = n + 2 < my_n;

    // ---- K(n): after it were issued V(n), and K(n+1), V(n+1) if they exist ----
    if (more1) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kVmV + kVmK + kVmV) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kVmV) : "memory");
    }
    bf16x8 kop[2][KS];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int row = 16 * mb + i16;
      if constexpr (FMT == 0) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kop[mb][ks] = *(const bf16x8 *)(kt + row * KROW + 16 * ((4 * ks + g4) ^ fk(row)));
      } else {
#pragma unroll
        for (int kp2 = 0; kp2 < KS / 2; ++kp2) {
          // 16 E4M3 codes: first 8 -> step 2*kp2, last 8 -> step 2*kp2+1
          const u32x4 w = *(const u32x4 *)(kt + row * KROW + 16 * ((4 * kp2 + g4) ^ fk(row)));
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            float f[8];
            e4m3x4_to_f32(w[2 * half], f);
            e4m3x4_to_f32(w[2 * half + 1], f + 4);
            u32x4 o4 = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                        pack_bf16x2(f[6], f[7])};
            kop[mb][2 * kp2 + half] = __builtin_bit_cast(bf16x8, o4);
          }
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (more2) issueK(n + 2, buf);

    // ---- S^T = K Q^T ----
    f32x4 s[2][NBW];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma16(kop[mb][ks], qop(nb, ks), acc);
        s[mb][nb] = acc;
      }

    // ---- scale, boundary mask, row maxima ----
    const bool full = (c0 >= a.full_lo) && (c0 + kChunk <= a.full_hi);
    float xs[NBW][8], xmax[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      float *x = xs[nb];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * mb + e] = s[mb][nb][e] * a.scale_log2;
      if (!full) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          // branch-free: row interval, or (tree) an ancestor-or-self node key
          const int32_t j = c0 + (t < 4 ? 4 * g4 + t : 16 + 4 * g4 + (t - 4));
          const uint32_t in_row = (uint32_t)(j - rlo[nb]) < (uint32_t)(rhi[nb] - rlo[nb]);
          const uint32_t ti = (uint32_t)(j - a.tree_lo);
          const uint32_t in_tree = (uint32_t)(ti < 16u) & (ranc[nb] >> (ti & 15u));
          x[t] = ((in_row | in_tree) & 1u) ? x[t] : -INFINITY;
        }
      }
      float mx = x[0];
#pragma unroll
      for (int t = 1; t < 8; ++t) mx = fmaxf(mx, x[t]);
      xmax[nb] = wave_max16x4(mx);
    }

    // ---- lazy reference maximum ----
    // Exponents are taken against mref, which moves only when a row's chunk
    // maximum exceeds it by more than kTau (so every p stays <= 2^kTau);
    // moving it rescales that row's O and l (a rare, wave-uniform branch).
    bool need = false;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      mtrue[nb] = fmaxf(mtrue[nb], xmax[nb]);
      need |= (mref[nb] != -INFINITY) && (xmax[nb] > mref[nb] + kTau);
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const bool mv = xmax[nb] > mref[nb] + kTau;
        const float nref = mv ? xmax[nb] : mref[nb];
        const float alpha = (mref[nb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mref[nb] - nref);
        lrow[nb] *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md) o[md][nb] *= alpha;
        mref[nb] = nref;
      }
    }
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) mref[nb] = (mref[nb] == -INFINITY) ? xmax[nb] : mref[nb];

    // ---- V(n): after it were issued K(n+1), V(n+1), K(n+2) if they exist ----
    if (more2) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kVmK + kVmV + kVmK) : "memory");
    } else if (more1) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kVmK + kVmV) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // V^T operand for block md: lane (i16 = d within the block, g4) takes the
    // keys {4g..4g+3, 16+4g..16+4g+3} of column d.
    bf16x8 vop[MD];
    float vs[8];
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
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const int d = 16 * md + i16;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int row = t < 4 ? 4 * g4 + t : 16 + 4 * g4 + (t - 4);
          const int8_t c = *(const int8_t *)(vt + row * KROW + d);
          vop[md][t] = (__bf16)(float)c;  // exact
        }
      }
      const float *sct = (const float *)(vt + kTileB);
#pragma unroll
      for (int t = 0; t < 8; ++t) vs[t] = sct[t < 4 ? 4 * g4 + t : 16 + 4 * g4 + (t - 4)];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (more2) issueV(n + 2, buf);

    // ---- P^T (B operand of PV) and l ----
    uint32_t pb[NBW][4];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const float m_use = (mref[nb] == -INFINITY) ? 0.f : mref[nb];
      float p[8], psum = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        p[t] = __builtin_amdgcn_exp2f(xs[nb][t] - m_use);
        psum += p[t];
      }
      lrow[nb] += psum;
      if constexpr (FMT == 1) {
#pragma unroll
        for (int t = 0; t < 8; ++t) p[t] *= vs[t];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[nb][e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        u32x4 pw = {pb[nb][0], pb[nb][1], pb[nb][2], pb[nb][3]};
        o[md][nb] = mfma16(vop[md], __builtin_bit_cast(bf16x8, pw), o[md][nb]);
      }
  };

  for (int32_t n = 0; n < my_n; ++n) step(n);

  // ---------------- merge the streams of each row group ----------------
  // Each wave publishes, per row, its exponent reference, its true maximum and
  // its l, plus its unnormalised O^T tile.  Then every wave of a row group
  // merges a 1/STREAMS share of the d blocks against the split's true
  // maximum M (weight 2^(ref_w - M) per wave) and stores it.
  __syncthreads();  // every wave has left its loop: the staging area is free
  float *sml = (float *)(smem + kBig);  // [wave][ROWS_W][3]: ref, true max, l
  f32x4 *otile = (f32x4 *)smem;         // [wave][MD][NBW][64 lanes]
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const float lt = wave_sum16x4(lrow[nb]);
    if (g4 == 0) {
      float *e = sml + (wave * ROWS_W + nb * 16 + i16) * 3;
      e[0] = mref[nb];
      e[1] = mtrue[nb];
      e[2] = lt;
    }
#pragma unroll
    for (int md = 0; md < MD; ++md) otile[((wave * MD + md) * NBW + nb) * 64 + lane] = o[md][nb];
  }
  __syncthreads();

  constexpr int MPW = MD / STREAMS;  // d blocks merged and stored by each wave
  const int64_t unit0 = ((int64_t)split * a.kv_heads + kvh) * a.mrows;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int row = nb * 16 + i16;
    float M = -INFINITY;
#pragma unroll
    for (int st = 0; st < STREAMS; ++st) M = fmaxf(M, sml[((st * RG + rg) * ROWS_W + row) * 3 + 1]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float f[STREAMS], L = 0.f;
#pragma unroll
    for (int st = 0; st < STREAMS; ++st) {
      const float *e = sml + ((st * RG + rg) * ROWS_W + row) * 3;
      f[st] = (e[0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(e[0] - Mu);
      L += f[st] * e[2];
    }
    const int m = 16 * (rg * NBW + nb) + i16;
    if (m < a.mrows) {
      const int r = m / a.group;
      const bool live = r < a.live_rows;
      if (stream == 0 && g4 == 0) {
        a.ws_ml[(unit0 + m) * 2 + 0] = live ? M : -INFINITY;
        a.ws_ml[(unit0 + m) * 2 + 1] = live ? L : 0.f;
      }
      float *op = a.ws_o + (unit0 + m) * D;
#pragma unroll
      for (int mi = 0; mi < MPW; ++mi) {
        const int md = stream * MPW + mi;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STREAMS; ++st) acc += f[st] * otile[(((st * RG + rg) * MD + md) * NBW + nb) * 64 + lane];
        if (!live) acc = (f32x4){0.f, 0.f, 0.f, 0.f};
        *(f32x4 *)(op + 16 * md + 4 * g4) = acc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Combine kernel: grid (rows * Hq, D / 64), 1024 threads.
// ---------------------------------------------------------------------------
constexpr int kMaxSplits = 4096;

constexpr int kCombThreads = 1024;
constexpr int kCombGroups = kCombThreads / 64;  // split groups per block
constexpr int kCombBatch = 16;                  // O loads each thread keeps in flight

__global__ __launch_bounds__(kCombThreads) void combine_kernel(const CombineArgs a) {
  constexpr int kPer = kMaxSplits / kCombThreads;  // (m, l) pairs per thread
  __shared__ float wts[kMaxSplits];
  __shared__ float red[2][kCombThreads / 64];
  __shared__ float gsum[kCombGroups][64];

  const int rh = blockIdx.x;
  const int r = rh / a.q_heads, h = rh % a.q_heads;
  const int D = a.head_dim;
  const int t = threadIdx.x;
  const int dl = t & 63, grp = t >> 6;
  const int d = 64 * blockIdx.y + dl;
  float *outp = a.out + ((int64_t)r * a.q_heads + h) * D;

  if (r >= a.live_rows) {  // padding row: no read of the workspace
    if (grp == 0) outp[d] = 0.f;
    if (a.lse && blockIdx.y == 0 && t == 0) a.lse[(int64_t)r * a.q_heads + h] = -INFINITY;
    return;
  }
  const int g = h / a.group;
  const int mrow = r * a.group + (h - g * a.group);
  const int S = a.splits;
  const int64_t stride_unit = (int64_t)a.kv_heads * a.mrows;  // units between splits
  const int64_t unit0 = (int64_t)g * a.mrows + mrow;
  const float sink2 = a.sink ? a.sink[h] * LOG2E_F : -INFINITY;

  // 1) every (m, l) pair of this row, loads issued together, kept in registers
  const f32x2 *ml = (const f32x2 *)a.ws_ml;
  float mv[kPer], lv[kPer];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = t + kCombThreads * i;
    f32x2 x = {-INFINITY, 0.f};
    if (s < S) x = ml[unit0 + s * stride_unit];
    mv[i] = x[0];
    lv[i] = x[1];
    mx = fmaxf(mx, x[0]);
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((t & 63) == 0) red[0][t >> 6] = mx;
  __syncthreads();
  float M = sink2;
#pragma unroll
  for (int i = 0; i < kCombThreads / 64; ++i) M = fmaxf(M, red[0][i]);
  const float Mu = (M == -INFINITY) ? 0.f : M;

  // 2) weights 2^(m_s - M) and the denominator
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = t + kCombThreads * i;
    if (s < S) {
      const float w = __builtin_amdgcn_exp2f(mv[i] - Mu);
      wts[s] = w;
      den += w * lv[i];
    }
  }
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
  if ((t & 63) == 0) red[1][t >> 6] = den;
  __syncthreads();
  float dsum = 0.f;
#pragma unroll
  for (int i = 0; i < kCombThreads / 64; ++i) dsum += red[1][i];
  den = dsum + __builtin_amdgcn_exp2f(sink2 - Mu);

  // 3) weighted sum of O.  Thread group grp takes splits s = grp (mod 16); it
  //    issues up to kCombBatch loads at once, then folds them into four
  //    independent FP32 accumulation chains.
  const float *ob = a.ws_o + unit0 * D + d;
  const int64_t sstride = stride_unit * D;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = grp; s0 < S; s0 += kCombGroups * kCombBatch) {
    float o[kCombBatch];
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) {
      const int s = s0 + kCombGroups * j;
      o[j] = s < S ? ob[(int64_t)s * sstride] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) {
      const int s = s0 + kCombGroups * j;
      if (s < S) acc[j & 3] = fmaf(wts[s], o[j], acc[j & 3]);
    }
  }
  gsum[grp][dl] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();

  // 4) reduce the groups and finish
  if (grp == 0) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kCombGroups; ++i) tot += gsum[i][dl];
    if (M == -INFINITY) {  // nothing visible and no sink
      outp[d] = 0.f;
      if (a.lse && blockIdx.y == 0 && dl == 0) a.lse[(int64_t)r * a.q_heads + h] = -INFINITY;
    } else {
      outp[d] = tot / den;
      if (a.lse && blockIdx.y == 0 && dl == 0)
        a.lse[(int64_t)r * a.q_heads + h] = (Mu + __log2f(den)) * LN2_F;
    }
  }
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
// Host side.
// ---------------------------------------------------------------------------
const va_plan_data *plan_of(const va_plan *plan) {
  if (!plan) return nullptr;
  const va_plan_data *d = reinterpret_cast<const va_plan_data *>(plan);
  return d->magic == VA_PLAN_MAGIC ? d : nullptr;
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

template <int D, int NBW, int RG, int FMT>
hipError_t launch_split(const SplitArgs &a, hipStream_t stream) {
  dim3 grid(a.splits, a.kv_heads);
  hipLaunchKernelGGL((split_kernel<D, NBW, RG, FMT>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, int FMT>
hipError_t dispatch_rows(const SplitArgs &a, int nb_total, hipStream_t stream) {
  switch (nb_total) {
    case 1: return launch_split<D, 1, 1, FMT>(a, stream);
    case 2: return launch_split<D, 2, 1, FMT>(a, stream);
    case 3: return launch_split<D, 3, 1, FMT>(a, stream);
    case 4: return launch_split<D, 2, 2, FMT>(a, stream);
    case 5:
    case 6: return launch_split<D, 3, 2, FMT>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace va_detail
using namespace va_detail;

extern "C" va_status verify_attn_split(const va_plan *plan, const void *q, const void *k, const void *v,
                                       const float *v_scale, int64_t v_scale_head_stride,
                                       int64_t kv_head_stride, int64_t kv_row_stride, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  const va_plan_data *d = plan_of(plan);
  if (!d) return VA_ERR_INVALID;
  if (!workspace || workspace_bytes < d->workspace_bytes) return VA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return VA_ERR_INVALID;
  if (d->splits > kMaxSplits) return VA_ERR_UNSUPPORTED;
  const bool quant = d->kv_fmt == VA_KV_K_E4M3_WHT_V_I8;
  const int64_t esz = quant ? 1 : 2;
  if (d->hi > d->lo) {
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
  a.base = d->tile_lo * VA_TILE;
  a.rows = d->rows;
  a.live_rows = d->live_rows;
  a.group = d->group;
  a.mrows = d->matrix_rows;
  a.q_heads = d->q_heads;
  a.kv_heads = d->kv_heads;
  a.splits = d->splits;
  a.tiles = (int32_t)d->tiles;
  a.tiles_q = (int32_t)(d->tiles / d->splits);
  a.tiles_r = (int32_t)(d->tiles % d->splits);
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
  {
    // tree keys relative to base; clamp far-away values into int32
    int64_t tl = d->prefix_len - a.base;
    a.tree_lo = (int32_t)(tl > (int64_t)1 << 30 ? (int64_t)1 << 30 : tl);
  }
  a.scale_log2 = d->scale * LOG2E_F;
  a.t0_rel = (d->mask == VA_MASK_TREE) ? 0 : (int32_t)(d->first_pos - a.base);
  a.window = (d->mask == VA_MASK_WINDOW) ? d->window : 0;
  for (int r = 0; r < VA_MAX_ROWS; ++r) a.anc[r] = d->anc[r];
  const int nb_total = (d->matrix_rows + 15) / 16;
  hipError_t e;
  if (quant) {
    e = dispatch_rows<128, 1>(a, nb_total, stream);
  } else if (d->head_dim == 64) {
    e = dispatch_rows<64, 0>(a, nb_total, stream);
  } else {
    e = dispatch_rows<128, 0>(a, nb_total, stream);
  }
  return e == hipSuccess ? VA_OK : VA_ERR_HIP;
}

extern "C" va_status verify_attn_combine(const va_plan *plan, const void *workspace, size_t workspace_bytes,
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
  dim3 grid(d->rows * d->q_heads, d->head_dim / 64);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(kCombThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
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
