// Chunked-prefill attention over a head-partitioned KV cache, bf16 MFMA on gfx950.
//
// A chunk holds positions c .. c+m-1 of one or more sequences. Query p attends to every key
// t <= p on a retrieval head (full-cache rows 0..c-1, then the chunk) and, on a streaming
// head, to the keys t <= p with t < S or t >= p - R + 1 (the sink + ring slots held before
// the chunk, then the chunk) (explainer, "Chunked Pre-filling" and "The Full and Streaming
// Attention Masks"). In chunk mode a streaming head sees every token its cache holds before
// the chunk and the chunk causally, the cache being pruned between chunks only (the same
// subsection, Figure 5). The cache is only read; the caller appends the chunk afterwards.
//
// One block = 4 waves = 128 query rows of one (sequence, KV head): 128 / G positions times
// the G query heads of the group, so every K/V tile staged in LDS serves the whole group
// (no KV head is repeated). K and V tiles of 64 keys go straight from global memory into a
// double-buffered LDS ring with global_load_lds_dwordx4 (no registers in flight), rows kept
// in their global order with 16-byte chunks XOR-swizzled per row so that both LDS read
// patterns below are free of bank conflicts. Per tile a wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (keys as MFMA rows, so each lane owns one query and its softmax
// statistics stay in the lane and its partner lane l ^ 32), takes the online softmax in fp32
// (log2 domain, lazy rescale above kTau), rounds P to fp16 (11 significant bits) and
// accumulates O^T += V^T P^T with v_mfma_f32_32x32x16_f16. Each V tile is converted to fp16 in
// LDS once, by the whole block, when it is about to be used (exact for |v| in [2^-14, 65504],
// since bf16 carries 8 significant bits). The V^T operand comes from ds_read_b64_tr_b16, which
// transposes 4x16 blocks of the row-major tile on the way out of LDS. The key order inside a
// 16-key MFMA slab is permuted identically in P and V^T, matching the accumulator layout of
// the first product.
//
// Tiles are classified per block: skipped when no key is visible to any query of the block
// (causally later, or outside every query's sink + recent window), computed without masks
// when every key is visible to every query, and masked per element otherwise. Retrieval
// query tiles, whose key range grows with the cache, are cut into `nsplit` key ranges run
// by separate blocks that write fp32 partials (O, m, l) merged by a second kernel; the
// heaviest query tiles are dispatched first.
#include <hip/hip_runtime.h>

#include "duo_internal.h"

namespace duo {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = kPrefillRows;  // query rows (position, head) per block
constexpr int kBN = 64;              // keys per tile
constexpr float kTau = 8.0f;
constexpr float kMInit = -1e30f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kNoPos = 0x7FFFFFFF;  // key position of an empty or padding slot

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 half8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats to a bf16 pair, round to nearest even (v_cvt_pk_bf16_f32); x in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, bf16x2_t));
}

// Two floats to an fp16 pair, round to nearest even; x in the low half.
__device__ __forceinline__ uint32_t pack_f16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, half2_t));
}

// A bf16 pair to an fp16 pair (exact for magnitudes in [2^-14, 65504]: bf16 carries 8
// significant bits, fp16 11; smaller values round to fp16 subnormals, within 2^-25).
__device__ __forceinline__ uint32_t bf16w_to_f16w(uint32_t w) {
  return pack_f16(__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xFFFF0000u));
}

template <int D>
struct Geo {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per K/V row
  static constexpr int kTileBytes = kBN * kRowBytes;       // one K (or V) tile
  static constexpr int kRowsPerKb = 1024 / kRowBytes;      // rows per 1 KB DMA instruction
  static constexpr int kDmaPerWave = kTileBytes / 1024 / kWaves;
  static constexpr int kSlabs = D / 16;                    // MFMA K-slabs of QK^T
  static constexpr int kDBlocks = D / 32;                  // 32-wide d blocks of O
  static_assert(kDmaPerWave >= 1, "tile must cover every wave");
};

// Physical 16-byte chunk of logical chunk c in LDS row r: c ^ swz(r). With 16 chunks per
// row (256 B, every row on the same banks) swz spreads the 16 rows of a K read over all
// 16 chunk positions, and gives the 4 consecutive rows of a transposed V read distinct
// aligned chunk pairs; with 8 chunks per row (128 B, rows alternate bank halves) the same
// holds per half.
template <int NCH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (NCH == 16) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

// Maximum and sum over the lane pair (l, l ^ 32) that shares one query row. (The VALU row
// swap, v_permlane32_swap, measured 2-3 % slower here than this LDS-pipe shuffle, which
// overlaps the surrounding MFMA work.)
__device__ __forceinline__ float max_pair32(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float sum_pair32(float x) { return x + __shfl_xor(x, 32); }

// Wait until at most N of this wave's vector memory operations are in flight and its LDS
// operations are done, then join the block's barrier. The K/V tiles arrive in LDS by DMA
// (global_load_lds), whose completions the vector memory counter tracks in issue order, so
// waiting for all but the last N DMAs leaves the most recent batch in flight.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt fields: vmcnt low bits 3:0 and high bits 15:14, expcnt 6:4 (7: no wait),
  // lgkmcnt 11:8 (0: wait for all)
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
}

// kMix: the streaming pass of gate-mixed attention (full-cache source, blended output); a
// separate instantiation so that the ordinary kernel carries none of it. kV16: the values
// arrive as fp16 copies (a.v16), so the V tiles need no conversion in LDS.
template <int D, int G, bool kMix, bool kV16 = false>
__global__ void __launch_bounds__(kThreads, 2) prefill_kernel(PrefillArgs a) {
  static_assert(!(kMix && kV16), "the gate-mixed pass reads bf16 values");
  using Gm = Geo<D>;
  constexpr int NCH = Gm::kChunks;
  constexpr int RB = Gm::kRowBytes;
  constexpr int kQpb = kRows / G;  // positions per block
  constexpr int kDma = Gm::kDmaPerWave;
  constexpr int kHalfSlabs = Gm::kSlabs / 2;  // QK^T K-slabs per quarter of a tile's scores
  // Two K buffers, two V buffers (+ key positions): in the iteration of tile i the waves read
  // V(i) and K(i+1) while the DMA fills V(i+1) and K(i+2) into the other buffers.
  __shared__ __attribute__((aligned(1024))) char sK0[Gm::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sK1[Gm::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sV0[Gm::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sV1[Gm::kTileBytes];
  __shared__ int sPos0[kBN];
  __shared__ int sPos1[kBN];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;

  // ---- block -> work item ------------------------------------------------------------
  const int n_ret_blocks = a.nb * a.Hr * a.n_qt * a.nsplit;
  int x = blockIdx.x, split = 0, nsplit = 1, qt, bi, j, cls;
  if (x < n_ret_blocks) {
    split = x % a.nsplit;
    x /= a.nsplit;
    cls = x % a.Hr;
    x /= a.Hr;
    bi = x % a.nb;
    qt = a.n_qt - 1 - x / a.nb;  // most keys first
    j = a.ret_kv[cls];
    nsplit = a.nsplit;
  } else {
    x -= n_ret_blocks;
    cls = x % a.Hs;
    x /= a.Hs;
    bi = x % a.nb;
    qt = a.n_qt - 1 - x / a.nb;
    j = a.str_kv[cls];
  }
  const bool retrieval = blockIdx.x < (unsigned)n_ret_blocks;
  // every held key is visible (retrieval, or a streaming head in chunk mode): causal only
  const bool causal_only = retrieval || a.chunk_mode != 0;
  // the cache part is a full cache, row r holding position r (otherwise the ring)
  const bool full_src = retrieval || kMix;
  const int b = a.b0 + bi;
  const int c0 = a.c0[bi];
  const int S = a.S, R = a.R, SR = a.S + a.R;

  const int ql0 = qt * kQpb;                 // first local position of the tile
  const int ql1 = min(a.m, ql0 + kQpb) - 1;  // last valid local position
  const int p_min = c0 + ql0, p_max = c0 + ql1;

  // this lane's query row (the same row in lanes col and col + 32)
  const int row = wave * 32 + col;
  const int q_local = ql0 + row / G;
  const int g = row % G;
  const bool q_valid = q_local < a.m;
  const int p = c0 + (q_valid ? q_local : ql1);
  // first key of this query's window (every key on a retrieval head)
  const int win_lo = causal_only ? -0x7FFFFFFF : p - a.R + 1;

  // ---- Q^T operand: 16-byte slabs of this lane's query row --------------------------
  bf16x8_t qf[Gm::kSlabs];
  {
    const int ql = q_valid ? q_local : ql1;
    const char* qrow = (const char*)a.q + (((int64_t)bi * a.m + ql) * a.Hq + j * G + g) * RB;
#pragma unroll
    for (int k = 0; k < Gm::kSlabs; ++k)
      qf[k] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qrow + (16 * k + 8 * half) * 2));
  }

  // ---- key tiles: cache part, then chunk part ------------------------------------------
  const int filled = full_src ? c0 : min(c0, SR);  // cache rows holding a token
  int n_cache_tiles;
  const char* cache_k;
  const char* cache_v;
  if (full_src) {
    n_cache_tiles = (c0 + kBN - 1) / kBN;
    const int64_t base = (kMix && !retrieval)
                             ? ((int64_t)(b - a.full_b0) * a.full_heads + a.cls_idx[j]) * a.cap * RB
                             : ((int64_t)(b - a.full_b0) * a.Hr + cls) * a.cap * RB;
    cache_k = (const char*)a.full_k + base;
    cache_v = (const char*)a.full_v +
              (kV16 ? ((int64_t)(b - a.v_b0) * a.Hr + cls) * a.vcap * RB : base);
  } else {
    n_cache_tiles = c0 > 0 ? (SR + kBN - 1) / kBN : 0;
    const int64_t base = ((int64_t)b * a.Hs + cls) * SR * RB;
    cache_k = (const char*)a.str_k + base;
    cache_v = (const char*)a.str_v + base;
  }
  const int n_chunk_tiles = ql1 / kBN + 1;  // causal limit: no key after the last query
  const int n_tiles = n_cache_tiles + n_chunk_tiles;
  const int t_begin = (int)((int64_t)n_tiles * split / nsplit);
  const int t_end = (int)((int64_t)n_tiles * (split + 1) / nsplit);
  const char* chunk_k = (const char*)a.k + ((int64_t)bi * a.m * a.Hkv + j) * RB;
  const char* chunk_v = (const char*)a.v + ((int64_t)bi * a.m * a.Hkv + j) * RB;
  const int64_t chunk_stride = (int64_t)a.Hkv * RB;

  // kind of tile ti: 0 = every key visible to every query, 1 = masked, -1 = skipped
  auto classify = [&](int ti) -> int {
    if (ti < n_cache_tiles) {
      if (ti * kBN >= filled) return -1;  // empty slots only
      if (causal_only) return (ti + 1) * kBN <= filled ? 0 : 1;
      if (kMix) {  // window over full-cache rows: skip rows left of every window
        const int k1 = min(filled, (ti + 1) * kBN) - 1;
        return (ti * kBN >= S && k1 < p_min - R + 1) ? -1 : 1;
      }
      // streaming cache: once every window starts past the cache only sink slots count
      if (ti * kBN >= S && p_min - R + 1 > c0 - 1) return -1;
      return 1;
    }
    const int k0 = c0 + (ti - n_cache_tiles) * kBN;  // first key position
    const int k1 = min(c0 + a.m, k0 + kBN) - 1;       // last valid key position
    const bool all_rows = k0 + kBN <= c0 + a.m;
    if (causal_only) return (all_rows && k1 <= p_min) ? 0 : 1;
    if (k0 >= S && k1 < p_min - R + 1) return -1;  // left of every window
    return (all_rows && k1 <= p_min && k0 >= p_max - R + 1) ? 0 : 1;
  };
  auto next_visible = [&](int ti) {
    while (ti < t_end && classify(ti) < 0) ++ti;
    return ti;
  };

  // Position of key row r of tile ti (kNoPos for an empty slot or padding). A streaming
  // cache slot holds the latest token t < c0 that maps to it: t = idx below S, else the
  // largest t <= c0 - 1 with t = idx (mod R) (the ring's slot map, inverted).
  // With bm = (c0 - 1 - S) mod R (once per block), (c0 - 1 - idx) mod R = bm - (idx - S),
  // plus R when negative, for a ring slot idx in [S, S + R).
  const int ring_bm = (!full_src && c0 > S) ? (c0 - 1 - S) % R : 0;
  auto key_pos = [&](int ti, int r) -> int {
    if (ti < n_cache_tiles) {
      const int idx = ti * kBN + r;
      if (idx >= filled) return kNoPos;
      if (full_src || idx < S) return idx;
      int back = ring_bm - (idx - S);
      back += back < 0 ? R : 0;
      return c0 - 1 - back;
    }
    const int i = (ti - n_cache_tiles) * kBN + r;
    return i < a.m ? c0 + i : kNoPos;
  };

  // Per-lane DMA geometry, fixed for the block: for 1 KB block i of this wave, the tile row
  // this lane copies and the byte offset of the logical chunk that lands in this lane's
  // (swizzled) LDS slot. The wave index is made explicitly uniform so that every LDS
  // destination is scalar arithmetic.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  int dma_r[kDma], dma_c[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    dma_r[i] = (wave_u * kDma + i) * Gm::kRowsPerKb + lane / NCH;
    dma_c[i] = ((lane % NCH) ^ swz<NCH>(dma_r[i])) * 16;
  }
  // Source of tile ti: base pointers, row stride, first source row and the number of rows
  // that hold data (later rows are clamped onto the last one, or onto row 0 for empty
  // streaming slots: finite data in bounds whose weight is zero).
  auto tile_src = [&](int ti, const char*& kb, const char*& vb, int64_t& stride, int& row0,
                      int& nrows) {
    if (ti < n_cache_tiles) {
      kb = cache_k;
      vb = cache_v;
      stride = RB;
      row0 = ti * kBN;
      nrows = filled - row0;
    } else {
      kb = chunk_k;
      vb = chunk_v;
      stride = chunk_stride;
      row0 = (ti - n_cache_tiles) * kBN;
      nrows = a.m - row0;
    }
  };
  // One tensor of tile ti into LDS (rows past the data clamped onto the last one; a batch
  // past the last tile reads row 0 and is never used). The tile's first row is a uniform
  // base and each lane adds a 32-bit offset of one 24-bit multiply-add (tile rows < 64,
  // row strides < 2^24), so issuing a DMA costs about two VALU operations.
  auto issue_one = [&](int ti, bool is_v, char* dst) {
    const char *kb, *vb;
    int64_t stride;
    int row0, nrows;
    tile_src(ti, kb, vb, stride, row0, nrows);
    if (nrows <= 0) {
      row0 = 0;
      nrows = 1;
    }
    const char* base = (is_v ? vb : kb) + (int64_t)row0 * stride;
    const uint32_t st = (uint32_t)stride;
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      const uint32_t r = (uint32_t)min(dma_r[i], nrows - 1);
      const uint32_t off = __umul24(r, st) + (uint32_t)dma_c[i];
      __builtin_amdgcn_global_load_lds((const void*)(base + off),
                                       (lds_void_t*)(dst + (wave_u * kDma + i) * 1024), 16, 0, 0);
    }
  };
  // Key positions of a tile (LDS, for the masks). Written before the iteration's DMAs are
  // issued: any wait on a vector load in between would also wait for those.
  auto write_pos = [&](int ti, int* sp) {
    if (tid < kBN) sp[tid] = key_pos(ti, tid);
  };
  auto issue_k = [&](int ti, char* sk) { issue_one(ti, false, sk); };
  auto issue_v = [&](int ti, char* sv) { issue_one(ti, true, sv); };

  // ---- accumulators --------------------------------------------------------------
  f32x16_t o[Gm::kDBlocks];
#pragma unroll
  for (int db = 0; db < Gm::kDBlocks; ++db) o[db] = f32x16_t{};
  float m = kMInit;    // running maximum of this query (log2 units), same in lanes col, col+32
  float thr = kMInit;  // raw-score threshold (m + kTau) / c2
  float l = 0.f;       // partial softmax sum over this lane's keys
  const float c2 = a.scale_log2, inv_c2 = 1.f / c2;

  // QK^T K-slabs [k0, k0 + n) of 32-key block blk of a tile: S^T += K Q^T (keys as MFMA
  // rows); element 4a + b of s[blk] holds key 8a + 4half + b of the block.
  // The first part of a block (k0 == 0) starts from a zero accumulator.
  auto qk_part = [&](f32x16_t& s, const char* sk, int blk, int k0) {
    const int r = blk * 32 + col;
    const char* krow = sk + r * RB;
    const int sw = swz<NCH>(r);
    bf16x8_t kf[kHalfSlabs];
#pragma unroll
    for (int k = 0; k < kHalfSlabs; ++k)
      kf[k] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(krow + ((2 * (k0 + k) + half) ^ sw) * 16));
#pragma unroll
    for (int k = 0; k < kHalfSlabs; ++k)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], qf[k0 + k],
                                                  (k0 == 0 && k == 0) ? f32x16_t{} : s, 0, 0, 0);
  };

  // One iteration: softmax and PV of the current tile (scores sc, V in sv, key positions in
  // sp), then the scores of the next tile (K in skn) into sn. Every group of MFMAs runs with
  // the LDS reads of the next group's operands in flight (two register sets, the issue order
  // fixed by scheduling barriers); the scores are computed after PV rather than under it so
  // that the current scores are dead by then, which keeps both operand sets in registers
  // without spills.
  auto iterate = [&](f32x16_t (&sc)[2], f32x16_t (&sn)[2], int kind, const char* skn,
                     const char* sv, const int* sp) {
    // V(cur) to fp16 in place (each 16-byte chunk keeps its swizzled place), shared by the
    // block's waves; the barrier waits for these LDS writes only: the DMAs in flight (at most
    // three batches) stay in flight. With fp16 copies of the values there is nothing to
    // convert, and V(cur) is already complete in LDS: the barrier at the end of the previous
    // iteration (or the prologue's) waited for its DMA.
    if constexpr (!kV16) {
      for (int c = tid; c < Gm::kTileBytes / 16; c += kThreads) {
        uint4* chunk = (uint4*)(const_cast<char*>(sv) + c * 16);
        const uint4 w = *chunk;
        *chunk = uint4{bf16w_to_f16w(w.x), bf16w_to_f16w(w.y), bf16w_to_f16w(w.z),
                       bf16w_to_f16w(w.w)};
      }
      wait_vm_barrier<3 * kDma>();
    }
    if (kind != 0) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int4 t4 = *(const int4*)(sp + blk * 32 + 8 * a4 + 4 * half);
          const int tt[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = tt[e];
            const bool vis = (t <= p) & ((t < S) | (t >= win_lo));
            sc[blk][4 * a4 + e] = vis ? sc[blk][4 * a4 + e] : kNegInf;
          }
        }
    }
    // online softmax statistics (row over this lane and lane ^ 32); the rescale branch is
    // taken by the whole wave when any row's maximum moves (al = 1 for the others)
    float mx = kNegInf;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[blk][e]);
    mx = max_pair32(mx);
    const bool up = mx > thr;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float mn = up ? mx * c2 : m;
      const float al = fexp2(m - mn);
      l *= al;
#pragma unroll
      for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= al;
      m = mn;
      thr = up ? (mn + kTau) * inv_c2 : thr;
    }
    // PV over four 16-key slabs; slab k holds keys 16k + {4half..4half+3} then
    // 16k + 8 + {4half..4half+3} in both operands (elements 8(k&1) .. 8(k&1)+7 of block
    // k>>1 of S^T). A transposed read gives lane l the four keys k0..k0+3 at
    // d = 32db + (l & 31), with k0 = 16k + 8part + 4half.
    const int gi = lane >> 4, jj = lane & 15, e4 = jj >> 2, q4 = jj & 3;
    auto load_vt = [&](bf16x8_t (&vf)[Gm::kDBlocks], int k) {
#pragma unroll
      for (int db = 0; db < Gm::kDBlocks; ++db) {
        s16x4_t vt[2];
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const int r = 16 * k + 8 * part + 4 * (gi >> 1) + e4;
          const int d = 32 * db + 16 * (gi & 1) + 4 * q4;
          const int c = (d >> 3) ^ swz<NCH>(r);
          vt[part] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(sv + r * RB + c * 16 + (q4 & 1) * 8));
        }
        const uint2 v0 = __builtin_bit_cast(uint2, vt[0]);
        const uint2 v1 = __builtin_bit_cast(uint2, vt[1]);
        vf[db] = __builtin_bit_cast(bf16x8_t, uint4{v0.x, v0.y, v1.x, v1.y});
      }
    };
    // K operands of quarter q of the next tile's scores (32-key block q >> 1, K-slabs
    // (q & 1) kHalfSlabs ..)
    auto load_k = [&](bf16x8_t (&kf)[kHalfSlabs], int q) {
      const int r = (q >> 1) * 32 + col;
      const char* krow = skn + r * RB;
      const int sw = swz<NCH>(r);
#pragma unroll
      for (int k = 0; k < kHalfSlabs; ++k)
        kf[k] = __builtin_bit_cast(
            bf16x8_t, *(const uint4*)(krow + ((2 * ((q & 1) * kHalfSlabs + k) + half) ^ sw) * 16));
    };
    bf16x8_t vA[Gm::kDBlocks], vB[Gm::kDBlocks];
    bf16x8_t kA[kHalfSlabs], kB[kHalfSlabs];
    load_vt(vA, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int blk = k >> 1, e0 = (k & 1) * 8;
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = fexp2(__builtin_fmaf(sc[blk][e0 + e], c2, -m));
        const float p1 = fexp2(__builtin_fmaf(sc[blk][e0 + e + 1], c2, -m));
        l += p0 + p1;
        pw[e / 2] = pack_f16(p0, p1);
      }
      const half8_t pf = __builtin_bit_cast(half8_t, uint4{pw[0], pw[1], pw[2], pw[3]});
      bf16x8_t (&vf)[Gm::kDBlocks] = (k & 1) ? vB : vA;
      bf16x8_t (&vn)[Gm::kDBlocks] = (k & 1) ? vA : vB;
      // the next slab's operands (after the last slab, the first K operands of the next
      // tile's scores) in flight under these MFMAs
      if (k < 3) load_vt(vn, k + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < Gm::kDBlocks; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, vf[db]), pf,
                                                       o[db], 0, 0, 0);
    }
    // K(next) came by DMA in the previous iteration: wait for it (this iteration's two
    // batches stay in flight), then the scores of the next tile, the K operands of each
    // quarter read under the previous one's MFMAs
    wait_vm_barrier<2 * kDma>();
    load_k(kA, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x8_t (&kf)[kHalfSlabs] = (q & 1) ? kB : kA;
      bf16x8_t (&kn)[kHalfSlabs] = (q & 1) ? kA : kB;
      if (q < 3) load_k(kn, q + 1);
      __builtin_amdgcn_sched_barrier(0);
      const int k0 = (q & 1) * kHalfSlabs;
#pragma unroll
      for (int k = 0; k < kHalfSlabs; ++k)
        sn[q >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            kf[k], qf[k0 + k], (k0 == 0 && k == 0) ? f32x16_t{} : sn[q >> 1], 0, 0, 0);
    }
  };

  // ---- tile loop ------------------------------------------------------------------
  // Prologue: K, V of the first visible tile and K of the second; scores of the first.
  // Iteration i (tiles cur = t_i, nxt = t_i+1, nn = t_i+2): DMA of V(nxt) into the other V
  // buffer and of K(nn) into the K buffer of cur, then iterate(). Its barrier before the
  // scores waits for K(nxt), issued one iteration earlier; the barrier at its end waits for
  // V(nxt) and frees the buffers read in it, while K(nn) stays in flight. So every wait
  // leaves the latest batch in flight, and the counts are constant: past the last tile the
  // batches still go out (in-bounds rows, never read) and the "next" scores are computed
  // from a stale buffer and discarded.
  f32x16_t sA[2], sB[2];
  int cur = next_visible(t_begin);
  if (cur < t_end) {
    int nxt = next_visible(cur + 1);
    write_pos(cur, sPos0);
    issue_k(cur, sK0);
    issue_v(cur, sV0);
    if (nxt < t_end) issue_k(nxt, sK1);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) qk_part(sA[q >> 1], sK0, q >> 1, (q & 1) * kHalfSlabs);
    int kind = classify(cur);
    while (true) {
      // even iteration: scores of cur in sA, V(cur) in sV0, K(nxt) in sK1
      int nn = nxt < t_end ? next_visible(nxt + 1) : t_end;
      if (nxt < t_end) write_pos(nxt, sPos1);
      issue_v(nxt, sV1);
      issue_k(nn, sK0);
      iterate(sA, sB, kind, sK1, sV0, sPos0);
      wait_vm_barrier<kDma>();  // V(nxt) in LDS; K(nn) stays in flight
      if (nxt >= t_end) break;
      cur = nxt;
      nxt = nn;
      kind = classify(cur);
      // odd iteration: scores of cur in sB, V(cur) in sV1, K(nxt) in sK0
      nn = nxt < t_end ? next_visible(nxt + 1) : t_end;
      if (nxt < t_end) write_pos(nxt, sPos0);
      issue_v(nxt, sV0);
      issue_k(nn, sK1);
      iterate(sB, sA, kind, sK0, sV1, sPos1);
      wait_vm_barrier<kDma>();
      if (nxt >= t_end) break;
      cur = nxt;
      nxt = nn;
      kind = classify(cur);
    }
    wait_vm_barrier<0>();  // no DMA into this block's LDS outlives the loop
  }

  // ---- epilogue ---------------------------------------------------------------------
  const float lt = sum_pair32(l);
  if (nsplit > 1) {  // fp32 partial of this key range
    const int64_t item = ((int64_t)bi * a.Hr + cls) * a.n_qt + qt;
    const int64_t prow = (item * nsplit + split) * kRows + row;
#pragma unroll
    for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = db * 32 + 8 * a4 + 4 * half;
        *(float4*)(a.part_o + prow * D + d) =
            float4{o[db][4 * a4], o[db][4 * a4 + 1], o[db][4 * a4 + 2], o[db][4 * a4 + 3]};
      }
    if (half == 0) *(float2*)(a.part_ml + prow * 2) = float2{m, lt};
    return;
  }
  if (!q_valid) return;
  const float inv = 1.f / lt;
  const int64_t orow = ((int64_t)bi * a.m + q_local) * a.Hq + j * G + g;
  // gate-mixed output: out (already holding the full-attention result) keeps weight alpha
  const float keep = kMix ? a.alpha[j] : 0.f;
  const float mine = 1.f - keep;
#pragma unroll
  for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = db * 32 + 8 * a4 + 4 * half;
      float v0 = o[db][4 * a4] * inv, v1 = o[db][4 * a4 + 1] * inv;
      float v2 = o[db][4 * a4 + 2] * inv, v3 = o[db][4 * a4 + 3] * inv;
      if constexpr (kMix) {
        float p0, p1, p2, p3;
        if (a.out_f32) {
          const float4 pv = *(const float4*)((const float*)a.out + orow * D + d);
          p0 = pv.x, p1 = pv.y, p2 = pv.z, p3 = pv.w;
        } else {
          const uint2 pw = *(const uint2*)((const uint16_t*)a.out + orow * D + d);
          p0 = __builtin_bit_cast(float, pw.x << 16);
          p1 = __builtin_bit_cast(float, pw.x & 0xFFFF0000u);
          p2 = __builtin_bit_cast(float, pw.y << 16);
          p3 = __builtin_bit_cast(float, pw.y & 0xFFFF0000u);
        }
        v0 = __builtin_fmaf(keep, p0, mine * v0);
        v1 = __builtin_fmaf(keep, p1, mine * v1);
        v2 = __builtin_fmaf(keep, p2, mine * v2);
        v3 = __builtin_fmaf(keep, p3, mine * v3);
      }
      if (a.out_f32) {
        *(float4*)((float*)a.out + orow * D + d) = float4{v0, v1, v2, v3};
      } else {
        const uint2 w = {pack_bf16(v0, v1), pack_bf16(v2, v3)};
        *(uint2*)((uint16_t*)a.out + orow * D + d) = w;
      }
    }
  if (half == 0 && a.lse) a.lse[orow] = (m + __builtin_log2f(lt)) * kLn2;
}

// Merge of the key-range partials of the retrieval query tiles: one block per (item, 16
// query rows); every thread owns D/16 output columns of one row. M = max_s m_s,
// L = sum_s l_s exp2(m_s - M), out = sum_s O_s exp2(m_s - M) / L, lse = (M + log2 L) ln 2;
// empty ranges (m = kMInit, l = 0) weigh zero.
constexpr int kMergeThreads = 256;
constexpr int kMergeRows = kMergeThreads / 16;

template <int D, int G>
__global__ void __launch_bounds__(kMergeThreads) prefill_merge_kernel(PrefillArgs a) {
  constexpr int kQpb = kRows / G;
  constexpr int kCols = D / 16;
  const int tid = threadIdx.x;
  const int64_t item = blockIdx.x / (kRows / kMergeRows);
  const int row = (int)(blockIdx.x % (kRows / kMergeRows)) * kMergeRows + tid / 16;
  const int d0 = (tid % 16) * kCols;
  const int qt = (int)(item % a.n_qt);
  const int cls = (int)((item / a.n_qt) % a.Hr);
  const int bi = (int)(item / ((int64_t)a.n_qt * a.Hr));
  const int q_local = qt * kQpb + row / G;
  if (q_local >= a.m) return;
  const int g = row % G;
  const int j = a.ret_kv[cls];
  const int ns = a.nsplit;
  const int64_t prow0 = item * ns * kRows + row;

  float M = kMInit;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_ml[(prow0 + (int64_t)s * kRows) * 2]);
  float L = 0.f, O[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) O[c] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const int64_t pr = prow0 + (int64_t)s * kRows;
    const float2 ml = *(const float2*)(a.part_ml + pr * 2);
    const float w = fexp2(ml.x - M);
    L = __builtin_fmaf(w, ml.y, L);
    const float4* src = (const float4*)(a.part_o + pr * D + d0);
#pragma unroll
    for (int c = 0; c < kCols / 4; ++c) {
      const float4 v = src[c];
      O[4 * c] = __builtin_fmaf(w, v.x, O[4 * c]);
      O[4 * c + 1] = __builtin_fmaf(w, v.y, O[4 * c + 1]);
      O[4 * c + 2] = __builtin_fmaf(w, v.z, O[4 * c + 2]);
      O[4 * c + 3] = __builtin_fmaf(w, v.w, O[4 * c + 3]);
    }
  }
  const float inv = 1.f / L;
  const int64_t orow = ((int64_t)bi * a.m + q_local) * a.Hq + j * G + g;
#pragma unroll
  for (int c = 0; c < kCols; c += 2) {
    if (a.out_f32) {
      *(float2*)((float*)a.out + orow * D + d0 + c) = float2{O[c] * inv, O[c + 1] * inv};
    } else {
      *(uint32_t*)((uint16_t*)a.out + orow * D + d0 + c) = pack_bf16(O[c] * inv, O[c + 1] * inv);
    }
  }
  if (tid % 16 == 0 && a.lse) a.lse[orow] = (M + __builtin_log2f(L)) * kLn2;
}

// fp16 copies of the values of one prefill chunk. Grid: (x, group), groups being the
// retrieval prefixes (nb * Hr), then the chunk's values, then the streaming values; every
// thread converts up to kV16PerThread 16-byte chunks of its group, 256 threads apart, all
// loads issued before the first store.
constexpr int kV16PerThread = 8;

__global__ void __launch_bounds__(256) v16_stage_kernel(V16StageArgs a) {
  const int g = blockIdx.y;
  const int64_t row16 = a.D / 8;  // 16-byte chunks per row
  const int npre = a.nb * a.Hr;
  const uint4* src;
  uint4* dst;
  int64_t n;  // chunks of this group
  if (g < npre) {
    const int i = g / a.Hr, r = g % a.Hr;
    src = (const uint4*)a.full_v + ((int64_t)(a.b0 + i) * a.Hr + r) * a.cap * row16;
    dst = (uint4*)a.out_pv + (int64_t)g * a.c_max * row16;
    n = (int64_t)a.c0[i] * row16;
  } else if (g == npre) {
    src = (const uint4*)a.v;
    dst = (uint4*)a.out_chunk;
    n = (int64_t)a.nb * a.m * a.Hkv * row16;
  } else {
    const int64_t off = (int64_t)a.b0 * a.Hs * a.SR * row16;
    src = (const uint4*)a.str_v + off;
    dst = (uint4*)a.out_str + off;
    n = (int64_t)a.nb * a.Hs * a.SR * row16;
  }
  const int64_t c0 = (int64_t)blockIdx.x * 256 * kV16PerThread + threadIdx.x;
  if (c0 >= n) return;
  uint4 w[kV16PerThread];
#pragma unroll
  for (int k = 0; k < kV16PerThread; ++k) {
    const int64_t c = c0 + 256 * k;
    if (c < n) w[k] = src[c];
  }
#pragma unroll
  for (int k = 0; k < kV16PerThread; ++k) {
    const int64_t c = c0 + 256 * k;
    if (c < n)
      dst[c] = uint4{bf16w_to_f16w(w[k].x), bf16w_to_f16w(w[k].y), bf16w_to_f16w(w[k].z),
                     bf16w_to_f16w(w[k].w)};
  }
}

// ---- fp32 inputs ------------------------------------------------------------------------
// The same attention for float32 q, k, v and caches, on v_mfma_f32_16x16x4_f32 with fp32
// accumulation. One block = 4 waves = 64 query rows of one (sequence, KV head), 16 per wave;
// K and V tiles of 32 keys are staged in LDS by plain 16-byte loads, rows padded by 4 words
// so that both read patterns below hit 64 distinct banks. Per tile a wave computes
// S^T = K Q^T (keys as MFMA rows; lane l holds query l % 16 against keys 4 (l / 16) + v of
// each 16-key block), an online softmax in fp32 (log2 domain), and O^T += V^T P^T where the
// k index of step s of a 16-key block is key 4 (l / 16) + s, so that every lane's B operand
// is one of its own softmax weights and P never leaves the lane. Tile classes and masks are
// those of the bf16 kernel. No split-K: every block covers the whole key range of its query
// rows.
constexpr int kF32Rows = 64;  // query rows per block
constexpr int kF32BN = 32;    // keys per tile

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 2) prefill_f32_kernel(PrefillArgs a, int n_qt) {
  constexpr int LD = D + 4;  // padded LDS row, in floats
  constexpr int kQpb = kF32Rows / G;
  constexpr int kSteps = D / 4;    // k steps of S^T over the head dimension
  constexpr int kDBlocks = D / 16;  // 16-wide d blocks of O^T
  __shared__ __attribute__((aligned(16))) float sK[kF32BN * LD];
  __shared__ __attribute__((aligned(16))) float sV[kF32BN * LD];
  __shared__ int sPos[kF32BN];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, qi = lane & 15, kq = lane >> 4;

  // ---- block -> work item (retrieval items first, most keys first) ----------------------
  const int n_ret_blocks = a.nb * a.Hr * n_qt;
  int x = blockIdx.x, qt, bi, j, cls;
  const bool retrieval = x < n_ret_blocks;
  if (retrieval) {
    cls = x % a.Hr;
    x /= a.Hr;
    bi = x % a.nb;
    qt = n_qt - 1 - x / a.nb;
    j = a.ret_kv[cls];
  } else {
    x -= n_ret_blocks;
    cls = x % a.Hs;
    x /= a.Hs;
    bi = x % a.nb;
    qt = n_qt - 1 - x / a.nb;
    j = a.str_kv[cls];
  }
  const bool mixed = a.mixed != 0;
  const bool causal_only = retrieval || a.chunk_mode != 0;
  const bool full_src = retrieval || mixed;
  const int b = a.b0 + bi;
  const int c0 = a.c0[bi];
  const int S = a.S, R = a.R, SR = a.S + a.R;
  const int ql0 = qt * kQpb;
  const int ql1 = min(a.m, ql0 + kQpb) - 1;
  const int p_min = c0 + ql0, p_max = c0 + ql1;

  // this lane's query row
  const int row = wave * 16 + qi;
  const int q_local = ql0 + row / G;
  const int g = row % G;
  const bool q_valid = q_local < a.m;
  const int p = c0 + (q_valid ? q_local : ql1);
  const int win_lo = causal_only ? -0x7FFFFFFF : p - R + 1;

  // B operand of S^T: element kq of each 4-wide slice of this lane's query row
  float qv[kSteps];
  {
    const int ql = q_valid ? q_local : ql1;
    const float* qrow = (const float*)a.q + (((int64_t)bi * a.m + ql) * a.Hq + j * G + g) * D;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qv[s] = qrow[4 * s + kq];
  }

  // ---- key tiles: cache part, then chunk part ------------------------------------------
  const int filled = full_src ? c0 : min(c0, SR);
  int n_cache_tiles;
  const float* cache_k;
  const float* cache_v;
  if (full_src) {
    n_cache_tiles = (c0 + kF32BN - 1) / kF32BN;
    const int64_t base = (mixed && !retrieval)
                             ? ((int64_t)(b - a.full_b0) * a.full_heads + a.cls_idx[j]) * a.cap * D
                             : ((int64_t)(b - a.full_b0) * a.Hr + cls) * a.cap * D;
    cache_k = (const float*)a.full_k + base;
    cache_v = (const float*)a.full_v + base;
  } else {
    n_cache_tiles = c0 > 0 ? (SR + kF32BN - 1) / kF32BN : 0;
    const int64_t base = ((int64_t)b * a.Hs + cls) * SR * D;
    cache_k = (const float*)a.str_k + base;
    cache_v = (const float*)a.str_v + base;
  }
  const int n_tiles = n_cache_tiles + ql1 / kF32BN + 1;
  const float* chunk_k = (const float*)a.k + ((int64_t)bi * a.m * a.Hkv + j) * D;
  const float* chunk_v = (const float*)a.v + ((int64_t)bi * a.m * a.Hkv + j) * D;
  const int64_t chunk_stride = (int64_t)a.Hkv * D;

  // skipped (-1) or computed (masked from the key positions) tile
  auto visible_tile = [&](int ti) -> bool {
    if (ti < n_cache_tiles) {
      if (ti * kF32BN >= filled) return false;
      if (causal_only) return true;
      if (mixed) {
        const int k1 = min(filled, (ti + 1) * kF32BN) - 1;
        return !(ti * kF32BN >= S && k1 < p_min - R + 1);
      }
      return !(ti * kF32BN >= S && p_min - R + 1 > c0 - 1);
    }
    const int k0 = c0 + (ti - n_cache_tiles) * kF32BN;
    const int k1 = min(c0 + a.m, k0 + kF32BN) - 1;
    if (causal_only) return true;
    return !(k0 >= S && k1 < p_min - R + 1);
  };
  const int ring_bm = (!full_src && c0 > S) ? (c0 - 1 - S) % R : 0;
  auto key_pos = [&](int ti, int r) -> int {
    if (ti < n_cache_tiles) {
      const int idx = ti * kF32BN + r;
      if (idx >= filled) return kNoPos;
      if (full_src || idx < S) return idx;
      int back = ring_bm - (idx - S);
      back += back < 0 ? R : 0;
      return c0 - 1 - back;
    }
    const int i = (ti - n_cache_tiles) * kF32BN + r;
    return i < a.m ? c0 + i : kNoPos;
  };

  f32x4_t o[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kMInit, l = 0.f;
  const float c2 = a.scale_log2;

  for (int ti = 0; ti < n_tiles; ++ti) {
    if (!visible_tile(ti)) continue;  // uniform over the block
    // ---- stage the tile (rows past the data clamped onto the last one, or row 0) --------
    const float* kb;
    const float* vb;
    int64_t stride;
    int row0, nrows;
    if (ti < n_cache_tiles) {
      kb = cache_k, vb = cache_v, stride = D, row0 = ti * kF32BN, nrows = filled - row0;
    } else {
      kb = chunk_k, vb = chunk_v, stride = chunk_stride, row0 = (ti - n_cache_tiles) * kF32BN;
      nrows = a.m - row0;
    }
    __syncthreads();  // the previous tile's LDS reads are done
    constexpr int kChunks = kF32BN * D / 4;  // 16-byte chunks per tensor
#pragma unroll
    for (int c = tid; c < kChunks; c += kThreads) {
      const int r = c / (D / 4), c4 = c % (D / 4);
      const int sr = r < nrows ? row0 + r : (nrows > 0 ? row0 + nrows - 1 : 0);
      const float4 kx = *(const float4*)(kb + sr * stride + 4 * c4);
      const float4 vx = *(const float4*)(vb + sr * stride + 4 * c4);
      *(float4*)(sK + r * LD + 4 * c4) = kx;
      *(float4*)(sV + r * LD + 4 * c4) = vx;
    }
    if (tid < kF32BN) sPos[tid] = key_pos(ti, tid);
    __syncthreads();

    // ---- S^T = K Q^T: two 16-key blocks ------------------------------------------------
    f32x4_t s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      s[kb2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const float* krow = sK + (16 * kb2 + qi) * LD + kq;
#pragma unroll
      for (int st = 0; st < kSteps; ++st)
        s[kb2] = __builtin_amdgcn_mfma_f32_16x16x4f32(krow[4 * st], qv[st], s[kb2], 0, 0, 0);
    }
    // ---- masks and online softmax (this query's 32 scores over the 4 lanes qi + 16 kq) ----
    float mx = kNegInf;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = sPos[16 * kb2 + 4 * kq + v];
        const bool vis = (t <= p) & ((t < S) | (t >= win_lo));
        s[kb2][v] = vis ? s[kb2][v] * c2 : kNegInf;
        mx = fmaxf(mx, s[kb2][v]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float al = fexp2(m - mn);
    m = mn;
    l *= al;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[db][v] *= al;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        s[kb2][v] = fexp2(s[kb2][v] - m);
        l += s[kb2][v];
      }
    // ---- O^T += V^T P^T: step st of block kb2 takes key 16 kb2 + 4 kq + st -------------
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float* vrow = sV + (16 * kb2 + 4 * kq + st) * LD + qi;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * db], s[kb2][st], o[db], 0, 0, 0);
      }
  }

  // ---- epilogue: lane (qi, kq) holds d = 16 db + 4 kq .. + 3 of its query ------------------
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (!q_valid) return;
  const float inv = 1.f / l;
  const int64_t orow = ((int64_t)bi * a.m + q_local) * a.Hq + j * G + g;
  float* orow_p = (float*)a.out + orow * D;
  const float keep = mixed ? a.alpha[j] : 0.f;
  const float mine = 1.f - keep;
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) {
    const int d = 16 * db + 4 * kq;
    float4 r = float4{o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv};
    if (mixed) {
      const float4 pv = *(const float4*)(orow_p + d);
      r = float4{__builtin_fmaf(keep, pv.x, mine * r.x), __builtin_fmaf(keep, pv.y, mine * r.y),
                 __builtin_fmaf(keep, pv.z, mine * r.z), __builtin_fmaf(keep, pv.w, mine * r.w)};
    }
    *(float4*)(orow_p + d) = r;
  }
  if (kq == 0 && a.lse && !mixed) a.lse[orow] = (m + __builtin_log2f(l)) * kLn2;
}

template <int D, int G>
int launch_f32(const PrefillArgs& args, void* stream, const KernelMarks& marks) {
  const int n_qt = (args.m + kF32Rows / G - 1) / (kF32Rows / G);
  const int64_t blocks = (int64_t)args.nb * n_qt * ((int64_t)args.Hr + args.Hs);
  if (blocks == 0) return 0;
  if (marks.begin) (void)hipEventRecord((hipEvent_t)marks.begin, (hipStream_t)stream);
  hipLaunchKernelGGL((prefill_f32_kernel<D, G>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, args, n_qt);
  if (marks.end) (void)hipEventRecord((hipEvent_t)marks.end, (hipStream_t)stream);
  return (int)hipGetLastError();
}

template <int D>
int dispatch_f32(int group, const PrefillArgs& a, void* stream, const KernelMarks& m) {
  switch (group) {
    case 1: return launch_f32<D, 1>(a, stream, m);
    case 2: return launch_f32<D, 2>(a, stream, m);
    case 4: return launch_f32<D, 4>(a, stream, m);
    case 8: return launch_f32<D, 8>(a, stream, m);
  }
  return -1;
}

template <int D, int G>
struct Variant {
  static int resident_blocks() {
    static int cached = 0;
    if (cached) return cached;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&prefill_kernel<D, G, false>), kThreads, 0) !=
            hipSuccess ||
        cus <= 0 || per_cu <= 0) {
      (void)hipGetLastError();
      return 512;
    }
    cached = cus * per_cu;
    return cached;
  }
  static int launch(const PrefillArgs& a, void* stream, const KernelMarks& marks) {
    const int64_t blocks = (int64_t)a.nb * a.n_qt * ((int64_t)a.Hr * a.nsplit + a.Hs);
    if (marks.begin) (void)hipEventRecord((hipEvent_t)marks.begin, (hipStream_t)stream);
    if (a.mixed)
      hipLaunchKernelGGL((prefill_kernel<D, G, true>), dim3((unsigned)blocks), dim3(kThreads), 0,
                         (hipStream_t)stream, a);
    else if (a.v16)
      hipLaunchKernelGGL((prefill_kernel<D, G, false, true>), dim3((unsigned)blocks),
                         dim3(kThreads), 0, (hipStream_t)stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<D, G, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                         (hipStream_t)stream, a);
    if (marks.end) (void)hipEventRecord((hipEvent_t)marks.end, (hipStream_t)stream);
    if (a.nsplit > 1 && a.Hr > 0) {
      const int64_t mblocks = (int64_t)a.nb * a.Hr * a.n_qt * (kRows / kMergeRows);
      hipLaunchKernelGGL((prefill_merge_kernel<D, G>), dim3((unsigned)mblocks),
                         dim3(kMergeThreads), 0, (hipStream_t)stream, a);
    }
    return (int)hipGetLastError();
  }
};

template <int D, int G>
int run(bool query, const PrefillArgs* a, void* stream, const KernelMarks* m) {
  return query ? Variant<D, G>::resident_blocks() : Variant<D, G>::launch(*a, stream, *m);
}

template <int D>
int dispatch_g(int group, bool query, const PrefillArgs* a, void* stream, const KernelMarks* m) {
  switch (group) {
    case 1: return run<D, 1>(query, a, stream, m);
    case 2: return run<D, 2>(query, a, stream, m);
    case 4: return run<D, 4>(query, a, stream, m);
    case 8: return run<D, 8>(query, a, stream, m);
  }
  return -1;
}

int dispatch(int head_dim, int group, bool query, const PrefillArgs* a, void* stream,
             const KernelMarks* m) {
  if (head_dim == 128) return dispatch_g<128>(group, query, a, stream, m);
  if (head_dim == 64) return dispatch_g<64>(group, query, a, stream, m);
  return -1;
}

}  // namespace

// Returns -1 for a variant that is not built, else a hipError_t value.
int launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int group, void* stream,
                   const KernelMarks& marks) {
  if (dtype == DUO_F32) {
    if (head_dim == 128) return dispatch_f32<128>(group, a, stream, marks);
    if (head_dim == 64) return dispatch_f32<64>(group, a, stream, marks);
    return -1;
  }
  return dispatch(head_dim, group, false, &a, stream, &marks);
}

int launch_v16_stage(const V16StageArgs& a, void* stream) {
  const int64_t row16 = a.D / 8;
  int64_t n_max = (int64_t)a.c_max * row16;
  n_max = n_max > (int64_t)a.nb * a.m * a.Hkv * row16 ? n_max : (int64_t)a.nb * a.m * a.Hkv * row16;
  n_max = n_max > (int64_t)a.nb * a.Hs * a.SR * row16 ? n_max : (int64_t)a.nb * a.Hs * a.SR * row16;
  const int64_t per_block = 256 * kV16PerThread;
  const int64_t gx = (n_max + per_block - 1) / per_block;
  if (gx == 0) return 0;
  if (gx > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(v16_stage_kernel, dim3((unsigned)gx, (unsigned)(a.nb * a.Hr + 2)), dim3(256),
                     0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int prefill_resident_blocks(int head_dim, int group) {
  return dispatch(head_dim, group, true, nullptr, nullptr, nullptr);
}

}  // namespace duo
