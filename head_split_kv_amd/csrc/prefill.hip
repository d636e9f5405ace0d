// Chunked-prefill attention over a head-partitioned KV cache, bf16 MFMA on gfx950.
//
// A chunk holds positions c .. c+m-1 of one or more sequences. Query p attends to every key
// t <= p on a retrieval head (full-cache rows 0..c-1, then the chunk) and, on a streaming
// head, to the keys t <= p with t < S or t >= p - R + 1 (the sink + ring slots held before
// the chunk, then the chunk) (explainer, "Chunked Pre-filling" and "The Full and Streaming
// Attention Masks"). The cache is only read; the caller appends the chunk afterwards.
//
// One block = 4 waves = 128 query rows of one (sequence, KV head): 128 / G positions times
// the G query heads of the group, so every K/V tile staged in LDS serves the whole group
// (no KV head is repeated). Per key tile of 64 keys a wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (keys as MFMA rows, so each lane owns one query and the softmax
// row statistics stay in the lane and its partner lane l ^ 32), takes the online softmax in
// fp32 (log2 domain, lazy rescale above kTau), splits P into two bf16 terms (hi + lo, about
// 16 significant bits) and accumulates O^T += V^T P^T with the same MFMA; V is staged
// transposed in LDS for that product. The key order inside a 16-key MFMA slab is permuted
// identically in P and V^T, which matches the accumulator layout of the first product and
// needs no data movement.
//
// Tiles are classified per block: skipped when no key is visible to any query of the block
// (causally later, or outside every query's sink + recent window), computed without masks
// when every key is visible to every query, and masked per element otherwise. Blocks of the
// same (sequence, KV head) are placed on the same XCD so that its L2 serves their shared K/V
// tiles, and query tiles with more keys start first.
#include <hip/hip_runtime.h>

#include "duo_internal.h"

namespace duo {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 128;  // query rows (position, head) per block
constexpr int kBN = 64;     // keys per tile
constexpr int kXcds = 8;
constexpr float kTau = 8.0f;
constexpr float kMInit = -1e30f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kNoPos = 0x7FFFFFFF;  // key position of an empty or padding slot

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats to a bf16 pair, round to nearest even (v_cvt_pk_bf16_f32); x in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, bf16x2_t));
}

// P = hi + lo with hi = bf16(P) and lo = bf16(P - hi): the two bf16 products carry about
// 16 significant bits of each softmax weight into the fp32 accumulation of O.
__device__ __forceinline__ void split_bf16(float x, float y, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(x, y);
  const float hx = __builtin_bit_cast(float, hi << 16);
  const float hy = __builtin_bit_cast(float, hi & 0xFFFF0000u);
  lo = pack_bf16(x - hx, y - hy);
}

template <int D>
struct Geo {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;    // 16-byte chunks per K/V row
  static constexpr int kKStride = kRowBytes + 16;   // LDS K row stride (padding vs conflicts)
  static constexpr int kVStride = kBN * 2 + 8;      // LDS V^T row (one d) stride
  static constexpr int kKLoads = kBN * kChunks / kThreads;         // 16-byte K loads/thread
  static constexpr int kVTasks = (kBN / 2) * kChunks / kThreads;   // row pairs per thread
  static constexpr int kSlabs = D / 16;             // MFMA K-slabs of the QK^T product
  static constexpr int kDBlocks = D / 32;           // 32-wide d blocks of the output
};

enum TileKind : int { kFull = 0, kMasked = 1 };

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 2) prefill_kernel(PrefillArgs a) {
  using Gm = Geo<D>;
  constexpr int kQpb = kRows / G;  // positions per block
  __shared__ __attribute__((aligned(16))) char sK[kBN * Gm::kKStride];
  __shared__ __attribute__((aligned(16))) char sV[D * Gm::kVStride];
  __shared__ int sPos[kBN];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;

  // ---- block -> (sequence, KV head, query tile), XCD-aware ---------------------------------
  const int n_qt = (a.m + kQpb - 1) / kQpb;
  const int n_blocks = a.nb * a.Hkv * n_qt;
  const int per_xcd = (n_blocks + kXcds - 1) / kXcds;
  const int logical = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
  if (logical >= n_blocks) return;
  const int qt = n_qt - 1 - logical % n_qt;  // most keys first
  const int j = (logical / n_qt) % a.Hkv;
  const int bi = logical / (n_qt * a.Hkv);
  const int b = a.b0 + bi;
  const int c0 = a.c0[bi];
  const int ci = a.cls_idx[j];
  const bool retrieval = ci >= 0;
  const int S = a.S, R = a.R, SR = a.S + a.R;
  constexpr int RB = Gm::kRowBytes;

  const int ql0 = qt * kQpb;                        // first local position of the tile
  const int ql1 = min(a.m, ql0 + kQpb) - 1;         // last valid local position
  const int p_min = c0 + ql0, p_max = c0 + ql1;

  // this lane's query row (same row in lanes col and col + 32)
  const int row = wave * 32 + col;
  const int q_local = ql0 + row / G;
  const int g = row % G;
  const bool q_valid = q_local < a.m;
  const int p = c0 + (q_valid ? q_local : ql1);

  // ---- Q^T operand: 16-byte slabs of this lane's query row ------------------------------
  bf16x8_t qf[Gm::kSlabs];
  {
    const int ql = q_valid ? q_local : ql1;
    const char* qrow = (const char*)a.q + (((int64_t)bi * a.m + ql) * a.Hq + j * G + g) * RB;
#pragma unroll
    for (int k = 0; k < Gm::kSlabs; ++k)
      qf[k] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qrow + (16 * k + 8 * half) * 2));
  }

  // ---- key tiles: cache part, then chunk part -----------------------------------------
  int n_cache_tiles;
  const char* cache_k;
  const char* cache_v;
  const int32_t* slots = nullptr;
  if (retrieval) {
    n_cache_tiles = (c0 + kBN - 1) / kBN;
    const int64_t base = ((int64_t)b * a.Hr + ci) * a.cap * RB;
    cache_k = (const char*)a.full_k + base;
    cache_v = (const char*)a.full_v + base;
  } else {
    const int s = -ci - 1;
    n_cache_tiles = c0 > 0 ? (SR + kBN - 1) / kBN : 0;
    const int64_t base = ((int64_t)b * a.Hs + s) * SR * RB;
    cache_k = (const char*)a.str_k + base;
    cache_v = (const char*)a.str_v + base;
    slots = a.slot_pos + (int64_t)b * SR;
  }
  const int n_chunk_tiles = ql1 / kBN + 1;  // causal limit: no key after the last query
  const int n_tiles = n_cache_tiles + n_chunk_tiles;
  const char* chunk_k = (const char*)a.k + ((int64_t)bi * a.m * a.Hkv + j) * RB;
  const char* chunk_v = (const char*)a.v + ((int64_t)bi * a.m * a.Hkv + j) * RB;
  const int64_t chunk_stride = (int64_t)a.Hkv * RB;

  // Returns the tile's kind, or -1 if no key of it is visible to any query of the block.
  auto classify = [&](int ti) -> int {
    if (ti < n_cache_tiles) {
      if (retrieval) return (ti + 1) * kBN <= c0 ? kFull : kMasked;
      // streaming cache: only sink slots can be visible once the window is past the cache
      if (ti * kBN >= S && p_min - R + 1 > c0 - 1) return -1;
      return kMasked;
    }
    const int k0 = c0 + (ti - n_cache_tiles) * kBN;             // first key position
    const int k1 = min(c0 + a.m, k0 + kBN) - 1;                  // last valid key position
    const bool all_rows = k0 + kBN - 1 <= c0 + a.m - 1;
    if (retrieval) return (all_rows && k1 <= p_min) ? kFull : kMasked;
    if (k0 >= S && k1 < p_min - R + 1) return -1;               // left of every window
    return (all_rows && k1 <= p_min && k0 >= p_max - R + 1) ? kFull : kMasked;
  };

  // ---- staging: global -> registers (next tile) -> LDS -------------------------------------
  uint4 kreg[Gm::kKLoads];
  uint4 vreg[Gm::kVTasks][2];
  int pos_reg = kNoPos;
  auto tile_row = [&](int ti, int r, const char*& kp, const char*& vp) -> int {
    // key row r of tile ti: source pointers (always in bounds) and position
    if (ti < n_cache_tiles) {
      const int idx = ti * kBN + r;
      if (retrieval) {
        const int rr = idx < c0 ? idx : c0 - 1;
        kp = cache_k + (int64_t)rr * RB;
        vp = cache_v + (int64_t)rr * RB;
        return idx < c0 ? idx : kNoPos;
      }
      const int rr = idx < SR ? idx : SR - 1;
      kp = cache_k + (int64_t)rr * RB;
      vp = cache_v + (int64_t)rr * RB;
      const int t = idx < SR ? slots[idx] : -1;
      return t >= 0 ? t : kNoPos;
    }
    const int i = (ti - n_cache_tiles) * kBN + r;
    const int ii = i < a.m ? i : a.m - 1;
    kp = chunk_k + (int64_t)ii * chunk_stride;
    vp = chunk_v + (int64_t)ii * chunk_stride;
    return i < a.m ? c0 + i : kNoPos;
  };
  auto load_tile = [&](int ti) {
#pragma unroll
    for (int u = 0; u < Gm::kKLoads; ++u) {
      const int idx = tid + u * kThreads;
      const int r = idx / Gm::kChunks, c = idx % Gm::kChunks;
      const char *kp, *vp;
      tile_row(ti, r, kp, vp);
      kreg[u] = *(const uint4*)(kp + c * 16);
    }
#pragma unroll
    for (int u = 0; u < Gm::kVTasks; ++u) {
      const int idx = tid + u * kThreads;
      const int pr = idx / Gm::kChunks, c = idx % Gm::kChunks;
      const char *kp, *vp0, *vp1;
      // rows of empty slots hold whatever the arena held: stage zeros, since their softmax
      // weight 0 times a non-finite value would still poison the product
      const bool ok0 = tile_row(ti, 2 * pr, kp, vp0) != kNoPos;
      const bool ok1 = tile_row(ti, 2 * pr + 1, kp, vp1) != kNoPos;
      const uint4 z = {0u, 0u, 0u, 0u};
      const uint4 x0 = *(const uint4*)(vp0 + c * 16);
      const uint4 x1 = *(const uint4*)(vp1 + c * 16);
      vreg[u][0] = ok0 ? x0 : z;
      vreg[u][1] = ok1 ? x1 : z;
    }
    if (tid < kBN) {
      const char *kp, *vp;
      pos_reg = tile_row(ti, tid, kp, vp);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < Gm::kKLoads; ++u) {
      const int idx = tid + u * kThreads;
      const int r = idx / Gm::kChunks, c = idx % Gm::kChunks;
      *(uint4*)(sK + r * Gm::kKStride + c * 16) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < Gm::kVTasks; ++u) {
      const int idx = tid + u * kThreads;
      const int pr = idx / Gm::kChunks, c = idx % Gm::kChunks;
      const uint32_t w0[4] = {vreg[u][0].x, vreg[u][0].y, vreg[u][0].z, vreg[u][0].w};
      const uint32_t w1[4] = {vreg[u][1].x, vreg[u][1].y, vreg[u][1].z, vreg[u][1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // d = 8c + 2e (low halves) and 8c + 2e + 1 (high halves); keys 2pr, 2pr + 1
        const uint32_t lo = (w0[e] & 0xFFFFu) | (w1[e] << 16);
        const uint32_t hi = (w0[e] >> 16) | (w1[e] & 0xFFFF0000u);
        *(uint32_t*)(sV + (8 * c + 2 * e) * Gm::kVStride + 4 * pr) = lo;
        *(uint32_t*)(sV + (8 * c + 2 * e + 1) * Gm::kVStride + 4 * pr) = hi;
      }
    }
    if (tid < kBN) sPos[tid] = pos_reg;
  };

  // ---- accumulators ------------------------------------------------------------------
  f32x16_t o[Gm::kDBlocks];
#pragma unroll
  for (int db = 0; db < Gm::kDBlocks; ++db) o[db] = f32x16_t{};
  float m = kMInit;  // running maximum of this query (log2 units), shared by lanes col, col+32
  float thr = kMInit;  // raw-score threshold (m + kTau) / c2
  float l = 0.f;     // partial softmax sum over this lane's keys
  const float c2 = a.scale_log2, inv_c2 = 1.f / c2;

  // first tile that has any visible key
  int ti = 0;
  while (ti < n_tiles && classify(ti) < 0) ++ti;
  if (ti < n_tiles) load_tile(ti);
  while (ti < n_tiles) {
    const int kind = classify(ti);
    store_tile();
    __syncthreads();
    int next = ti + 1;
    while (next < n_tiles && classify(next) < 0) ++next;
    if (next < n_tiles) load_tile(next);  // in flight during this tile's math

    // S^T = K Q^T: two 32-key blocks, keys 8a + 4half + b of block blk in element 4a + b
    f32x16_t s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x16_t{};
      const char* krow = sK + (blk * 32 + col) * Gm::kKStride + 8 * half * 2;
#pragma unroll
      for (int k = 0; k < Gm::kSlabs; ++k) {
        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, *(const uint4*)(krow + 32 * k));
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[k], s[blk], 0, 0, 0);
      }
    }
    if (kind == kMasked) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int4 t4 = *(const int4*)(sPos + blk * 32 + 8 * a4 + 4 * half);
          const int tt[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = tt[e];
            const bool vis = t <= p && (retrieval || t < S || t >= p - R + 1);
            if (!vis) s[blk][4 * a4 + e] = kNegInf;
          }
        }
    }
    // online softmax (row statistics over this lane and lane ^ 32)
    float mx = kNegInf;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[blk][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (mx > thr) {
      const float mn = mx * c2;
      const float al = fexp2(m - mn);
      l *= al;
#pragma unroll
      for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= al;
      m = mn;
      thr = (mn + kTau) * inv_c2;
    }
    uint32_t ph[2][8], pl[2][8];  // P = hi + lo in bf16, pairs of consecutive elements
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = fexp2(__builtin_fmaf(s[blk][e], c2, -m));
        const float p1 = fexp2(__builtin_fmaf(s[blk][e + 1], c2, -m));
        l += p0 + p1;
        split_bf16(p0, p1, ph[blk][e / 2], pl[blk][e / 2]);
      }
    // O^T += V^T P^T over four 16-key slabs; slab k holds keys 16k + {4half..4half+3} and
    // 16k + 8 + {4half..4half+3}, in that order, in both operands
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int blk = k >> 1, e0 = (k & 1) * 4;
      const uint4 hw = {ph[blk][e0], ph[blk][e0 + 1], ph[blk][e0 + 2], ph[blk][e0 + 3]};
      const uint4 lw = {pl[blk][e0], pl[blk][e0 + 1], pl[blk][e0 + 2], pl[blk][e0 + 3]};
      const bf16x8_t pfh = __builtin_bit_cast(bf16x8_t, hw);
      const bf16x8_t pfl = __builtin_bit_cast(bf16x8_t, lw);
#pragma unroll
      for (int db = 0; db < Gm::kDBlocks; ++db) {
        const char* vrow = sV + (db * 32 + col) * Gm::kVStride;
        const uint2 v0 = *(const uint2*)(vrow + (16 * k + 4 * half) * 2);
        const uint2 v1 = *(const uint2*)(vrow + (16 * k + 8 + 4 * half) * 2);
        const uint4 vw = {v0.x, v0.y, v1.x, v1.y};
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, vw);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfh, o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfl, o[db], 0, 0, 0);
      }
    }
    __syncthreads();
    ti = next;
  }

  // ---- epilogue -------------------------------------------------------------------------
  const float lt = l + __shfl_xor(l, 32);
  if (!q_valid) return;
  const float inv = 1.f / lt;
  const int64_t orow = ((int64_t)bi * a.m + q_local) * a.Hq + j * G + g;
#pragma unroll
  for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = db * 32 + 8 * a4 + 4 * half;
      const float v0 = o[db][4 * a4] * inv, v1 = o[db][4 * a4 + 1] * inv;
      const float v2 = o[db][4 * a4 + 2] * inv, v3 = o[db][4 * a4 + 3] * inv;
      if (a.out_f32) {
        *(float4*)((float*)a.out + orow * D + d) = float4{v0, v1, v2, v3};
      } else {
        const uint2 w = {pack_bf16(v0, v1), pack_bf16(v2, v3)};
        *(uint2*)((uint16_t*)a.out + orow * D + d) = w;
      }
    }
  if (half == 0 && a.lse) a.lse[orow] = (m + __builtin_log2f(lt)) * kLn2;
}

template <int D, int G>
int launch_t(const PrefillArgs& a, void* stream) {
  constexpr int kQpb = kRows / G;
  const int64_t n_qt = (a.m + kQpb - 1) / kQpb;
  const int64_t n_blocks = (int64_t)a.nb * a.Hkv * n_qt;
  const int64_t grid = (n_blocks + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((prefill_kernel<D, G>), dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

template <int D>
int launch_g(const PrefillArgs& a, int group, void* stream) {
  switch (group) {
    case 1: return launch_t<D, 1>(a, stream);
    case 2: return launch_t<D, 2>(a, stream);
    case 4: return launch_t<D, 4>(a, stream);
    case 8: return launch_t<D, 8>(a, stream);
  }
  return -1;
}

}  // namespace

// Returns -1 for a variant that is not built (fp32 inputs), else a hipError_t value.
int launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int group, void* stream) {
  if (dtype != DUO_BF16) return -1;
  if (head_dim == 128) return launch_g<128>(a, group, stream);
  if (head_dim == 64) return launch_g<64>(a, group, stream);
  return -1;
}

}  // namespace duo
