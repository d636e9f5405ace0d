// Split-K flash-decode over a head-partitioned KV cache, for gfx950 (wave64).
//
// One work item is (sequence b, KV head j, context split). Retrieval heads attend over rows
// [0, n) of their full cache, dealt to `nsplit` splits in round-robin tiles; a streaming
// head attends over its min(n, S+R) valid slots in one item, which after the append hold
// exactly the sinks and the last R tokens (explainer, "Decoding Procedure", steps 2-4). Row order inside a head does
// not matter to a softmax, so the ring order of the streaming slots needs no unrolling.
//
// Inside a block of 4 waves, every wave streams groups of 64/LPT tokens: LPT lanes (8 or
// 16) share one token row (each lane owns D/LPT elements of it) and every lane keeps the
// running state of all G query heads of the GQA group, so one load of each K/V row serves the
// whole group without repeating KV heads (OpenReview thread, "GQA Compatibility"). Logits are
// reduced over the LPT lanes with DPP, bf16 dot products use v_dot2_f32_bf16 with fp32
// accumulation, and the softmax is online in the log2 domain with a lazy rescale: the running
// maximum of a lane group only moves when a logit exceeds it by more than kTau, which keeps
// every weight below 2^kTau and leaves the quotient out/l exact. At the end the lane groups
// of a wave are merged with lane shuffles, the waves through LDS, and the context splits of a
// retrieval head by a second, small kernel with the log-sum-exp weights exp2(m_i - m).
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "duo_internal.h"

namespace duo {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr float kNegInf = -__builtin_inff();
// Initial running maximum: finite, so exp2(dot * c2 - m) of a masked token (dot = -inf) is
// exactly 0 and exp2(m - m') of an empty group is 0 (or 1 times a zero sum) with no checks.
constexpr float kMInit = -1e30f;
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Butterflies across the 16-lane rows on the VALU (no LDS): v_permlane16_swap (32_swap) with
// x in both operands returns x and its partner at lane ^ 16 (^ 32), in an order that depends
// on the row, so the sum (maximum) of the two results is the butterfly, the same on both
// partners.
__device__ __forceinline__ float xor16_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];  // (bit_cast of a vector element misreads element 1)
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];  // (bit_cast of a vector element misreads element 1)
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float xor16_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];  // (bit_cast of a vector element misreads element 1)
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
__device__ __forceinline__ float xor32_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];  // (bit_cast of a vector element misreads element 1)
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, int out_f32) {
  if (out_f32) {
    ((float*)out)[idx] = v;
  } else if constexpr (sizeof(T) == 2) {
    ((uint16_t*)out)[idx] = f32_to_bf16(v);
  } else {
    ((float*)out)[idx] = v;
  }
}

// Geometry of one K/V row split over LPT lanes (8 or 16) in 16-byte chunks: lane `sub`
// owns chunks sub, sub + LPT, ... of the row.
template <typename T, int D, int LPT>
struct RowGeom {
  static constexpr int kChunks = D * (int)sizeof(T) / 16;
  static constexpr int kCpl = kChunks / LPT;            // chunks per lane
  static constexpr int kEpc = 16 / (int)sizeof(T);      // elements per chunk
  static constexpr int kE = kCpl * kEpc;                // elements per lane (= D / LPT)
  static_assert(kCpl >= 1 && kChunks % LPT == 0, "row must split over the lanes");
  __device__ static int elem_d(int sub, int c, int e) { return (sub + LPT * c) * kEpc + e; }
};

// Sum over each aligned group of LPT lanes; every lane of the group gets the sum.
template <int LPT>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: lane i <-> 7 - i inside 8 lanes
  if constexpr (LPT == 16) x += dpp<0x128>(x);  // row_ror:8: lane ^ 8 inside 16 lanes
  return x;
}

template <typename T, int D, int LPT>
struct Frag {
  uint4 k[RowGeom<T, D, LPT>::kCpl];
  uint4 v[RowGeom<T, D, LPT>::kCpl];
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: every K/V row is read once per step, and the streaming
// hint keeps these reads from displacing other lines in the caches (measured on a plain
// 256 MiB read: about 7.0 TB/s against 6.4 TB/s with ordinary loads).
__device__ __forceinline__ uint4 load_stream(const char* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

template <typename T, int D, int LPT>
__device__ __forceinline__ void load_frag(Frag<T, D, LPT>& f, const char* kbase,
                                          const char* vbase, int64_t row, int sub) {
  constexpr int RB = D * (int)sizeof(T);
#pragma unroll
  for (int c = 0; c < RowGeom<T, D, LPT>::kCpl; ++c) {
    f.k[c] = load_stream(kbase + row * RB + (sub + LPT * c) * 16);
    f.v[c] = load_stream(vbase + row * RB + (sub + LPT * c) * 16);
  }
}

template <typename T, int D, int G, int LPT>
struct QRegs {
  uint4 q[G][RowGeom<T, D, LPT>::kCpl];
};

template <typename T, int D, int G, int LPT>
__device__ __forceinline__ float dot_partial(const Frag<T, D, LPT>& f,
                                             const QRegs<T, D, G, LPT>& q, int g) {
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < RowGeom<T, D, LPT>::kCpl; ++c) {
    const uint32_t kw[4] = {f.k[c].x, f.k[c].y, f.k[c].z, f.k[c].w};
    const uint32_t qw[4] = {q.q[g][c].x, q.q[g][c].y, q.q[g][c].z, q.q[g][c].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (sizeof(T) == 2) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw[w]),
                                              __builtin_bit_cast(bf16x2_t, qw[w]), acc, false);
      } else {
        acc = __builtin_fmaf(__builtin_bit_cast(float, kw[w]), __builtin_bit_cast(float, qw[w]),
                             acc);
      }
    }
  }
  return acc;
}

template <typename T, int D, int G, int LPT>
__device__ __forceinline__ void accumulate_pv(const Frag<T, D, LPT>& f, const float (&p)[G],
                                              float (&o)[G][RowGeom<T, D, LPT>::kE]) {
#pragma unroll
  for (int c = 0; c < RowGeom<T, D, LPT>::kCpl; ++c) {
    const uint32_t vw[4] = {f.v[c].x, f.v[c].y, f.v[c].z, f.v[c].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (sizeof(T) == 2) {
        const float lo = __builtin_bit_cast(float, vw[w] << 16);
        const float hi = __builtin_bit_cast(float, vw[w] & 0xFFFF0000u);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          o[g][c * 8 + 2 * w] = __builtin_fmaf(p[g], lo, o[g][c * 8 + 2 * w]);
          o[g][c * 8 + 2 * w + 1] = __builtin_fmaf(p[g], hi, o[g][c * 8 + 2 * w + 1]);
        }
      } else {
        const float x = __builtin_bit_cast(float, vw[w]);
#pragma unroll
        for (int g = 0; g < G; ++g) o[g][c * 4 + w] = __builtin_fmaf(p[g], x, o[g][c * 4 + w]);
      }
    }
  }
}

// Steps (of 4 * 64 / LPT rows) per tile dealt to one split.
constexpr int kTileSteps = 1;

// Register slots of token groups per wave (NS - 1 groups in flight while one is processed).
template <typename T, int D, int G>
constexpr int stages() { return 3; }

// Lanes per token row: 8 unless the per-lane state of all G heads would not fit the
// register budget of two waves per SIMD, then 16 (halves the elements each lane owns).
template <typename T, int D, int G>
constexpr int lanes_per_token() {
  constexpr int chunks = D * (int)sizeof(T) / 16;
  constexpr int e8 = D / 8;
  constexpr int words8 =
      G * e8 + G * e8 * (int)sizeof(T) / 4 + stages<T, D, G>() * 2 * (chunks / 8) * 4;
  return (words8 > 200 && chunks >= 16) ? 16 : 8;
}

// The leading scalar arguments repeat a.nsplit, a.Hr, a.Hs, a.B, a.nss and whether the step
// is fused (a.new_k != null). They arrive preloaded in SGPRs (the library's build asks for six
// preloaded argument dwords), so a block decodes its work item without a memory round trip
// and its first argument loads (lengths, head tables, pointers) go out together.
template <typename T, int D, int G, int LPT, int NS>
__global__ void __launch_bounds__(kThreads, 2)
    decode_kernel(int32_t lead_nsplit, int32_t lead_hr, int32_t lead_hs, int32_t lead_b,
                  int32_t lead_nss, int32_t lead_fused, DecodeArgs a) {
  using Geo = RowGeom<T, D, LPT>;
  using F = Frag<T, D, LPT>;
  constexpr int kTpw = 64 / LPT;        // tokens per wave per step
  constexpr int kTpb = kWaves * kTpw;   // tokens per block per step
  constexpr int kTile = kTpb * kTileSteps;  // rows per tile of the round-robin split
  constexpr int E = Geo::kE;
  constexpr int RB = D * (int)sizeof(T);
  static_assert(NS == 3 || NS == 4, "3 or 4 register slots");

  __shared__ float s_o[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, grp = lane / LPT, sub = lane % LPT;

  // ---- work item -------------------------------------------------------------------------
  // In a fused step (a.new_k != null) the token at p = n - 1 is not in the cache yet: the
  // cache rows of this item exclude it (and, on a streaming head, the slot it is about to
  // take), and the one block that covers p reads its K/V from the input, then stores them.
  const bool fused = lead_fused != 0;
  // 32-bit work-item arithmetic (blocks < 2^32; a 64-bit division is a long software
  // sequence on the path to the first loads)
  const uint32_t bid = blockIdx.x;
  const uint32_t n_ret_items = (uint32_t)lead_b * lead_hr * lead_nsplit;
  int b, j, split, nsplit, cls;
  int64_t head_row0;  // first row of this head in its cache
  const char* kbase;
  const char* vbase;
  int t1, skip = -1, new_row = -1;  // new_row: cache row of the new token if this block has it
  if (bid < n_ret_items) {
    const uint32_t q = bid / (uint32_t)lead_nsplit;
    split = (int)(bid - q * (uint32_t)lead_nsplit);
    cls = (int)(q % (uint32_t)lead_hr);
    b = (int)(q / (uint32_t)lead_hr);
    j = a.ret_kv[cls];
    nsplit = lead_nsplit;
    const int n = a.n[b];
    t1 = fused ? n - 1 : n;
    if (fused && ((n - 1) / kTile) % nsplit == split) new_row = n - 1;
    head_row0 = ((int64_t)b * lead_hr + cls) * a.cap;
    kbase = (const char*)a.full_k;
    vbase = (const char*)a.full_v;
  } else {
    const uint32_t i = bid - n_ret_items;
    cls = (int)(i % (uint32_t)lead_hs);
    b = (int)(i / (uint32_t)lead_hs);
    j = a.str_kv[cls];
    split = 0;
    nsplit = 1;
    const int n = a.n[b];
    const int SR = a.S + a.R;
    if (!fused) {
      t1 = min(n, SR);
    } else {
      const int pnew = n - 1;
      new_row = pnew < a.S ? pnew : a.S + (pnew - a.S) % a.R;
      // before the ring wraps the new slot is the first unused one; afterwards it holds the
      // evicted token p - R, which is outside the window
      t1 = min(pnew, SR);
      if (pnew >= SR) skip = new_row;
    }
    head_row0 = ((int64_t)b * lead_hs + cls) * (a.S + a.R);
    kbase = (const char*)a.str_k;
    vbase = (const char*)a.str_v;
  }
  kbase += head_row0 * RB;
  vbase += head_row0 * RB;
  const int h0 = j * G;

  // ---- query registers (raw element bits, same chunk layout as K rows) --------------------
  QRegs<T, D, G, LPT> q;
  {
    const char* qb = (const char*)a.q + ((int64_t)b * a.Hq + h0) * RB;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < Geo::kCpl; ++c)
        q.q[g][c] = *(const uint4*)(qb + (int64_t)g * RB + (sub + LPT * c) * 16);
  }
  const float c2 = a.scale_log2;  // logit in log2 units = dot * c2 (c2 > 0)
  const float inv_c2 = 1.f / c2;

  // m: running maximum (log2 units) of this lane group; thr: the raw dot product above which
  // the maximum must move ((m + kTau) / c2), so the hot path compares unscaled dots.
  float m[G], thr[G], l[G], o[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kMInit;
    thr[g] = kMInit;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[g][e] = 0.f;
  }

  // One step: the token of this lane group's row (masked when not valid).
  auto process = [&](const F& f, bool valid) {
    float dz[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      dz[g] = group_sum<LPT>(dot_partial<T, D, G, LPT>(f, q, g));
      dz[g] = valid ? dz[g] : kNegInf;
    }
    bool need = false;
#pragma unroll
    for (int g = 0; g < G; ++g) need |= dz[g] > thr[g];
    if (need) {  // rare after the first token of the group: move the running maximum
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (dz[g] > thr[g]) {
          const float mn = dz[g] * c2;
          const float al = fexp2(m[g] - mn);
          l[g] *= al;
#pragma unroll
          for (int e = 0; e < E; ++e) o[g][e] *= al;
          m[g] = mn;
          thr[g] = (mn + kTau) * inv_c2;
        }
      }
    }
    float p[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      p[g] = fexp2(__builtin_fmaf(dz[g], c2, -m[g]));
      l[g] += p[g];
    }
    accumulate_pv<T, D, G, LPT>(f, p, o);
  };

  // ---- main loop: token groups interleaved over the waves, NS register slots -------------
  // Tiles of kTile rows are dealt round-robin to the splits of a head (tile i to split
  // i mod nsplit), so that at any time the blocks of a head read neighbouring tiles.
  const int ntiles = (t1 + kTile - 1) / kTile;
  const int my_tiles = ntiles > split ? (ntiles - 1 - split) / nsplit + 1 : 0;
  if (my_tiles > 0) {
    const int n_it = my_tiles * kTileSteps;  // steps, the last ones possibly partial
    auto tok_of = [&](int it) {
      const int tl = it / kTileSteps, st = it - tl * kTileSteps;
      return ((tl * nsplit + split) * kTileSteps + st) * kTpb + wave * kTpw + grp;
    };
    auto row_of = [&](int it) -> int64_t {
      const int t = tok_of(it);
      return (int64_t)(t < t1 ? t : t1 - 1);  // clamped: always inside this head's rows
    };
    // Separate variables (not an array) so that the compiler rotates the slots without
    // copies; loads are unconditional so its wait counts stay exact across the back-edge.
    F f0, f1, f2, f3;
    load_frag<T, D, LPT>(f0, kbase, vbase, row_of(0), sub);
    load_frag<T, D, LPT>(f1, kbase, vbase, row_of(1), sub);
    load_frag<T, D, LPT>(f2, kbase, vbase, row_of(2), sub);
    if constexpr (NS == 4) load_frag<T, D, LPT>(f3, kbase, vbase, row_of(3), sub);

    auto valid_at = [&](int it) {
      const int t = tok_of(it);
      return t < t1 && t != skip;
    };
    for (int it = 0; it < n_it; it += NS) {
      process(f0, valid_at(it));
      load_frag<T, D, LPT>(f0, kbase, vbase, row_of(it + NS), sub);
      process(f1, valid_at(it + 1));
      load_frag<T, D, LPT>(f1, kbase, vbase, row_of(it + NS + 1), sub);
      process(f2, valid_at(it + 2));
      load_frag<T, D, LPT>(f2, kbase, vbase, row_of(it + NS + 2), sub);
      if constexpr (NS == 4) {
        process(f3, valid_at(it + 3));
        load_frag<T, D, LPT>(f3, kbase, vbase, row_of(it + NS + 3), sub);
      }
    }
  }

  // ---- fused step: the new token from the input, then its store into the cache -----------
  if (new_row >= 0) {
    const char* nk = (const char*)a.new_k + ((int64_t)b * a.Hkv + j) * RB;
    const char* nv = (const char*)a.new_v + ((int64_t)b * a.Hkv + j) * RB;
    F f;
    load_frag<T, D, LPT>(f, nk, nv, 0, sub);
    process(f, wave == 0 && grp == 0);
    if (wave == 0) {
      constexpr int kRowChunks = RB / 16;
      for (int c = lane; c < 2 * kRowChunks; c += 64) {
        const bool is_v = c >= kRowChunks;
        const int cc = is_v ? c - kRowChunks : c;
        const uint4 x = *(const uint4*)((is_v ? nv : nk) + cc * 16);
        *(uint4*)(const_cast<char*>(is_v ? vbase : kbase) + (int64_t)new_row * RB + cc * 16) = x;
      }
      if (j == 0 && lane == 0) {  // one block per sequence updates the tables
        const int n = a.n[b];
        const int pnew = n - 1;
        const int SR = a.S + a.R;
        a.slot_pos[(int64_t)b * SR + (pnew < a.S ? pnew : a.S + (pnew - a.S) % a.R)] = pnew;
        a.seq_len[b] = n;
      }
    }
  }

  // ---- merge the lane groups of this wave ------------------------------------------------
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = m[g];
    if constexpr (LPT == 8) mx = fmaxf(mx, dpp<0x128>(mx));  // row_ror:8 -> lane ^ 8
    mx = xor16_max(mx);
    mx = xor32_max(mx);
    const float sc = fexp2(m[g] - mx);
    float lg = l[g] * sc;
    if constexpr (LPT == 8) lg += dpp<0x128>(lg);
    lg = xor16_sum(lg);
    lg = xor32_sum(lg);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float x = o[g][e] * sc;
      if constexpr (LPT == 8) x += dpp<0x128>(x);
      x = xor16_sum(x);
      x = xor32_sum(x);
      o[g][e] = x;
    }
    if (grp == 0) {
#pragma unroll
      for (int c = 0; c < Geo::kCpl; ++c)
#pragma unroll
        for (int e = 0; e < Geo::kEpc; ++e)
          s_o[wave][g][Geo::elem_d(sub, c, e)] = o[g][c * Geo::kEpc + e];
      if (sub == 0) {
        s_m[wave][g] = mx;
        s_l[wave][g] = lg;
      }
    }
  }
  __syncthreads();

  // ---- merge the waves; finish or write this split's partial ------------------------------
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, d = idx % D;
    float M = kMInit;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = fexp2(s_m[w][g] - M);
      L += s_l[w][g] * sc;
      O += s_o[w][g][d] * sc;
    }
    const int h = h0 + g;
    if (nsplit == 1) {
      const int64_t oi = ((int64_t)b * a.Hq + h) * D + d;
      store_out<T>(a.out, oi, O / L, a.out_f32);
      if (d == 0 && a.lse) a.lse[(int64_t)b * a.Hq + h] = (M + __builtin_log2f(L)) * kLn2;
    } else {
      const int64_t pi = ((int64_t)b * a.Hq + h) * a.max_splits + split;
      a.part_o[pi * D + d] = O;
      if (d == 0) {
        a.part_ml[pi * 2 + 0] = M;
        a.part_ml[pi * 2 + 1] = L;
      }
    }
  }
}

// ---- 4-bit full caches -------------------------------------------------------------------
// Complete groups of kQ4Group tokens of a retrieval head hold 4-bit codes, and both products
// of a group run on MFMA (v_mfma_f32_16x16x32_f16): the logits, transposed, S^T = K Q'^T of 16
// tokens against the G query heads (columns, padded to 16), and O^T += V^T P'^T over 32
// tokens for 16 channels. Keys share per-channel (scale s_c, zero z_c) in a group, so
// S = sum_c (q_c s_c) k_c + sum_c q_c z_c: the scales are folded into the query operand once
// per group and the zero term is a per-column bias. Values carry per-token (s_t, z_t):
// O = sum_t (p_t s_t) v_t + sum_t p_t z_t, the scales folded into the weights and the zero
// term one sum per query. In the transposed layout a lane's logits are the weights its value
// operand needs, so the softmax stays in registers.
// Codes become fp16 operands with no conversion: masked in place, a code c reads as the fp16
// denormal c 2^-24 (or 16 c 2^-24 for a high nibble), exact and taken as such by the matrix
// unit; the partner operand carries 1/16 where the nibble was high and the products are
// scaled back by 2^24 (also exact). Masking takes the elements of a word in the order
// 0, 4, 1, 5, 2, 6, 3, 7, which the partner operand follows. A wave streams whole groups in
// steps of 32 tokens through two register slots, each refilled two steps ahead as soon as it
// is used, with the next group's (bf16) key parameters also in flight. Codes are stored
// in operand order (layout in duo.h): the KC key words of one token that a lane needs are
// contiguous, and a wave's value words of a step are D / 64 contiguous KB, so every load
// instruction reads one contiguous KB. The incomplete last group (bf16 residual rows) and the
// streaming heads take the bf16 path, in blocks of their own.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Eight codes (byte i: element 2i in the low nibble, 2i + 1 in the high one) as fp16
// denormals: operand slot e holds element kCodeOrder[e] times 2^-24, times 16 in the slots
// where kCodeHigh is set.
constexpr int kCodeOrder[8] = {0, 4, 1, 5, 2, 6, 3, 7};
constexpr bool kCodeHigh[8] = {false, false, true, true, false, false, true, true};
constexpr bool code_tables_match() {  // the closed forms the query fill uses
  for (int e = 0; e < 8; ++e)
    if (kCodeOrder[e] != (e >> 1) + 4 * (e & 1) || kCodeHigh[e] != ((e & 2) != 0)) return false;
  return true;
}
static_assert(code_tables_match(), "slot order: x = e / 2 + 4 (e % 2), high nibble where e & 2");
// (element x sits in slot 2 (x mod 4) + x / 4, the inverse of kCodeOrder)
constexpr float kTwo24 = 16777216.f;
__device__ __forceinline__ half8_t codes_to_f16(uint32_t w) {
  const uint32_t w8 = w >> 8;
  const u32x4_t r = {w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
  return __builtin_bit_cast(half8_t, r);
}
// 8-bit caches: two words of four byte codes (w0 elements 0..3, w1 elements 4..7) as fp16
// denormals c 2^-24 (c <= 255, exact), pair j of the operand holding elements j and j + 4: the
// slot order of codes_to_f16, with no high nibbles.
__device__ __forceinline__ uint32_t byte_pair(uint32_t w0, uint32_t w1, int j) {
  // one v_perm_b32: result bytes (0, 1, 2, 3) = (w0 byte j, 0, w1 byte j, 0); the selector
  // indexes the bytes of {w1, w0} (w0 = bytes 0..3), 0x0c gives a zero byte
  return __builtin_amdgcn_perm(w1, w0, 0x0c000c00u | ((4u + j) << 16) | (uint32_t)j);
}
__device__ __forceinline__ half8_t bytes_to_f16(uint32_t w0, uint32_t w1) {
  const u32x4_t r = {byte_pair(w0, w1, 0), byte_pair(w0, w1, 1), byte_pair(w0, w1, 2),
                     byte_pair(w0, w1, 3)};
  return __builtin_bit_cast(half8_t, r);
}

constexpr int kBfStages = 6;  // bf16 row fragments in flight in decode_q4_kernel

// What a wave's look-ahead reads when it has no group there: always-valid memory that stays
// in cache (the values are never used). 16 KB covers every offset a look-ahead adds.
__device__ __attribute__((aligned(256))) uint32_t g_q4_idle[4096];

// Pre-RoPE keys (kRope; a.rope_base and a.rope_tau16 set): a key of position t = 128 g + tau
// is attended turned by RoPE at t, R(t) = R(128 g) R(tau) pair by pair, so a query q meets it
// as R(-128 g) q . R(tau) k. Per group the query is turned by -128 g (float32 tables, fp16
// operand) and the scales are no longer folded into it: each dequantized key c s + z is
// formed in packed fp16 (a code OR 0x6400 reads as 1024 + c, exact, minus 1024) and turned
// by tau from an fp16 table in LDS, and the MFMA takes the turned keys as its A operand in
// real units. The bf16 rows (the residual group, streaming slots at the positions they hold,
// a fused step's token) are turned in float32 and dotted with the query in float32; every
// cache keeps the keys as given.
// 8-bit caches (BITS = 8) run the same kernel: a token's key codes and a step's value codes
// take twice the words (bytes_to_f16 instead of codes_to_f16, same operand slots), and no
// operand carries the 1/16 of high nibbles.
// Leading arguments as for decode_kernel.
template <int D, int G, int LPT, int NS, bool kRope, int BITS>
__global__ void __launch_bounds__(kThreads, kRope ? 1 : 2)
    decode_q4_kernel(int32_t lead_nsplit, int32_t lead_hr, int32_t lead_hs, int32_t lead_b,
                     int32_t lead_nss, int32_t lead_fused, DecodeArgs a) {
  using T = uint16_t;
  using Geo = RowGeom<T, D, LPT>;
  using F = Frag<T, D, LPT>;
  constexpr int kCpl = Geo::kCpl;
  constexpr int kTpw = 64 / LPT;
  constexpr int kTpb = kWaves * kTpw;
  constexpr int RB = D * 2;
  constexpr int CBY = D * BITS / 8;  // code bytes of one key token row
  constexpr int KC = D / 32;   // 32-channel k-chunks of the logit product
  constexpr int CBK = D / 16;  // 16-channel blocks of the value product
  constexpr int KW = KC * BITS / 4;   // key code words of a lane per token
  constexpr int VW = CBK * BITS / 4;  // value code words of a lane per step
  static_assert(BITS == 4 || BITS == 8, "4- or 8-bit codes");
  constexpr int kStep = 32;    // tokens per wave step
  constexpr int kSteps = kQ4Group / kStep;
  static_assert(G <= 16 && kSteps % 2 == 0, "query rows must fit the 16-row tile");
  constexpr int kRotRow = D / 2 + 4;  // words of one tau16 row

  __shared__ float s_o[2 * kWaves][G][D];  // partials: bf16 path per wave, then MFMA path
  __shared__ float s_m[2 * kWaves][G];
  __shared__ float s_l[2 * kWaves][G];
  // the G query rows in bf16, then a zero row that the padding columns read
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G + 1][D];
  // the query in float32 in operand slot order (slot e of the 8-channel block at 8 b holds
  // channel 8 b + kCodeOrder[e]), over 16 in the high-nibble slots of 4-bit codes; row G zero
  __shared__ __attribute__((aligned(16))) float s_qf[kRope ? 1 : G + 1][kRope ? 4 : D];
  __shared__ __attribute__((aligned(16))) uint32_t s_rot[kRope ? kQ4Group * kRotRow : 4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, grp = lane / LPT, sub = lane % LPT;
  const int col = lane & 15;              // MFMA column: the query of S^T and of O^T

  // ---- work item -------------------------------------------------------------------------
  // Blocks: the quantized groups of every (sequence, retrieval head) over lead_nsplit splits;
  // one block per (sequence, retrieval head) for its bf16 residual rows, which starts
  // reading them at once instead of after some split's groups; then the streaming windows,
  // each over lead_nss blocks. A retrieval head's partials are its nsplit splits plus the
  // residual block's. In a fused step (a.new_k != null) the token at p = a.n[b] - 1 is not
  // in the cache yet and completes no group: the residual block (or the last block of the
  // streaming window) also takes it from the input and then stores it, as in decode_kernel.
  const bool fused = lead_fused != 0;
  // 32-bit work-item arithmetic, as in decode_kernel
  const uint32_t bid = blockIdx.x;
  const uint32_t n_ret_items = (uint32_t)lead_b * lead_hr * lead_nsplit;
  const uint32_t n_res_items = (uint32_t)lead_b * lead_hr;
  const bool ret = bid < n_ret_items;
  const bool res = !ret && bid < n_ret_items + n_res_items;
  int b, j, split, nsplit, nparts, n;  // n: tokens in the cache (streaming: slots of this block)
  int new_row = -1, skip = -1, r0 = 0;  // r0: first bf16 row of this block
  const char* kq = nullptr;  // retrieval head: K region (codes, parameters, residual)
  const char* vq = nullptr;
  const char* kbase;         // bf16 rows: the residual group, or the streaming slots
  const char* vbase;
  if (ret || res) {
    int cls;
    if (ret) {
      const uint32_t q = bid / (uint32_t)lead_nsplit;
      split = (int)(bid - q * (uint32_t)lead_nsplit);
      cls = (int)(q % (uint32_t)lead_hr);
      b = (int)(q / (uint32_t)lead_hr);
    } else {
      const uint32_t i = bid - n_ret_items;
      split = lead_nsplit;  // the partial after the splits'
      cls = (int)(i % (uint32_t)lead_hr);
      b = (int)(i / (uint32_t)lead_hr);
    }
    j = a.ret_kv[cls];
    nsplit = lead_nsplit;
    nparts = lead_nsplit + 1;
    n = fused ? a.n[b] - 1 : a.n[b];
    if (res && fused) new_row = n % kQ4Group;
    const int64_t head = ((int64_t)b * lead_hr + cls) * a.q4_stride;
    kq = (const char*)a.full_k + head;
    vq = (const char*)a.full_v + head;
    kbase = kq + a.q4_resid;
    vbase = vq + a.q4_resid;
  } else {
    // a streaming head's window is cut over lead_nss blocks; the last one takes the fused
    // step's token
    const uint32_t i = bid - n_ret_items - n_res_items;
    nsplit = nparts = lead_nss;
    const uint32_t q = i / (uint32_t)nsplit;
    split = (int)(i - q * (uint32_t)nsplit);
    const int cls = (int)(q % (uint32_t)lead_hs);
    b = (int)(q / (uint32_t)lead_hs);
    j = a.str_kv[cls];
    const int SR = a.S + a.R;
    int nw;  // held slots of the window
    if (!fused) {
      nw = min(a.n[b], SR);
    } else {
      const int pnew = a.n[b] - 1;
      const int slot = pnew < a.S ? pnew : a.S + (pnew - a.S) % a.R;
      nw = min(pnew, SR);
      if (pnew >= SR) skip = slot;  // the evicted token p - R, outside the window
      if (split == nsplit - 1) new_row = slot;
    }
    const int per = (nw + nsplit - 1) / nsplit;
    r0 = min(nw, split * per);
    n = min(nw, r0 + per) - r0;
    const int64_t row0 = ((int64_t)b * lead_hs + cls) * SR;
    kbase = (const char*)a.str_k + row0 * RB;
    vbase = (const char*)a.str_v + row0 * RB;
  }
  const int h0 = j * G;
  const float c2 = a.scale_log2;
  const float inv_c2 = 1.f / c2;

  // ---- quantized groups on MFMA ------------------------------------------------------------
  // The logits come transposed, S^T = K' Q'^T: lane (col, jj = lane / 16) holds query col's
  // logits of tokens 4 jj + i (tile 0) and 16 + 4 jj + i (tile 1), i = 0..3, of a 32-token
  // step, which are the very weights its B operand of the value product takes (the value
  // codes are stored in that token order), so P' never leaves the lane. State of query col,
  // per lane: running maximum (log2 units, equal in the 4 lanes of col), its raw-product
  // threshold, and this lane's parts of the weight sum and the value-zero sum. Columns past G
  // carry a zero query, never move their maximum (threshold +inf) and weigh
  // exp2(x - 1e30) = 0.
  const int jj = lane >> 4;
  const bool live = col < G;
  float mq = live ? kMInit : 1e30f;
  float thq = live ? kMInit : __builtin_inff();
  float lq = 0.f, zq = 0.f;
  // The logit products accumulate without the group's key-zero term (bias): the threshold is
  // compared as thb = thq - bias, and the weight of a product x is exp2(x c2s + nb) with
  // nb = bias c2s - mq (both set by fold() and on a rescale).
  float thb = thq, nb = -mq;
  // logit (log2 units) per unit of the raw product (codes read as multiples of 2^-24, or the
  // turned keys in real units)
  const float c2s = kRope ? c2 : c2 * kTwo24;
  const float inv_c2s = 1.f / c2s;
  f32x4_t oacc[CBK];  // O^T: lane holds channels 16 cb + 4 jj + i of query col
#pragma unroll
  for (int cb = 0; cb < CBK; ++cb) oacc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Groups of a retrieval head: chunks of kWaves consecutive groups are dealt round-robin
  // to the splits, and wave w of a split takes group w of each of its chunks (wave gw of the
  // head takes groups i W + gw), so the blocks of a head read neighbouring groups at any
  // time. The ng - q W groups left over after q whole rounds go by steps when there are
  // enough waves: the four waves of block k each take one 32-token step of leftover group
  // k, instead of a few waves taking a whole extra group and ending last.
  const int ng = ret ? n / kQ4Group : 0;
  const int W = kWaves * nsplit, gw = kWaves * split + wave;
  const int q_rounds = ng / W, rem = ng - q_rounds * W;
  const bool by_steps = 4 * rem <= W;
  const int n_full = q_rounds + (!by_steps && gw < rem ? 1 : 0);  // whole groups of the wave
  const int t_step = by_steps && gw < 4 * rem ? gw % kSteps : -1;   // its leftover step, if any
  const int t_group = q_rounds * W + gw / kSteps;
  const int n_wave = n_full + (t_step >= 0 ? 1 : 0);
  auto group_of = [&](int i) {  // clamped past the last group
    const int ii = i < n_wave ? i : n_wave - 1;
    return ii == n_full && t_step >= 0 ? t_group : ii * W + gw;
  };
  {
    const uint16_t* kpar = (const uint16_t*)(kq + a.q4_params);  // bf16 [group][2][D]
    // bf16 key scale and zero of this lane's operand channels 32 kc + 8 jj + e
    uint4 ps[KC], pz[KC];
    // kRope: (cos, sin) of the group's base angle 128 g f_i of pairs 32 kh + 8 jj + 2 k, + 1
    [[maybe_unused]] float4 bq[KC / 2][4];
    const char* idle = (const char*)g_q4_idle;
    auto load_params = [&](int gi) {
      const uint16_t* p = kpar + (int64_t)group_of(gi) * 2 * D;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int ch = 32 * kc + 8 * jj;
        ps[kc] = *(const uint4*)(p + ch);
        pz[kc] = *(const uint4*)(p + D + ch);
      }
      if constexpr (kRope) {
        const float4* bp = (const float4*)(a.rope_base + (int64_t)group_of(gi) * D);
#pragma unroll
        for (int kh = 0; kh < KC / 2; ++kh)
#pragma unroll
          for (int k = 0; k < 4; ++k) bq[kh][k] = bp[(32 * kh + 8 * jj) / 2 + k];
      }
    };
    half8_t qa[KC];  // B operand: Q'^T, channel slots of query col
    float bias;      // key-zero term of query col, in units of the raw product
    // kRope: fp16 (scale, scale) and (zero, zero) of the channels of slot pair j of chunk kc
    // (elements j and j + 4; the scale over 16 where the nibbles are high)
    [[maybe_unused]] half2_t rs[KC][4], rz[KC][4];
    auto fold = [&]() {
      if constexpr (kRope) {
        // the query turned by -128 g: (q_i c + q_i' s, q_i' c - q_i s) for pair (i, i' = i + D/2)
        const float qlive = live ? 1.f : 0.f;
#pragma unroll
        for (int kh = 0; kh < KC / 2; ++kh) {
          const uint4 q1 = *(const uint4*)&s_q[live ? col : 0][32 * kh + 8 * jj];
          const uint4 q2 = *(const uint4*)&s_q[live ? col : 0][32 * (kh + KC / 2) + 8 * jj];
          const uint32_t w1[4] = {q1.x, q1.y, q1.z, q1.w}, w2[4] = {q2.x, q2.y, q2.z, q2.w};
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const float a1 = qlive * __builtin_bit_cast(
                                         float, (x & 1) ? w1[x >> 1] & 0xFFFF0000u : w1[x >> 1] << 16);
            const float a2 = qlive * __builtin_bit_cast(
                                         float, (x & 1) ? w2[x >> 1] & 0xFFFF0000u : w2[x >> 1] << 16);
            const float4 bv = bq[kh][x >> 1];
            const float cb = (x & 1) ? bv.z : bv.x, sb = (x & 1) ? bv.w : bv.y;
            const int e = 2 * (x & 3) + (x >> 2);  // operand slot of element x
            qa[kh][e] = (_Float16)__builtin_fmaf(a1, cb, a2 * sb);
            qa[kh + KC / 2][e] = (_Float16)__builtin_fmaf(a2, cb, -a1 * sb);
          }
        }
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const uint32_t sw[4] = {ps[kc].x, ps[kc].y, ps[kc].z, ps[kc].w};
          const uint32_t zw[4] = {pz[kc].x, pz[kc].y, pz[kc].z, pz[kc].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // elements j and j + 4 sit in words j / 2 and j / 2 + 2, half j % 2
            const uint32_t s0 = (j & 1) ? sw[j >> 1] & 0xFFFF0000u : sw[j >> 1] << 16;
            const uint32_t s1 = (j & 1) ? sw[2 + (j >> 1)] & 0xFFFF0000u : sw[2 + (j >> 1)] << 16;
            const uint32_t z0 = (j & 1) ? zw[j >> 1] & 0xFFFF0000u : zw[j >> 1] << 16;
            const uint32_t z1 = (j & 1) ? zw[2 + (j >> 1)] & 0xFFFF0000u : zw[2 + (j >> 1)] << 16;
            const float hs = (BITS == 4 && (j & 1)) ? 0.0625f : 1.f;
            rs[kc][j] = half2_t{(_Float16)(__builtin_bit_cast(float, s0) * hs),
                                (_Float16)(__builtin_bit_cast(float, s1) * hs)};
            rz[kc][j] = half2_t{(_Float16)__builtin_bit_cast(float, z0),
                                (_Float16)__builtin_bit_cast(float, z1)};
          }
        }
        bias = 0.f;
        thb = thq;
        nb = -mq;
        return;
      }
      float bp = 0.f;  // this lane's part of query col's bias
      const int qrow = live ? col : G;  // padding columns read the zero row
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        // channels 32 kc + 8 jj + 0..7 of query col: bf16 in channel order (one 16-byte
        // read) for the zero term, float32 in slot order (two reads) for the scaled operand
        const uint4 qv = *(const uint4*)&s_q[qrow][32 * kc + 8 * jj];
        const float4 f0 = *(const float4*)&s_qf[qrow][32 * kc + 8 * jj];
        const float4 f1 = *(const float4*)&s_qf[qrow][32 * kc + 8 * jj + 4];
        const float qs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
        const uint32_t sw[4] = {ps[kc].x, ps[kc].y, ps[kc].z, ps[kc].w};
        const uint32_t zw[4] = {pz[kc].x, pz[kc].y, pz[kc].z, pz[kc].w};
        // zero term: channel pairs (2 i, 2 i + 1) of the query and of the zeros
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bp = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[i]),
                                               __builtin_bit_cast(bf16x2_t, zw[i]), bp, false);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int x = kCodeOrder[e];  // channel 32 kc + 8 jj + x in operand slot e
          const uint32_t hs = (x & 1) ? sw[x >> 1] & 0xFFFF0000u : sw[x >> 1] << 16;
          qa[kc][e] = (_Float16)(qs[e] * __builtin_bit_cast(float, hs));
        }
      }
      bp = xor16_sum(bp);
      bp = xor32_sum(bp);
      bias = bp * (1.f / kTwo24);  // the product accumulates in units of 2^-24
      thb = thq - bias;
      nb = bias * c2s - mq;
    };
    struct Ld {
      uint32_t k[2][KW];  // key code words of the two 16-token tiles
      uint32_t v[VW];     // value code words of the channel blocks
      u32x4_t vp[2];      // bf16 value scale | zero of tokens 16 tau + 4 jj + 0..3
    };
    // Loads address a wave-uniform group base plus a constant 32-bit lane offset plus an
    // immediate for the step and tile. Past this wave's last group the look-ahead reads the
    // idle buffer instead (cached), so it costs no HBM traffic. The choice is a select of the
    // base and of the lane offset, not a branch: a branch would split the loop body and let
    // the compiler move the last uses of a slot below its reload.
    const int64_t q4p = a.q4_params;
    const uint32_t lk = col * CBY + jj * KW * 4;          // token col's key words of slice jj
    const uint32_t lv = lane * 16;                         // this lane's 16 bytes of each KB
    const uint32_t lp = 16 * jj;                           // value parameters of tokens 4 jj ..
    const uint32_t lk_d = lk & 1023;
    auto load_step = [&](Ld& f, int gi, int st) {
      const bool real = gi < n_full || (gi == n_full && st == t_step);  // wave-uniform
      const int64_t gg = group_of(gi);
      const char* kb = real ? kq + gg * kQ4Group * CBY : idle;
      const char* vb = real ? vq + gg * kQ4Group * CBY : idle;
      const char* pb = real ? vq + q4p + gg * kQ4Group * 4 : idle;
      const uint32_t ok = real ? lk : lk_d;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        // token 32 st + 16 tau + col: words KW jj .. KW jj + KW - 1 of its row
        const char* kr = kb + ok + (st * kStep + 16 * tau) * CBY;
        if constexpr (KW >= 4) {
#pragma unroll
          for (int i = 0; i < KW / 4; ++i) {
            const u32x4_t x =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kr + 16 * i));
            f.k[tau][4 * i] = x.x; f.k[tau][4 * i + 1] = x.y;
            f.k[tau][4 * i + 2] = x.z; f.k[tau][4 * i + 3] = x.w;
          }
        } else {
          const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(kr));
          f.k[tau][0] = x.x; f.k[tau][1] = x.y;
        }
        // parameters of tokens 32 st + 16 tau + 4 jj .. + 3
        f.vp[tau] = *(const u32x4_t*)(pb + lp + (st * kStep + 16 * tau) * 4);
      }
      // step st: VW / 4 contiguous KB, word w of this lane's 16 bytes in KB h is channel
      // block 4 h + w (4 bits), or channel block 2 h + w / 2, tile w % 2 (8 bits)
      const char* vr = vb + lv + st * (VW / 4) * 1024;
#pragma unroll
      for (int h = 0; h < VW / 4; ++h) {
        const u32x4_t x =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vr + h * 1024));
        f.v[4 * h] = x.x; f.v[4 * h + 1] = x.y; f.v[4 * h + 2] = x.z; f.v[4 * h + 3] = x.w;
      }
    };
    auto step = [&](const Ld& f, int st) {
      f32x4_t sacc[2];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        sacc[tau] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (kRope) {
          // token 32 st + 16 tau + col of the group: dequantize its channels in packed fp16,
          // turn pair (i, i + D/2) by its angle, feed the turned keys
          half2_t dq[KC][4];
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            uint32_t m[4];
            if constexpr (BITS == 4) {
              const uint32_t w = f.k[tau][kc], w8 = w >> 8;
              m[0] = (w & 0x000F000Fu) | 0x64006400u;
              m[1] = (w & 0x00F000F0u) | 0x64006400u;
              m[2] = (w8 & 0x000F000Fu) | 0x64006400u;
              m[3] = (w8 & 0x00F000F0u) | 0x64006400u;
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j)
                m[j] = byte_pair(f.k[tau][2 * kc], f.k[tau][2 * kc + 1], j) | 0x64006400u;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
              dq[kc][j] = __builtin_elementwise_fma(
                  __builtin_bit_cast(half2_t, m[j]) - half2_t{(_Float16)1024.f, (_Float16)1024.f},
                  rs[kc][j], rz[kc][j]);
          }
          const uint32_t* rot = &s_rot[(st * kStep + 16 * tau + col) * kRotRow + 8 * jj];
          half8_t ka[KC];
#pragma unroll
          for (int kh = 0; kh < KC / 2; ++kh) {
            // words copied out of the vectors first: hipcc 7.2 takes element 0 for every j
            // when __builtin_bit_cast is given a vector element directly
            const u32x4_t cv = *(const u32x4_t*)(rot + 32 * kh);
            const u32x4_t sv = *(const u32x4_t*)(rot + 32 * kh + 4);
            const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w}, sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const half2_t c = __builtin_bit_cast(half2_t, cw[j]);
              const half2_t sn = __builtin_bit_cast(half2_t, sw[j]);
              const half2_t k1 = dq[kh][j], k2 = dq[kh + KC / 2][j];
              const half2_t r1 = __builtin_elementwise_fma(k1, c, -(k2 * sn));
              const half2_t r2 = __builtin_elementwise_fma(k1, sn, k2 * c);
              ka[kh][2 * j] = r1.x;
              ka[kh][2 * j + 1] = r1.y;
              ka[kh + KC / 2][2 * j] = r2.x;
              ka[kh + KC / 2][2 * j + 1] = r2.y;
            }
          }
#pragma unroll
          for (int kc = 0; kc < KC; ++kc)
            sacc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[kc], qa[kc], sacc[tau], 0, 0, 0);
        } else {
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            const half8_t ka = BITS == 4 ? codes_to_f16(f.k[tau][kc])
                                         : bytes_to_f16(f.k[tau][2 * kc], f.k[tau][2 * kc + 1]);
            sacc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qa[kc], sacc[tau], 0, 0, 0);
          }
        }
      }
      // online softmax of query col over the 32 tokens: the common case compares the lane's
      // largest raw product with the threshold; only when one passes it does the wave take
      // the maxima over the 4 lanes of each column and rescale
      float lm = sacc[0][0];
#pragma unroll
      for (int i = 1; i < 4; ++i) lm = fmaxf(lm, sacc[0][i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) lm = fmaxf(lm, sacc[1][i]);
      if (__ballot(lm > thb) != 0) {  // rare
        float cm = xor16_max(lm);
        cm = xor32_max(cm);
        if (cm > thb) {
          const float mn = (cm + bias) * c2s;
          const float al = fexp2(mq - mn);
          lq *= al;
          zq *= al;
#pragma unroll
          for (int cb = 0; cb < CBK; ++cb) oacc[cb] *= al;
          mq = mn;
          thq = (mn + kTau) * inv_c2s;
          thb = thq - bias;
          nb = bias * c2s - mq;
        }
      }
      // element x of a value word is token 16 (x / 4) + 4 jj + x % 4 and sits in operand slot
      // 2 (x % 4) + x / 4, with 1/16 for the odd (high-nibble) elements
      half8_t pb;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int tau = x >> 2, i = x & 3;
        const uint32_t w = f.vp[tau][i];
        const float p = fexp2(__builtin_fmaf(sacc[tau][i], c2s, nb));
        lq += p;
        zq = __builtin_fmaf(p, __builtin_bit_cast(float, w & 0xFFFF0000u), zq);
        pb[2 * i + tau] = (_Float16)(p * __builtin_bit_cast(float, w << 16) *
                                     ((BITS == 4 && (x & 1)) ? 0.0625f : 1.f));
      }
#pragma unroll
      for (int cb = 0; cb < CBK; ++cb) {
        const half8_t va = BITS == 4 ? codes_to_f16(f.v[cb])
                                     : bytes_to_f16(f.v[2 * cb], f.v[2 * cb + 1]);
        oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, oacc[cb], 0, 0, 0);
      }
    };

    static_assert(kSteps == 4, "a group is four steps, walked by two register slots");
    // The query first, on a quiet memory system (fetched together with every wave's first
    // group, it waited behind that burst and the compute started later), then the first
    // group's loads.
    {
      const uint32_t* qw = (const uint32_t*)((const char*)a.q + ((int64_t)b * a.Hq + h0) * RB);
      for (int w = tid; w < (G + 1) * D / 2; w += kThreads)
        reinterpret_cast<uint32_t*>(&s_q[0][0])[w] = w < G * D / 2 ? qw[w] : 0u;
      if constexpr (!kRope) {
        const uint16_t* qh = (const uint16_t*)qw;
        for (int i = tid; i < (G + 1) * D; i += kThreads) {
          const int row = i / D, e = i % 8;
          const int ch = (i % D - e) + (e >> 1) + 4 * (e & 1);  // kCodeOrder[e]
          const float hs = (BITS == 4 && (e & 2)) ? 0.0625f : 1.f;  // kCodeHigh[e]
          s_qf[row][i % D] =
              row < G ? __builtin_bit_cast(float, (uint32_t)qh[row * D + ch] << 16) * hs : 0.f;
        }
      }
      if constexpr (kRope) {  // the tau16 table, copied whole
        const uint4* src = (const uint4*)a.rope_tau16;
        for (int w = tid; w < kQ4Group * kRotRow / 4; w += kThreads)
          reinterpret_cast<uint4*>(s_rot)[w] = src[w];
      }
    }
    __syncthreads();
    {
      // Two register slots of one step each, a slot refilled two steps ahead (steps 2 and 3
      // of the same group, then steps 0 and 1 of the next): 8 KB in flight per wave with 4-bit
      // codes, 16 KB with 8-bit ones. Four slots (a whole group ahead) put 35 MB of 4-bit
      // loads in flight at the start and measured 3 % slower (6 % with pre-RoPE keys).
      Ld f0, f1;
      if (n_wave > 0) {
        load_params(0);
        load_step(f0, 0, 0);
        load_step(f1, 0, 1);
      }
      for (int gi = 0; gi < n_full; ++gi) {
        fold();
        load_params(gi + 1);  // clamped past the last group
        // the barriers keep each slot's last use ahead of its reload, so the reload lands in
        // the same registers (no loop-carried copy, which would wait for the load)
        step(f0, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_step(f0, gi, 2);
        step(f1, 1);
        __builtin_amdgcn_sched_barrier(0);
        load_step(f1, gi, 3);
        step(f0, 2);
        __builtin_amdgcn_sched_barrier(0);
        load_step(f0, gi + 1, 0);
        step(f1, 3);
        __builtin_amdgcn_sched_barrier(0);
        load_step(f1, gi + 1, 1);
      }
      if (t_step >= 0) {  // the leftover step: steps 0 and 1 are in their slots, 2 and 3 load here
        fold();
        if (t_step == 0) {
          step(f0, 0);
        } else if (t_step == 1) {
          step(f1, 1);
        } else if (t_step == 2) {
          load_step(f0, n_full, 2);
          step(f0, 2);
        } else {
          load_step(f1, n_full, 3);
          step(f1, 3);
        }
      }
    }
  }
  // MFMA partial of query col: sums over the 4 lanes of the column; every channel of O^T gets
  // the column's value-zero sum
  {
    lq = xor16_sum(lq);
    lq = xor32_sum(lq);
    zq = xor16_sum(zq);
    zq = xor32_sum(zq);
    if (live) {
#pragma unroll
      for (int cb = 0; cb < CBK; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_o[kWaves + wave][col][16 * cb + 4 * jj + i] = __builtin_fmaf(oacc[cb][i], kTwo24, zq);
      if (jj == 0) {
        s_m[kWaves + wave][col] = mq;
        s_l[kWaves + wave][col] = lq;
      }
    }
  }

  // ---- bf16 rows: the residual group (its split only) or the streaming slots ---------------
  float m[G], thr[G], l[G], o[G][Geo::kE];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kMInit;
    thr[g] = kMInit;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < Geo::kE; ++e) o[g][e] = 0.f;
  }
  const int t1 = ret ? 0 : (res ? n % kQ4Group : n);
  // kRope: rows are turned at their positions in float32 and dotted with the query in
  // float32. Position of bf16 row r of this block: residual row r is 128 (n / 128) + r; a
  // streaming slot s holds s if s < S, else the latest position p <= nl with slot(p) = s,
  // nl the last position in the cache (before a fused step's token).
  [[maybe_unused]] const int str_nl = fused ? a.n[b] - 2 : a.n[b] - 1;
  [[maybe_unused]] auto pos_of = [&](int64_t r64) -> int {
    const int r = (int)r64;
    if (res) return (n / kQ4Group) * kQ4Group + r;
    return r < a.S ? r : r + a.R * ((str_nl - r) / a.R);
  };
  // (cos, sin) of the base angle 128 (p / 128) f_i of this lane's pairs i = 8 (sub mod D/16)
  // + 2 k, + 1
  [[maybe_unused]] auto load_base = [&](float4 (&bb)[4], int p) {
    const float4* bp = (const float4*)(a.rope_base + (int64_t)(p / kQ4Group) * D +
                                       16 * (sub & (D / 16 - 1)));
#pragma unroll
    for (int k = 0; k < 4; ++k) bb[k] = bp[k];
  };
  // Logits of query g against the row's key turned at p (base angles bb, the rest tk = p mod
  // 128 from the LDS table), summed over the row's LPT lanes. The partner channels of pair i
  // sit in the same lane (two chunks per lane) or in lane sub ^ D/16 of the row's lane group
  // (one chunk per lane).
  [[maybe_unused]] auto rope_logits = [&](const F& f, const float4 (&bb)[4], int tk,
                                          const QRegs<T, D, G, LPT>& q, float (&dz)[G]) {
    const uint32_t* row = &s_rot[tk * kRotRow + 8 * (sub & (D / 16 - 1))];
    // words copied out of the vectors first: hipcc 7.2 takes element 0 for every index when
    // __builtin_bit_cast is given a vector element directly
    const u32x4_t cv = *(const u32x4_t*)row, sv = *(const u32x4_t*)(row + 4);
    const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w}, sw[4] = {sv.x, sv.y, sv.z, sv.w};
    float cs[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float4 bv = bb[e >> 1];
      const float cb = (e & 1) ? bv.z : bv.x, sb = (e & 1) ? bv.w : bv.y;
      const float ct = (float)__builtin_bit_cast(half2_t, cw[e & 3])[e >> 2];
      const float st = (float)__builtin_bit_cast(half2_t, sw[e & 3])[e >> 2];
      cs[e] = __builtin_fmaf(cb, ct, -sb * st);
      sn[e] = __builtin_fmaf(sb, ct, cb * st);
    }
    auto elem = [](uint32_t w, int h) {
      return __builtin_bit_cast(float, h ? w & 0xFFFF0000u : w << 16);
    };
    float kr[kCpl][8];  // the turned key, this lane's chunks
    if constexpr (kCpl == 2) {
      const uint32_t x1[4] = {f.k[0].x, f.k[0].y, f.k[0].z, f.k[0].w};
      const uint32_t x2[4] = {f.k[1].x, f.k[1].y, f.k[1].z, f.k[1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a1 = elem(x1[e >> 1], e & 1), a2 = elem(x2[e >> 1], e & 1);
        kr[0][e] = __builtin_fmaf(a1, cs[e], -a2 * sn[e]);
        kr[1][e] = __builtin_fmaf(a1, sn[e], a2 * cs[e]);
      }
    } else {
      static_assert(kCpl == 1 && LPT == D / 8, "one chunk per lane: partner lane sub ^ D/16");
      const bool first = sub < D / 16;
      const uint32_t x[4] = {f.k[0].x, f.k[0].y, f.k[0].z, f.k[0].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t pw = (uint32_t)__shfl_xor((int)x[w], D / 16);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = 2 * w + h;
          const float xv = elem(x[w], h), pv = elem(pw, h);
          kr[0][e] = first ? __builtin_fmaf(xv, cs[e], -pv * sn[e])
                           : __builtin_fmaf(pv, sn[e], xv * cs[e]);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < kCpl; ++c) {
        const uint32_t qw[4] = {q.q[g][c].x, q.q[g][c].y, q.q[g][c].z, q.q[g][c].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(kr[c][e], elem(qw[e >> 1], e & 1), acc);
      }
      dz[g] = group_sum<LPT>(acc);
    }
  };
  if (t1 > 0 || new_row >= 0) {
    QRegs<T, D, G, LPT> q;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < kCpl; ++c) q.q[g][c] = *(const uint4*)&s_q[g][(sub + LPT * c) * 8];
    // online softmax and P V of one row given its logits
    auto update = [&](const F& f, float (&dz)[G], bool valid) {
#pragma unroll
      for (int g = 0; g < G; ++g) dz[g] = valid ? dz[g] : kNegInf;
      bool need = false;
#pragma unroll
      for (int g = 0; g < G; ++g) need |= dz[g] > thr[g];
      if (need) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (dz[g] > thr[g]) {
            const float mn = dz[g] * c2;
            const float al = fexp2(m[g] - mn);
            l[g] *= al;
#pragma unroll
            for (int e = 0; e < Geo::kE; ++e) o[g][e] *= al;
            m[g] = mn;
            thr[g] = (mn + kTau) * inv_c2;
          }
        }
      }
      float p[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        p[g] = fexp2(__builtin_fmaf(dz[g], c2, -m[g]));
        l[g] += p[g];
      }
      accumulate_pv<T, D, G, LPT>(f, p, o);
    };
    auto process = [&](const F& f, bool valid) {
      float dz[G];
#pragma unroll
      for (int g = 0; g < G; ++g) dz[g] = group_sum<LPT>(dot_partial<T, D, G, LPT>(f, q, g));
      update(f, dz, valid);
    };
    const int n_it = (t1 + kTpb - 1) / kTpb;
    auto row_of = [&](int it) -> int64_t {
      const int t = it * kTpb + wave * kTpw + grp;
      return (int64_t)r0 + (t < t1 ? t : t1 - 1);
    };
    auto valid_at = [&](int it) {
      const int t = it * kTpb + wave * kTpw + grp;
      return t < t1 && r0 + t != skip;
    };
    if (t1 > 0) {
      // kBfStages row fragments in flight: this path runs after the MFMA loop, whose
      // registers are free by then, and its blocks (a streaming head's S + R slots over 4
      // waves) wait on memory once per kBfStages iterations
      F g[kBfStages];
      [[maybe_unused]] float4 gb[kRope ? kBfStages : 1][4];  // kRope: each row's base angles
#pragma unroll
      for (int st = 0; st < kBfStages; ++st) {
        load_frag<T, D, LPT>(g[st], kbase, vbase, row_of(st), sub);
        if constexpr (kRope) load_base(gb[st], pos_of(row_of(st)));
      }
      for (int it = 0; it < n_it; it += kBfStages) {
#pragma unroll
        for (int st = 0; st < kBfStages; ++st) {
          if constexpr (kRope) {
            float dz[G];
            rope_logits(g[st], gb[st], pos_of(row_of(it + st)) % kQ4Group, q, dz);
            update(g[st], dz, valid_at(it + st));
            load_base(gb[st], pos_of(row_of(it + st + kBfStages)));
          } else {
            process(g[st], valid_at(it + st));
          }
          load_frag<T, D, LPT>(g[st], kbase, vbase, row_of(it + st + kBfStages), sub);
        }
      }
    }
    // fused step: the new token from the input, then its store (residual row or ring slot)
    if (new_row >= 0) {
      const char* nk = (const char*)a.new_k + ((int64_t)b * a.Hkv + j) * RB;
      const char* nv = (const char*)a.new_v + ((int64_t)b * a.Hkv + j) * RB;
      F f;
      load_frag<T, D, LPT>(f, nk, nv, 0, sub);
      if constexpr (kRope) {
        const int pnew = a.n[b] - 1;
        float4 bb[4];
        load_base(bb, pnew);
        float dz[G];
        rope_logits(f, bb, pnew % kQ4Group, q, dz);
        update(f, dz, wave == 0 && grp == 0);
      } else {
        process(f, wave == 0 && grp == 0);
      }
      if (wave == 0) {
        constexpr int kRowChunks = RB / 16;
        for (int c = lane; c < 2 * kRowChunks; c += 64) {
          const bool is_v = c >= kRowChunks;
          const int cc = is_v ? c - kRowChunks : c;
          const uint4 x = *(const uint4*)((is_v ? nv : nk) + cc * 16);
          *(uint4*)(const_cast<char*>(is_v ? vbase : kbase) + (int64_t)new_row * RB + cc * 16) = x;
        }
        if (j == 0 && lane == 0) {  // one block per sequence updates the tables
          const int pnew = a.n[b] - 1;
          const int SR = a.S + a.R;
          a.slot_pos[(int64_t)b * SR + (pnew < a.S ? pnew : a.S + (pnew - a.S) % a.R)] = pnew;
          a.seq_len[b] = a.n[b];
        }
      }
    }
  }
  // lane groups of this wave -> s_*[wave]; a block with no bf16 rows (nearly every retrieval
  // block) skips the reduction and merges its MFMA partials alone
  const bool bf16_rows = t1 > 0 || new_row >= 0;  // block-uniform
#pragma unroll
  for (int g = 0; g < G && bf16_rows; ++g) {
    float mx = m[g];
    if constexpr (LPT == 8) mx = fmaxf(mx, dpp<0x128>(mx));
    mx = xor16_max(mx);
    mx = xor32_max(mx);
    const float sc = fexp2(m[g] - mx);
    float lg = l[g] * sc;
    if constexpr (LPT == 8) lg += dpp<0x128>(lg);
    lg = xor16_sum(lg);
    lg = xor32_sum(lg);
#pragma unroll
    for (int e = 0; e < Geo::kE; ++e) {
      float x = o[g][e] * sc;
      if constexpr (LPT == 8) x += dpp<0x128>(x);
      x = xor16_sum(x);
      x = xor32_sum(x);
      o[g][e] = x;
    }
    if (grp == 0) {
#pragma unroll
      for (int c = 0; c < kCpl; ++c)
#pragma unroll
        for (int e = 0; e < Geo::kEpc; ++e)
          s_o[wave][g][Geo::elem_d(sub, c, e)] = o[g][c * Geo::kEpc + e];
      if (sub == 0) {
        s_m[wave][g] = mx;
        s_l[wave][g] = lg;
      }
    }
  }
  __syncthreads();

  // ---- merge the 2 x 4 partials; finish or write this split's partial ---------------------
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, d = idx % D;
    const int w0 = bf16_rows ? 0 : kWaves;
    float M = kMInit;
    for (int w = w0; w < 2 * kWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float L = 0.f, O = 0.f;
    for (int w = w0; w < 2 * kWaves; ++w) {
      const float sc = fexp2(s_m[w][g] - M);
      L += s_l[w][g] * sc;
      O += s_o[w][g][d] * sc;
    }
    const int h = h0 + g;
    if (nparts == 1) {
      const int64_t oi = ((int64_t)b * a.Hq + h) * D + d;
      store_out<T>(a.out, oi, O / L, a.out_f32);
      if (d == 0 && a.lse) a.lse[(int64_t)b * a.Hq + h] = (M + __builtin_log2f(L)) * kLn2;
    } else {
      const int64_t pi = ((int64_t)b * a.Hq + h) * a.max_splits + split;
      a.part_o[pi * D + d] = O;
      if (d == 0) {
        a.part_ml[pi * 2 + 0] = M;
        a.part_ml[pi * 2 + 1] = L;
      }
    }
  }
}

// Merge of the context splits of one query head (sequence b, head h) over 64
// output columns: M = max_s m_s, L = sum_s l_s exp2(m_s - M), out = sum_s o_s exp2(m_s - M)
// / L, lse = (M + log2 L) ln 2. Each of the 8 waves takes every 8th split with an online
// log-sum-exp, issuing the loads of kMergeBatch splits together, and the waves combine
// through LDS; with up to 128 splits every wave waits on memory once. Empty splits
// (m = kMInit, l = 0) weigh zero. A separate launch: the partials need no fences.
// Its arguments are 14 dwords of leading scalars, all preloaded into SGPRs (16 user SGPRs,
// two of them the argument pointer; the build asks for the preload in this file), and the
// grid is (G x 64-column slices, KV head, sequence), so a block reaches its first partial
// load with no memory access and no division. ret_mask bit j marks KV head j as retrieval (it
// merges ret_parts partials, a streaming head str_parts); blocks of heads with a single part
// return at once.
constexpr int kMergeWaves = 8;
constexpr int kMergeThreads = kMergeWaves * 64;
constexpr int kMergeBatch = 16;

template <typename T, int D, int G, bool OutF32>
__global__ void __launch_bounds__(kMergeThreads)
    merge_kernel(uint64_t ret_mask, int32_t ret_parts, int32_t str_parts, int32_t Hq,
                 int32_t max_splits, const float* part_o, const float* part_ml, void* out,
                 float* lse) {
  __shared__ float s_m[kMergeWaves], s_l[kMergeWaves];
  __shared__ float s_o[kMergeWaves][64];
  constexpr int kSlices = D / 64;
  const int j = blockIdx.y;
  const int nsplit = ((ret_mask >> j) & 1) ? ret_parts : str_parts;
  if (nsplit <= 1) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x / kSlices, slice = blockIdx.x % kSlices;
  const int b = blockIdx.z;
  const int h = j * G + g;
  const int64_t p0 = ((int64_t)b * Hq + h) * max_splits;
  const int d = slice * 64 + lane;
  const float* po = part_o + p0 * D + d;
  const float2* pml = reinterpret_cast<const float2*>(part_ml) + p0;

  float M = kMInit, L = 0.f, O = 0.f;
  for (int s0 = wave; s0 < nsplit; s0 += kMergeWaves * kMergeBatch) {
    float2 ml[kMergeBatch];
    float ov[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int sp = s0 + kMergeWaves * i;
      const int spc = sp < nsplit ? sp : nsplit - 1;  // clamped; the extra ones weigh 0
      ml[i] = pml[spc];
      ov[i] = po[(int64_t)spc * D];
    }
    float bm = M;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
      if (s0 + kMergeWaves * i < nsplit) bm = fmaxf(bm, ml[i].x);
    const float sc = fexp2(M - bm);
    L *= sc;
    O *= sc;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const float w = (s0 + kMergeWaves * i < nsplit) ? fexp2(ml[i].x - bm) : 0.f;
      L = __builtin_fmaf(w, ml[i].y, L);
      O = __builtin_fmaf(w, ov[i], O);
    }
    M = bm;
  }
  s_o[wave][lane] = O;
  if (lane == 0) {
    s_m[wave] = M;
    s_l[wave] = L;
  }
  __syncthreads();
  if (wave != 0) return;
  float Mt = kMInit;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) Mt = fmaxf(Mt, s_m[w]);
  float Lt = 0.f, Ot = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    const float sc = fexp2(s_m[w] - Mt);
    Lt = __builtin_fmaf(sc, s_l[w], Lt);
    Ot = __builtin_fmaf(sc, s_o[w][lane], Ot);
  }
  store_out<T>(out, ((int64_t)b * Hq + h) * D + d, Ot / Lt, OutF32);
  if (slice == 0 && lane == 0 && lse) lse[(int64_t)b * Hq + h] = (Mt + __builtin_log2f(Lt)) * kLn2;
}

template <typename T, int D, int G>
struct Variant {
  static constexpr int LPT = lanes_per_token<T, D, G>();
  static constexpr int NS = stages<T, D, G>();

  // Decode blocks that fit on the device at once (of the 4-bit kernel when q4, its pre-RoPE
  // form when rope), counting at most max_per_cu per CU; the occupancy is queried once per
  // process. The host sizes one round of splits from it (two blocks per CU for a batch, one
  // for a single sequence).
  static int resident_blocks(int qbits, bool rope, int max_per_cu) {
    static int cus_cached = 0, per_cu_cached[5] = {0, 0, 0, 0, 0};
    const int kind = qbits ? (qbits == 8 ? 3 : 1) + (rope ? 1 : 0) : 0;
    if (!per_cu_cached[kind]) {
      const void* fn = reinterpret_cast<const void*>(&decode_kernel<T, D, G, LPT, NS>);
      if constexpr (sizeof(T) == 2) {
        if (kind == 1) fn = reinterpret_cast<const void*>(&decode_q4_kernel<D, G, LPT, 4, false, 4>);
        if (kind == 2) fn = reinterpret_cast<const void*>(&decode_q4_kernel<D, G, LPT, 4, true, 4>);
        if (kind == 3) fn = reinterpret_cast<const void*>(&decode_q4_kernel<D, G, LPT, 4, false, 8>);
        if (kind == 4) fn = reinterpret_cast<const void*>(&decode_q4_kernel<D, G, LPT, 4, true, 8>);
      }
      int dev = 0, cus = 0, per_cu = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess ||
          cus <= 0 || per_cu <= 0) {
        (void)hipGetLastError();
        return 512;
      }
      cus_cached = cus;
      per_cu_cached[kind] = per_cu;
    }
    const int per_cu = per_cu_cached[kind];
    return cus_cached * (per_cu < max_per_cu ? per_cu : max_per_cu);
  }

  static int launch(const DecodeArgs& a, void* stream, const KernelMarks& marks) {
    const int64_t blocks = (int64_t)a.B * a.Hr * a.nsplit + (a.qbits ? (int64_t)a.B * a.Hr : 0) +
                           (int64_t)a.B * a.Hs * a.nss;
    if (marks.begin) (void)hipEventRecord((hipEvent_t)marks.begin, (hipStream_t)stream);
    if constexpr (sizeof(T) == 2) {
      const dim3 grid((unsigned)blocks), block(kThreads);
      hipStream_t st = (hipStream_t)stream;
      const int fused = a.new_k != nullptr ? 1 : 0;
      if (a.qbits == 4 && a.rope_base)
        hipLaunchKernelGGL((decode_q4_kernel<D, G, LPT, 4, true, 4>), grid, block, 0, st,
                           a.nsplit, a.Hr, a.Hs, a.B, a.nss, fused, a);
      else if (a.qbits == 4)
        hipLaunchKernelGGL((decode_q4_kernel<D, G, LPT, 4, false, 4>), grid, block, 0, st,
                           a.nsplit, a.Hr, a.Hs, a.B, a.nss, fused, a);
      else if (a.qbits == 8 && a.rope_base)
        hipLaunchKernelGGL((decode_q4_kernel<D, G, LPT, 4, true, 8>), grid, block, 0, st,
                           a.nsplit, a.Hr, a.Hs, a.B, a.nss, fused, a);
      else if (a.qbits == 8)
        hipLaunchKernelGGL((decode_q4_kernel<D, G, LPT, 4, false, 8>), grid, block, 0, st,
                           a.nsplit, a.Hr, a.Hs, a.B, a.nss, fused, a);
      else if (a.qbits)
        return -1;
      else
        hipLaunchKernelGGL((decode_kernel<T, D, G, LPT, NS>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, (hipStream_t)stream, a.nsplit, a.Hr, a.Hs, a.B, a.nss,
                           a.new_k != nullptr ? 1 : 0, a);
    } else {
      if (a.qbits) return -1;
      hipLaunchKernelGGL((decode_kernel<T, D, G, LPT, NS>), dim3((unsigned)blocks),
                         dim3(kThreads), 0, (hipStream_t)stream, a.nsplit, a.Hr, a.Hs, a.B, a.nss,
                           a.new_k != nullptr ? 1 : 0, a);
    }
    if (marks.end) (void)hipEventRecord((hipEvent_t)marks.end, (hipStream_t)stream);
    // split heads (retrieval heads when nsplit > 1, streaming heads when nss > 1)
    const int ret_parts = a.nsplit + (a.qbits ? 1 : 0);
    if ((ret_parts > 1 && a.Hr > 0) || (a.nss > 1 && a.Hs > 0)) {
      uint64_t ret_mask = 0;
      for (int r = 0; r < a.Hr; ++r) ret_mask |= 1ull << a.ret_kv[r];
      const dim3 grid(G * (D / 64), a.Hkv, a.B);
      if (a.out_f32)
        hipLaunchKernelGGL((merge_kernel<T, D, G, true>), grid, dim3(kMergeThreads), 0,
                           (hipStream_t)stream, ret_mask, ret_parts, a.nss, a.Hq, a.max_splits,
                           (const float*)a.part_o, (const float*)a.part_ml, a.out, a.lse);
      else
        hipLaunchKernelGGL((merge_kernel<T, D, G, false>), grid, dim3(kMergeThreads), 0,
                           (hipStream_t)stream, ret_mask, ret_parts, a.nss, a.Hq, a.max_splits,
                           (const float*)a.part_o, (const float*)a.part_ml, a.out, a.lse);
    }
    return (int)hipGetLastError();
  }
};

template <typename T, int D, int G>
int run(bool query, const DecodeArgs* a, void* stream, const KernelMarks* marks) {
  // a query reads a->qbits, whether a->rope_base is set and the per-CU cap in a->nsplit
  return query ? Variant<T, D, G>::resident_blocks(a->qbits, a->rope_base != nullptr,
                                                   a->nsplit)
               : Variant<T, D, G>::launch(*a, stream, *marks);
}

template <typename T, int D>
int dispatch_g(int group, bool query, const DecodeArgs* a, void* stream, const KernelMarks* m) {
  switch (group) {
    case 1: return run<T, D, 1>(query, a, stream, m);
    case 2: return run<T, D, 2>(query, a, stream, m);
    case 4: return run<T, D, 4>(query, a, stream, m);
    case 8: return run<T, D, 8>(query, a, stream, m);
  }
  return -1;
}

int dispatch(int dtype, int head_dim, int group, bool query, const DecodeArgs* a,
             void* stream, const KernelMarks* m) {
  if (dtype == DUO_BF16) {
    if (head_dim == 128) return dispatch_g<uint16_t, 128>(group, query, a, stream, m);
    if (head_dim == 64) return dispatch_g<uint16_t, 64>(group, query, a, stream, m);
  } else {
    if (head_dim == 128) return dispatch_g<float, 128>(group, query, a, stream, m);
    if (head_dim == 64) return dispatch_g<float, 64>(group, query, a, stream, m);
  }
  return -1;
}

}  // namespace

int launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group, void* stream,
                  const KernelMarks& marks) {
  return dispatch(dtype, head_dim, group, false, &a, stream, &marks);
}

// Split-K partials of duo_attn_decode_noalloc: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends. On the host `scratch` names a stand-in,
// not the device copy, so host code never passes it to a kernel: its device address is looked
// up once per device with hipGetSymbolAddress (with that device current) and kept here.
static __device__ __align__(256) char scratch[kScratchBytes];

int static_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t rc = hipGetDevice(&dev);
  if (rc != hipSuccess) return (int)rc;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (rc != hipSuccess) return (int)rc;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int decode_resident_blocks(int dtype, int head_dim, int group, int qbits, bool rope,
                           int max_per_cu) {
  static const float marker = 0.f;
  DecodeArgs probe;  // only qbits, rope_base (null or not) and nsplit (the per-CU cap) are read
  std::memset(&probe, 0, sizeof(probe));
  probe.qbits = qbits;
  probe.rope_base = rope ? &marker : nullptr;
  probe.nsplit = max_per_cu;
  return dispatch(dtype, head_dim, group, true, &probe, nullptr, nullptr);
}

}  // namespace duo
