// Split-K flash-decode over a head-partitioned KV cache, for gfx950 (wave64).
//
// One work item is (sequence b, KV head j, context split). Retrieval heads attend over rows
// [0, n) of their full cache, cut into `nsplit` splits; a streaming head attends over its
// min(n, S+R) valid slots in one item, which after the append hold exactly the sinks and the
// last R tokens (explainer, "Decoding Procedure", steps 2-4). Row order inside a head does
// not matter to a softmax, so the ring order of the streaming slots needs no unrolling.
//
// Inside a block of 4 waves, every wave streams groups of 64/LPT tokens: LPT lanes (8 or
// 16) share one token row (each lane owns D/LPT elements of it) and every lane keeps the
// running state of all G query heads of the GQA group, so one load of each K/V row serves the whole group without
// repeating KV heads (OpenReview thread, "GQA Compatibility"). Logits are reduced over the
// LPT lanes with DPP, bf16 dot products use v_dot2_f32_bf16 with fp32 accumulation, and the
// softmax is online in the log2 domain with a lazy rescale: the running maximum of a lane
// group is only moved when a logit exceeds it by more than kTau, which keeps every weight
// below 2^kTau and leaves the quotient out/l exact. At the end the lane groups of a wave are
// merged with lane shuffles, the waves through LDS, and the splits of one (b, j) by the last
// block to finish (atomic ticket), with the log-sum-exp weights exp2(m_i - m) .
#include <hip/hip_runtime.h>

#include "duo_internal.h"

namespace duo {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 3;       // register slots of token groups per wave
constexpr float kTau = 8.0f;     // lazy-rescale threshold (log2 units)
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

template <typename T, int D, int LPT>
__device__ __forceinline__ void load_frag(Frag<T, D, LPT>& f, const char* kbase,
                                          const char* vbase, int64_t row, int sub) {
  constexpr int RB = D * (int)sizeof(T);
#pragma unroll
  for (int c = 0; c < RowGeom<T, D, LPT>::kCpl; ++c) {
    f.k[c] = *(const uint4*)(kbase + row * RB + (sub + LPT * c) * 16);
    f.v[c] = *(const uint4*)(vbase + row * RB + (sub + LPT * c) * 16);
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

// Lanes per token row: 8 unless the per-lane state of all G heads would not fit the
// register budget of two waves per SIMD, then 16 (halves the elements each lane owns).
template <typename T, int D, int G>
constexpr int lanes_per_token() {
  constexpr int chunks = D * (int)sizeof(T) / 16;
  constexpr int e8 = D / 8;
  constexpr int words8 =
      G * e8 + G * e8 * (int)sizeof(T) / 4 + kStages * 2 * (chunks / 8) * 4;
  return (words8 > 200 && chunks >= 16) ? 16 : 8;
}

template <typename T, int D, int G, int LPT>
__global__ void __launch_bounds__(kThreads, 2) decode_kernel(DecodeArgs a) {
  using Geo = RowGeom<T, D, LPT>;
  constexpr int kTpw = 64 / LPT;  // tokens per wave per step
  constexpr int E = Geo::kE;
  constexpr int RB = D * (int)sizeof(T);

  __shared__ float s_o[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, grp = lane / LPT, sub = lane % LPT;

  // ---- work item -------------------------------------------------------------------------
  const int64_t n_ret_items = (int64_t)a.B * a.Hr * a.nsplit;
  int b, j, split, nsplit;
  int64_t head_row0;  // first row of this head in its cache
  const char* kbase;
  const char* vbase;
  int t0, t1;
  if ((int64_t)blockIdx.x < n_ret_items) {
    const int64_t i = blockIdx.x;
    split = (int)(i % a.nsplit);
    const int r = (int)((i / a.nsplit) % a.Hr);
    b = (int)(i / ((int64_t)a.nsplit * a.Hr));
    j = a.ret_kv[r];
    nsplit = a.nsplit;
    const int n = a.seq_len[b];
    constexpr int kQuant = kWaves * kTpw;
    int chunk = (n + nsplit - 1) / nsplit;
    chunk = (chunk + kQuant - 1) / kQuant * kQuant;
    t0 = split * chunk;
    t1 = min(n, t0 + chunk);
    head_row0 = ((int64_t)b * a.Hr + r) * a.cap;
    kbase = (const char*)a.full_k;
    vbase = (const char*)a.full_v;
  } else {
    const int64_t i = blockIdx.x - n_ret_items;
    const int s = (int)(i % a.Hs);
    b = (int)(i / a.Hs);
    j = a.str_kv[s];
    split = 0;
    nsplit = 1;
    const int n = a.seq_len[b];
    t0 = 0;
    t1 = min(n, a.S + a.R);
    head_row0 = ((int64_t)b * a.Hs + s) * (a.S + a.R);
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

  float m[G], l[G], o[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[g][e] = 0.f;
  }

  // ---- main loop: token groups of 8, interleaved over the waves, prefetched ---------------
  if (t1 > t0) {
    const int n_it = (t1 - t0 + kWaves * kTpw - 1) / (kWaves * kTpw);
    auto row_of = [&](int it) -> int64_t {
      int t = t0 + (it * kWaves + wave) * kTpw + grp;
      return (int64_t)(t < t1 ? t : t1 - 1);  // clamped: always inside this head's rows
    };
    // kStages register slots rotate: slot s is consumed, then refilled with the group
    // kStages steps ahead, so kStages - 1 groups stay in flight while one is processed.
    // Loads are unconditional (rows past the end are clamped to the item's last row), which
    // keeps the compiler's wait counts exact across the loop back-edge.
    Frag<T, D, LPT> buf[kStages];
#pragma unroll
    for (int s = 0; s < kStages; ++s) load_frag<T, D, LPT>(buf[s], kbase, vbase, row_of(s), sub);

    for (int it = 0; it < n_it; it += kStages) {
#pragma unroll
      for (int s = 0; s < kStages; ++s) {
        const int cur = it + s;
        const bool valid = t0 + (cur * kWaves + wave) * kTpw + grp < t1;
        float z[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          z[g] = group_sum<LPT>(dot_partial<T, D, G, LPT>(buf[s], q, g)) * a.scale_log2;
          if (!valid) z[g] = kNegInf;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (z[g] > m[g] + kTau) {  // new running maximum for this lane group
            const float al = fexp2(m[g] - z[g]);
            l[g] *= al;
#pragma unroll
            for (int e = 0; e < E; ++e) o[g][e] *= al;
            m[g] = z[g];
          }
        }
        float p[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          p[g] = valid ? fexp2(z[g] - m[g]) : 0.f;
          l[g] += p[g];
        }
        accumulate_pv<T, D, G, LPT>(buf[s], p, o);
        load_frag<T, D, LPT>(buf[s], kbase, vbase, row_of(cur + kStages), sub);
      }
    }
  }

  // ---- merge the lane groups of this wave ------------------------------------------------
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = m[g];
    if constexpr (LPT == 8) mx = fmaxf(mx, dpp<0x128>(mx));  // row_ror:8 -> lane ^ 8
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float sc = (m[g] == kNegInf) ? 0.f : fexp2(m[g] - mx);
    float lg = l[g] * sc;
    if constexpr (LPT == 8) lg += dpp<0x128>(lg);
    lg += __shfl_xor(lg, 16);
    lg += __shfl_xor(lg, 32);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float x = o[g][e] * sc;
      if constexpr (LPT == 8) x += dpp<0x128>(x);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
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
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = (s_m[w][g] == kNegInf) ? 0.f : fexp2(s_m[w][g] - M);
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
  if (nsplit == 1) return;

  // ---- last block of (b, j) merges the splits ----------------------------------------------
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned ticket = atomicAdd(&a.counters[(int64_t)b * a.Hkv + j], 1u);
    s_last = (ticket == (unsigned)(nsplit - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, d = idx % D;
    const int h = h0 + g;
    const int64_t p0 = ((int64_t)b * a.Hq + h) * a.max_splits;
    float M = kNegInf;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, a.part_ml[(p0 + s) * 2]);
    float L = 0.f, O = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = a.part_ml[(p0 + s) * 2];
      const float sc = (ms == kNegInf) ? 0.f : fexp2(ms - M);
      L += a.part_ml[(p0 + s) * 2 + 1] * sc;
      O += a.part_o[(p0 + s) * D + d] * sc;
    }
    const int64_t oi = ((int64_t)b * a.Hq + h) * D + d;
    store_out<T>(a.out, oi, O / L, a.out_f32);
    if (d == 0 && a.lse) a.lse[(int64_t)b * a.Hq + h] = (M + __builtin_log2f(L)) * kLn2;
  }
  if (tid == 0) atomicExch(&a.counters[(int64_t)b * a.Hkv + j], 0u);
}

template <typename T, int D, int G>
int launch_t(const DecodeArgs& a, void* stream) {
  const int64_t blocks = (int64_t)a.B * a.Hr * a.nsplit + (int64_t)a.B * a.Hs;
  constexpr int LPT = lanes_per_token<T, D, G>();
  hipLaunchKernelGGL((decode_kernel<T, D, G, LPT>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

template <typename T, int D>
int launch_g(const DecodeArgs& a, int group, void* stream) {
  switch (group) {
    case 1: return launch_t<T, D, 1>(a, stream);
    case 2: return launch_t<T, D, 2>(a, stream);
    case 4: return launch_t<T, D, 4>(a, stream);
    case 8: return launch_t<T, D, 8>(a, stream);
  }
  return -1;
}

}  // namespace

int launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group, void* stream) {
  if (dtype == DUO_BF16) {
    if (head_dim == 128) return launch_g<uint16_t, 128>(a, group, stream);
    if (head_dim == 64) return launch_g<uint16_t, 64>(a, group, stream);
  } else {
    if (head_dim == 128) return launch_g<float, 128>(a, group, stream);
    if (head_dim == 64) return launch_g<float, 64>(a, group, stream);
  }
  return -1;
}

}  // namespace duo
