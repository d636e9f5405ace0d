// Append into 4-bit full caches (explainer, "Combination with Quantization": the retrieval
// heads' full caches in 4 bits). Keys are quantized per channel over aligned groups of
// kQ4Group tokens, values per token, both only when their group is complete, the codes
// stored in the operand layouts of the decode kernel (below). Until a group is complete the
// group's tokens wait in a bf16 residual block (row t % kQ4Group). Parameters of a block with
// minimum mn and maximum mx: scale = bf16((mx - mn) / 15) and zero = bf16(mn), stored; the code
// of x is rint((x - zero) / scale) clamped to 0..15 (0 when scale is 0), in IEEE float32
// against the stored values, so the decision is reproducible.
//
// Blocks per (sequence, retrieval head): block 0 is the edge block. It completes the first
// group if that group already had residual rows (reading them), then, after a barrier,
// writes the new incomplete tail into the residual. Blocks 1.. each quantize one complete
// group whose rows all come from the input. Only the edge block touches the residual, so its
// barrier orders every read of the residual before every write.
#include <hip/hip_runtime.h>

#include "duo_internal.h"

namespace duo {
namespace {

constexpr int kThreads = 256;
constexpr int kG = kQ4Group;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// float32 -> bfloat16 bits, round to nearest even (the stored scale and zero)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint32_t code_of(float x, float mn, float scale) {
  if (scale == 0.f) return 0u;
  const float r = __builtin_rintf((x - mn) / scale);
  return (uint32_t)fminf(fmaxf(r, 0.f), 15.f);
}

// Codes are stored in the operand layouts of the decode kernel's matrix products. A code
// word holds 8 codes, element e in bits 4e .. 4e + 3.
//   Keys: per token row, D / 8 words; the word in slot KC j + kc (KC = D / 32) holds channels
//         32 kc + 8 j .. + 7, so the KC words one lane needs for a token are contiguous.
//   Values: per group, word ((s (D / 64) + h) 64 + l) 4 + w, with l = 16 j + (c % 16) and
//         c / 16 = 4 h + w, holds channel c; its element e is token 32 s + 16 (e / 4) + 4 j +
//         e % 4 (the tokens whose logits lane l of the transposed logit tile holds). A wave's
//         value load for step s reads 1 KB contiguous per h.
static_assert(kG == 128, "four 32-token steps per group");

// Quantize the group staged in s (rows 0..kG-1, bf16) as keys: per channel over the rows.
// codes: the group's first code row; params: bf16 [2][D] (scale row, zero row); sk: the
// stored values (as float) in LDS for the code pass, which decides against them.
template <int D>
__device__ void quantize_keys(const uint16_t (*s)[D], uint8_t* codes, uint16_t* params,
                              float* sk) {
  const int c = threadIdx.x;
  if (c < D) {
    float mn = bf16_to_f32(s[0][c]), mx = mn;
    for (int r = 1; r < kG; ++r) {
      const float x = bf16_to_f32(s[r][c]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    const uint16_t sb = f32_to_bf16_bits((mx - mn) / 15.f), zb = f32_to_bf16_bits(mn);
    params[c] = sb;
    params[D + c] = zb;
    sk[c] = bf16_to_f32(sb);
    sk[D + c] = bf16_to_f32(zb);
  }
  __syncthreads();
  constexpr int KC = D / 32, W = D / 8;
  uint32_t* cw = (uint32_t*)codes;
  for (int w = threadIdx.x; w < kG * W; w += kThreads) {
    const int r = w / W, slot = w % W;
    const int c0 = 32 * (slot % KC) + 8 * (slot / KC);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      word |= code_of(bf16_to_f32(s[r][c0 + e]), sk[D + c0 + e], sk[c0 + e]) << (4 * e);
    cw[(int64_t)r * W + slot] = word;
  }
}

// Quantize the staged group as values: per token over the channels (one wave per token for
// the minimum and maximum). params: one word per token of the group, bf16 scale in the low
// half and bf16 zero in the high half; sp: the stored values (as float) in LDS.
template <int D>
__device__ void quantize_values(const uint16_t (*s)[D], uint8_t* codes, uint32_t* params,
                                float* sp) {
  constexpr int kPer = D / 64;  // channels per lane: lane, lane + 64
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = wave; r < kG; r += kThreads / 64) {
    float x[kPer];
    float mn, mx;
#pragma unroll
    for (int u = 0; u < kPer; ++u) x[u] = bf16_to_f32(s[r][lane + 64 * u]);
    mn = x[0];
    mx = x[0];
#pragma unroll
    for (int u = 1; u < kPer; ++u) {
      mn = fminf(mn, x[u]);
      mx = fmaxf(mx, x[u]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, off));
      mx = fmaxf(mx, __shfl_xor(mx, off));
    }
    const uint16_t sb = f32_to_bf16_bits((mx - mn) / 15.f), zb = f32_to_bf16_bits(mn);
    if (lane == 0) {
      params[r] = (uint32_t)sb | ((uint32_t)zb << 16);
      sp[2 * r] = bf16_to_f32(sb);
      sp[2 * r + 1] = bf16_to_f32(zb);
    }
  }
  __syncthreads();
  constexpr int kHalves = D / 64;  // 16-byte loads per lane and step
  uint32_t* cw = (uint32_t*)codes;
  for (int w = threadIdx.x; w < D * kG / 8; w += kThreads) {
    const int l = (w >> 2) & 63, x = w >> 8;
    const int h = x % kHalves, st = x / kHalves, j = l >> 4;
    const int c = 16 * (4 * h + (w & 3)) + (l & 15), t0 = 32 * st + 4 * j;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = t0 + 16 * (e >> 2) + (e & 3);
      word |= code_of(bf16_to_f32(s[t][c]), sp[2 * t + 1], sp[2 * t]) << (4 * e);
    }
    cw[w] = word;
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads) kv4_append_kernel(AppendArgs a) {
  __shared__ uint16_t s[kG][D];
  __shared__ float sp[kG > D ? 2 * kG : 2 * D];  // parameters of the group in LDS
  constexpr int kRowWords = D / 2;  // 32-bit words of a bf16 row
  const int per_head = 1 + a.q4_mid;
  const int unit = blockIdx.x % per_head;
  const int r_cls = (blockIdx.x / per_head) % a.Hr;
  const int bi = blockIdx.x / (per_head * a.Hr);
  const int b = a.b0 + bi;
  const int j = a.ret_kv[r_cls];
  const int n0 = a.n_old[bi], n1 = n0 + a.m;
  const int g_first = n0 / kG;
  const bool has_old = (n0 % kG) != 0;
  const int g_complete_end = n1 / kG;  // groups [.., g_complete_end) are complete after
  const int64_t head = ((int64_t)b * a.Hr + r_cls) * a.q4_stride;

  // group g staged from the residual (rows below n0 % kG when it is g_first) and the input
  auto stage = [&](int g, bool is_v) {
    const uint32_t* res = (const uint32_t*)((const char*)(is_v ? a.full_v : a.full_k) + head +
                                            a.q4_resid);
    const uint32_t* in = (const uint32_t*)(is_v ? a.v : a.k);
    const int old_rows = (g == g_first) ? n0 % kG : 0;
    for (int w = threadIdx.x; w < kG * kRowWords; w += kThreads) {
      const int r = w / kRowWords, c = w % kRowWords;
      uint32_t x;
      if (r < old_rows) {
        x = res[(int64_t)r * kRowWords + c];
      } else {
        const int i = g * kG + r - n0;  // input row of token g * kG + r
        x = in[(((int64_t)bi * a.m + i) * a.Hkv + j) * kRowWords + c];
      }
      reinterpret_cast<uint32_t*>(&s[r][0])[c] = x;
    }
  };
  auto quantize = [&](int g) {
    for (int is_v = 0; is_v < 2; ++is_v) {
      stage(g, is_v != 0);
      __syncthreads();
      char* base = (char*)(is_v ? a.full_v : a.full_k) + head;
      uint8_t* codes = (uint8_t*)base + (int64_t)g * kG * (D / 2);
      if (is_v)
        quantize_values<D>(s, codes, (uint32_t*)(base + a.q4_params) + (int64_t)g * kG, sp);
      else
        quantize_keys<D>(s, codes, (uint16_t*)(base + a.q4_params) + (int64_t)g * 2 * D, sp);
      __syncthreads();
    }
  };

  if (unit == 0) {
    if (has_old && g_first < g_complete_end) quantize(g_first);  // reads the residual
    __syncthreads();
    if (n1 % kG != 0) {  // the incomplete tail into the residual
      const int t0 = max(n0, g_complete_end * kG);
      const int rows = n1 - t0;
      for (int w = threadIdx.x; w < 2 * rows * kRowWords; w += kThreads) {
        const int is_v = w >= rows * kRowWords;
        const int ww = is_v ? w - rows * kRowWords : w;
        const int t = t0 + ww / kRowWords, c = ww % kRowWords;
        const uint32_t* in = (const uint32_t*)(is_v ? a.v : a.k);
        uint32_t* res = (uint32_t*)((char*)(is_v ? a.full_v : a.full_k) + head + a.q4_resid);
        res[(int64_t)(t % kG) * kRowWords + c] =
            in[(((int64_t)bi * a.m + (t - n0)) * a.Hkv + j) * kRowWords + c];
      }
    }
    return;
  }
  const int g = (has_old ? g_first + 1 : g_first) + unit - 1;
  if (g >= g_complete_end) return;
  quantize(g);
}

}  // namespace

int launch_append_kv4(const AppendArgs& a, int head_dim, void* stream) {
  const int64_t blocks = (int64_t)a.nb * a.Hr * (1 + a.q4_mid);
  if (blocks == 0) return 0;
  if (head_dim == 128)
    hipLaunchKernelGGL(kv4_append_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(kv4_append_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, a);
  else
    return -1;
  return (int)hipGetLastError();
}

}  // namespace duo
