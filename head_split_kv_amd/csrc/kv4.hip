// Append into 4-bit or 8-bit full caches (explainer, "Combination with Quantization": the
// retrieval heads' full caches in 4 bits; "Category 3: KV Cache Quantization": 4 or 8 bits).
// Keys are quantized per channel over aligned groups of kQ4Group tokens, values per token,
// both only when their group is complete, the codes stored in the operand layouts of the
// decode kernel (below). Until a group is complete the group's tokens wait in a bf16 residual
// block (row t % kQ4Group). Parameters of a block with minimum mn and maximum mx, L = 15 (4
// bits) or 255 (8 bits): scale = bf16((mx - mn) / L) and zero = bf16(mn), stored; the code of
// x is rint((x - zero) / scale) clamped to 0..L (0 when scale is 0), in IEEE float32 against
// the stored values, so the decision is reproducible.
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

template <int BITS>
__device__ __forceinline__ uint32_t code_of(float x, float mn, float scale) {
  constexpr float kLevels = (float)((1 << BITS) - 1);
  if (scale == 0.f) return 0u;
  const float r = __builtin_rintf((x - mn) / scale);
  return (uint32_t)fminf(fmaxf(r, 0.f), kLevels);
}

// Codes are stored in the operand layouts of the decode kernel's matrix products. 4 bits: a
// code word holds 8 codes, element e in bits 4e .. 4e + 3. 8 bits: a word holds 4 codes,
// element e in byte e.
//   Keys, 4 bits: per token row, D / 8 words; the word in slot KC j + kc (KC = D / 32) holds
//         channels 32 kc + 8 j .. + 7, so the KC words one lane needs for a token are
//         contiguous.
//   Keys, 8 bits: per token row, D / 4 words; the word in slot 2 KC j + 2 kc + h holds
//         channels 32 kc + 8 j + 4 h .. + 3 (the 2 KC words of a lane contiguous).
//   Values, 4 bits: per group, word ((s (D / 64) + h) 64 + l) 4 + w, with l = 16 j + (c % 16)
//         and c / 16 = 4 h + w, holds channel c; its element e is token 32 s + 16 (e / 4) +
//         4 j + e % 4 (the tokens whose logits lane l of the transposed logit tile holds). A
//         wave's value load for step s reads 1 KB contiguous per h.
//   Values, 8 bits: per group, word ((s (D / 32) + h) 64 + l) 4 + u, with l = 16 j + (c % 16)
//         and c / 16 = 2 h + u / 2, holds channel c; its element e is token 32 s +
//         16 (u % 2) + 4 j + e. Again 1 KB contiguous per h and step.
static_assert(kG == 128, "four 32-token steps per group");

// Quantize the group staged in s (rows 0..kG-1, bf16) as keys: per channel over the rows.
// codes: the group's first code row; params: bf16 [2][D] (scale row, zero row); sk: the
// stored values (as float) in LDS for the code pass, which decides against them.
template <int D, int BITS>
__device__ void quantize_keys(const uint16_t (*s)[D], uint8_t* codes, uint16_t* params,
                              float* sk) {
  constexpr float kLevels = (float)((1 << BITS) - 1);
  const int c = threadIdx.x;
  if (c < D) {
    float mn = bf16_to_f32(s[0][c]), mx = mn;
    for (int r = 1; r < kG; ++r) {
      const float x = bf16_to_f32(s[r][c]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    const uint16_t sb = f32_to_bf16_bits((mx - mn) / kLevels), zb = f32_to_bf16_bits(mn);
    params[c] = sb;
    params[D + c] = zb;
    sk[c] = bf16_to_f32(sb);
    sk[D + c] = bf16_to_f32(zb);
  }
  __syncthreads();
  constexpr int KC = D / 32, CPW = 32 / BITS, W = D / CPW;  // codes per word, words per row
  uint32_t* cw = (uint32_t*)codes;
  for (int w = threadIdx.x; w < kG * W; w += kThreads) {
    const int r = w / W, slot = w % W;
    const int c0 = BITS == 4 ? 32 * (slot % KC) + 8 * (slot / KC)
                             : 32 * ((slot % (2 * KC)) / 2) + 8 * (slot / (2 * KC)) + 4 * (slot % 2);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < CPW; ++e)
      word |= code_of<BITS>(bf16_to_f32(s[r][c0 + e]), sk[D + c0 + e], sk[c0 + e]) << (BITS * e);
    cw[(int64_t)r * W + slot] = word;
  }
}

// Quantize the staged group as values: per token over the channels (one wave per token for
// the minimum and maximum). params: one word per token of the group, bf16 scale in the low
// half and bf16 zero in the high half; sp: the stored values (as float) in LDS.
template <int D, int BITS>
__device__ void quantize_values(const uint16_t (*s)[D], uint8_t* codes, uint32_t* params,
                                float* sp) {
  constexpr float kLevels = (float)((1 << BITS) - 1);
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
    const uint16_t sb = f32_to_bf16_bits((mx - mn) / kLevels), zb = f32_to_bf16_bits(mn);
    if (lane == 0) {
      params[r] = (uint32_t)sb | ((uint32_t)zb << 16);
      sp[2 * r] = bf16_to_f32(sb);
      sp[2 * r + 1] = bf16_to_f32(zb);
    }
  }
  __syncthreads();
  constexpr int kChunks = D * BITS / 256;  // 16-byte loads per lane and step
  uint32_t* cw = (uint32_t*)codes;
  for (int w = threadIdx.x; w < D * kG * BITS / 32; w += kThreads) {
    const int u = w & 3, l = (w >> 2) & 63, x = w >> 8;
    const int h = x % kChunks, st = x / kChunks, j = l >> 4;
    uint32_t word = 0;
    if constexpr (BITS == 4) {
      const int c = 16 * (4 * h + u) + (l & 15), t0 = 32 * st + 4 * j;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = t0 + 16 * (e >> 2) + (e & 3);
        word |= code_of<4>(bf16_to_f32(s[t][c]), sp[2 * t + 1], sp[2 * t]) << (4 * e);
      }
    } else {
      const int c = 16 * (2 * h + (u >> 1)) + (l & 15), t0 = 32 * st + 16 * (u & 1) + 4 * j;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + e;
        word |= code_of<8>(bf16_to_f32(s[t][c]), sp[2 * t + 1], sp[2 * t]) << (8 * e);
      }
    }
    cw[w] = word;
  }
}

template <int D, int BITS>
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
      uint8_t* codes = (uint8_t*)base + (int64_t)g * kG * (D * BITS / 8);
      if (is_v)
        quantize_values<D, BITS>(s, codes, (uint32_t*)(base + a.q4_params) + (int64_t)g * kG, sp);
      else
        quantize_keys<D, BITS>(s, codes, (uint16_t*)(base + a.q4_params) + (int64_t)g * 2 * D,
                               sp);
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

// 8 channels c0 .. c0 + 7 of key t of a retrieval head whose group is complete, read back
// through the key layout above: c * scale + zero in float32 (c * scale is exact: at most 8 + 8
// significant bits; one rounding for the sum).
template <int D, int BITS>
__device__ __forceinline__ void key_values8(const char* head, int64_t q4_params, int t, int c0,
                                            float val[8]) {
  constexpr int KC = D / 32;
  const int g = t / kG;
  const uint16_t* par = (const uint16_t*)(head + q4_params) + (int64_t)g * 2 * D;
  const uint4 sv = *(const uint4*)(par + c0), zv = *(const uint4*)(par + D + c0);
  const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w}, zw[4] = {zv.x, zv.y, zv.z, zv.w};
  const uint32_t* row = (const uint32_t*)(head + (int64_t)t * (D * BITS / 8));
  const int k = c0 / 32, j = (c0 % 32) / 8;
  uint32_t code[8];
  if constexpr (BITS == 4) {
    const uint32_t cw = row[KC * j + k];
#pragma unroll
    for (int e = 0; e < 8; ++e) code[e] = (cw >> (4 * e)) & 15u;
  } else {
    const uint2 cw = *(const uint2*)(row + 2 * KC * j + 2 * k);
#pragma unroll
    for (int e = 0; e < 8; ++e) code[e] = ((e < 4 ? cw.x : cw.y) >> (8 * (e & 3))) & 255u;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sb = (e & 1) ? sw[e >> 1] >> 16 : sw[e >> 1] & 0xFFFFu;
    const uint32_t zb = (e & 1) ? zw[e >> 1] >> 16 : zw[e >> 1] & 0xFFFFu;
    val[e] = __builtin_fmaf((float)code[e], bf16_to_f32((uint16_t)sb), bf16_to_f32((uint16_t)zb));
  }
}

__device__ __forceinline__ void bf16x8_to_f32(uint4 w, float val[8]) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    val[2 * i] = __builtin_bit_cast(float, ww[i] << 16);
    val[2 * i + 1] = __builtin_bit_cast(float, ww[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint4 f32x8_to_bf16(const float val[8]) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (uint32_t)f32_to_bf16_bits(val[2 * i]) | ((uint32_t)f32_to_bf16_bits(val[2 * i + 1]) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// A bf16 pair to an fp16 pair through float32, rounding to nearest even: exact for magnitudes
// in [2^-14, 65504] (bf16 carries 8 significant bits, fp16 11), which is how the prefill kernel
// takes bf16 values into its fp16 PV product.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
__device__ __forceinline__ uint32_t bf16w_to_f16w(uint32_t w) {
  const f32x2_t x = {__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xFFFF0000u)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, half2_t));
}
__device__ __forceinline__ uint4 bf16x8_to_f16(uint4 w) {
  return make_uint4(bf16w_to_f16w(w.x), bf16w_to_f16w(w.y), bf16w_to_f16w(w.z), bf16w_to_f16w(w.w));
}

// Read-back into bf16 rows (DequantArgs): one thread per (K or V, sequence, head, token, 8
// channels), reading the codes through the layouts above. A value is c * scale + zero in
// float32, rounded to bf16 to nearest even. With a.rope_base set only the values are read
// back here (launch_rope_stage writes the keys). With a.v_f16 the value rows are written as
// fp16 (the bf16 value, converted exactly) for the prefill kernel's fp16-value form.
template <int D, int BITS>
__global__ void __launch_bounds__(kThreads) kv4_dequant_kernel(DequantArgs a) {
  constexpr int CH = D / 8;
  const int64_t per_tensor = (int64_t)a.nb * a.Hr * a.cap_s * CH;
  const int64_t u0 = a.rope_base ? per_tensor : 0;
  for (int64_t u = u0 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < 2 * per_tensor;
       u += (int64_t)gridDim.x * blockDim.x) {
    const bool is_v = u >= per_tensor;
    int64_t w = is_v ? u - per_tensor : u;
    const int x = (int)(w % CH);
    w /= CH;
    const int t = (int)(w % a.cap_s);
    w /= a.cap_s;
    const int r = (int)(w % a.Hr);
    const int bi = (int)(w / a.Hr);
    const int n = a.c0[bi];
    if (t >= n) continue;
    const char* head = (const char*)(is_v ? a.full_v : a.full_k) +
                       ((int64_t)(a.b0 + bi) * a.Hr + r) * a.q4_stride;
    uint4* dst = (uint4*)((uint16_t*)(is_v ? a.out_v : a.out_k) +
                          (((int64_t)bi * a.Hr + r) * a.cap_s + t) * D + 8 * x);
    if (t >= (n / kG) * kG) {  // residual row
      const uint4 bw = *(const uint4*)(head + a.q4_resid + (int64_t)(t % kG) * D * 2 + 16 * x);
      *dst = (is_v && a.v_f16) ? bf16x8_to_f16(bw) : bw;
      continue;
    }
    const int g = t / kG, tt = t % kG, c0 = 8 * x;
    float val[8];
    if (!is_v) {  // per-channel scale and zero of the group
      key_values8<D, BITS>(head, a.q4_params, t, c0, val);
    } else {  // per-token scale and zero
      const uint32_t pw = ((const uint32_t*)(head + a.q4_params))[t];
      const float sc = bf16_to_f32((uint16_t)(pw & 0xFFFFu)), ze = bf16_to_f32((uint16_t)(pw >> 16));
      const uint32_t* grp = (const uint32_t*)(head + (int64_t)g * kG * (D * BITS / 8));
      const int st = tt / 32, rr = tt % 32, j = (rr % 16) / 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = c0 + e, cb = c / 16, lane = 16 * j + c % 16;
        uint32_t code;
        if constexpr (BITS == 4) {
          const int el = 4 * (rr / 16) + rr % 4;  // element of the token in its word
          const uint32_t cw = grp[((st * (D / 64) + cb / 4) * 64 + lane) * 4 + cb % 4];
          code = (cw >> (4 * el)) & 15u;
        } else {
          const int uu = 2 * (cb % 2) + rr / 16;
          const uint32_t cw = grp[((st * (D / 32) + cb / 2) * 64 + lane) * 4 + uu];
          code = (cw >> (8 * (rr % 4))) & 255u;
        }
        val[e] = __builtin_fmaf((float)code, sc, ze);
      }
    }
    const uint4 bw = f32x8_to_bf16(val);
    *dst = (is_v && a.v_f16) ? bf16x8_to_f16(bw) : bw;
  }
}

// Keys of a pre-RoPE cache turned at their positions into bf16 staging (DequantArgs with
// rope_base set; OpenReview thread, the authors' reply on KV quantization: keys quantized
// before RoPE). RoPE in its rotate-half form: channels i and i + D/2 turn by t f_i,
// f_i = theta^(-2 i / D). One thread per (position, 8 pairs, group of kStageHeads heads): the
// angles of pairs 8 x .. 8 x + 7 at one position, then those pairs of the group's key rows at
// that position, from three sources in turn: the retrieval heads' earlier tokens (dequantized
// as in kv4_dequant_kernel, or residual rows), the chunk's keys as given (position c0 + i),
// and the held streaming slots (slot s < S holds position s, a ring slot the latest t < c0
// with t = s (mod R) past the sinks). The angle of position t = 128 g + tau is composed from the base table's (cos, sin)
// of 128 g f_i (float32 from float64) and sincosf(tau f_i), where tau f_i < 128 keeps the
// float32 argument accurate; the pair turns in float32 and each result is rounded to bf16 to
// nearest even.
constexpr int kStageHeads = 4;
__host__ __device__ constexpr int stage_groups(int heads) {
  return (heads + kStageHeads - 1) / kStageHeads;
}
template <int D, int BITS>
__global__ void __launch_bounds__(kThreads) kv4_rope_stage_kernel(DequantArgs a) {
  constexpr int HX = D / 16;  // pieces of 8 pairs per row
  constexpr int H = D / 2;
  const int SR = a.S + a.R;
  const int gr = stage_groups(a.Hr), gc = stage_groups(a.Hkv), gs = stage_groups(a.Hs);
  const int64_t n_pre = (int64_t)a.nb * a.cap_s * HX * gr;
  const int64_t n_chunk = (int64_t)a.nb * a.m * HX * gc;
  const int64_t n_str = (int64_t)a.nb * SR * HX * gs;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_pre + n_chunk + n_str;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int part = u < n_pre ? 0 : u < n_pre + n_chunk ? 1 : 2;
    int64_t w = part == 0 ? u : part == 1 ? u - n_pre : u - n_pre - n_chunk;
    const int x = (int)(w % HX);
    w /= HX;
    const int ngr = part == 0 ? gr : part == 1 ? gc : gs;
    const int h0 = (int)(w % ngr) * kStageHeads;  // first head of this item's group
    w /= ngr;
    const int rows = part == 0 ? a.cap_s : part == 1 ? a.m : SR;
    const int row = (int)(w % rows);
    const int bi = (int)(w / rows);
    const int n = a.c0[bi];
    if (part != 1 && row >= n) continue;  // past the prefix, or an empty slot (never read)
    int pos;
    if (part == 0) pos = row;
    else if (part == 1) pos = n + row;
    else pos = row < a.S ? row : row + a.R * ((n - 1 - row) / a.R);
    // (cos, sin) of pairs 8 x + e at pos
    const int g = pos / kG, tau = pos % kG;
    const float2* base = (const float2*)a.rope_base + (int64_t)g * H + 8 * x;
    float cs[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = exp2f(-(float)(2 * (8 * x + e)) / (float)D * a.log2_theta);
      float st, ct;
      sincosf((float)tau * f, &st, &ct);
      const float2 bb = base[e];
      cs[e] = bb.x * ct - bb.y * st;
      sn[e] = bb.y * ct + bb.x * st;
    }
    auto turn = [&](const float (&x1)[8], const float (&x2)[8], uint16_t* dst) {
      float y1[8], y2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y1[e] = x1[e] * cs[e] - x2[e] * sn[e];
        y2[e] = x1[e] * sn[e] + x2[e] * cs[e];
      }
      *(uint4*)(dst + 8 * x) = f32x8_to_bf16(y1);
      *(uint4*)(dst + H + 8 * x) = f32x8_to_bf16(y2);
    };
    float x1[8], x2[8];
    if (part == 0) {
      const bool resid = row >= (n / kG) * kG;
#pragma unroll
      for (int r = h0; r < h0 + kStageHeads; ++r) {
        if (r >= a.Hr) break;
        const char* head = (const char*)a.full_k + ((int64_t)(a.b0 + bi) * a.Hr + r) * a.q4_stride;
        if (resid) {
          const uint16_t* src = (const uint16_t*)(head + a.q4_resid) + (int64_t)(row % kG) * D;
          bf16x8_to_f32(*(const uint4*)(src + 8 * x), x1);
          bf16x8_to_f32(*(const uint4*)(src + H + 8 * x), x2);
        } else {
          key_values8<D, BITS>(head, a.q4_params, row, 8 * x, x1);
          key_values8<D, BITS>(head, a.q4_params, row, H + 8 * x, x2);
        }
        turn(x1, x2, (uint16_t*)a.out_k + (((int64_t)bi * a.Hr + r) * a.cap_s + row) * D);
      }
    } else if (part == 1) {
#pragma unroll
      for (int j = h0; j < h0 + kStageHeads; ++j) {
        if (j >= a.Hkv) break;
        const int64_t off = (((int64_t)bi * a.m + row) * a.Hkv + j) * D;
        const uint16_t* src = (const uint16_t*)a.chunk_k + off;
        bf16x8_to_f32(*(const uint4*)(src + 8 * x), x1);
        bf16x8_to_f32(*(const uint4*)(src + H + 8 * x), x2);
        turn(x1, x2, (uint16_t*)a.out_chunk_k + off);
      }
    } else {
#pragma unroll
      for (int cls = h0; cls < h0 + kStageHeads; ++cls) {
        if (cls >= a.Hs) break;
        const int64_t off = (((int64_t)(a.b0 + bi) * a.Hs + cls) * SR + row) * D;
        const uint16_t* src = (const uint16_t*)a.str_k + off;
        bf16x8_to_f32(*(const uint4*)(src + 8 * x), x1);
        bf16x8_to_f32(*(const uint4*)(src + H + 8 * x), x2);
        turn(x1, x2, (uint16_t*)a.out_str_k + off);
      }
    }
  }
}

}  // namespace

int launch_dequant_kv4(const DequantArgs& a, int head_dim, void* stream) {
  // K and V, or V alone for a pre-RoPE cache
  const int64_t work = (a.rope_base ? 1 : 2) * (int64_t)a.nb * a.Hr * a.cap_s * (head_dim / 8);
  if (work == 0) return 0;
  int64_t blocks = (work + kThreads - 1) / kThreads;
  if (blocks > 16384) blocks = 16384;
  const dim3 grid((unsigned)blocks), block(kThreads);
  hipStream_t st = (hipStream_t)stream;
  if (head_dim == 128 && a.qbits == 4)
    hipLaunchKernelGGL((kv4_dequant_kernel<128, 4>), grid, block, 0, st, a);
  else if (head_dim == 64 && a.qbits == 4)
    hipLaunchKernelGGL((kv4_dequant_kernel<64, 4>), grid, block, 0, st, a);
  else if (head_dim == 128 && a.qbits == 8)
    hipLaunchKernelGGL((kv4_dequant_kernel<128, 8>), grid, block, 0, st, a);
  else if (head_dim == 64 && a.qbits == 8)
    hipLaunchKernelGGL((kv4_dequant_kernel<64, 8>), grid, block, 0, st, a);
  else
    return -1;
  return (int)hipGetLastError();
}

int launch_rope_stage(const DequantArgs& a, int head_dim, void* stream) {
  // one work item per position, 8-pair piece and group of kStageHeads heads
  const int64_t rows = (int64_t)a.nb * a.cap_s * stage_groups(a.Hr) +
                       (int64_t)a.nb * a.m * stage_groups(a.Hkv) +
                       (int64_t)a.nb * (a.S + a.R) * stage_groups(a.Hs);
  const int64_t work = rows * (head_dim / 16);
  if (work == 0) return 0;
  int64_t blocks = (work + kThreads - 1) / kThreads;
  if (blocks > 16384) blocks = 16384;
  const dim3 grid((unsigned)blocks), block(kThreads);
  hipStream_t st = (hipStream_t)stream;
  if (head_dim == 128 && a.qbits == 4)
    hipLaunchKernelGGL((kv4_rope_stage_kernel<128, 4>), grid, block, 0, st, a);
  else if (head_dim == 64 && a.qbits == 4)
    hipLaunchKernelGGL((kv4_rope_stage_kernel<64, 4>), grid, block, 0, st, a);
  else if (head_dim == 128 && a.qbits == 8)
    hipLaunchKernelGGL((kv4_rope_stage_kernel<128, 8>), grid, block, 0, st, a);
  else if (head_dim == 64 && a.qbits == 8)
    hipLaunchKernelGGL((kv4_rope_stage_kernel<64, 8>), grid, block, 0, st, a);
  else
    return -1;
  return (int)hipGetLastError();
}

int launch_append_kv4(const AppendArgs& a, int head_dim, void* stream) {
  const int64_t blocks = (int64_t)a.nb * a.Hr * (1 + a.q4_mid);
  if (blocks == 0) return 0;
  const dim3 grid((unsigned)blocks), block(kThreads);
  hipStream_t st = (hipStream_t)stream;
  if (head_dim == 128 && a.qbits == 4)
    hipLaunchKernelGGL((kv4_append_kernel<128, 4>), grid, block, 0, st, a);
  else if (head_dim == 64 && a.qbits == 4)
    hipLaunchKernelGGL((kv4_append_kernel<64, 4>), grid, block, 0, st, a);
  else if (head_dim == 128 && a.qbits == 8)
    hipLaunchKernelGGL((kv4_append_kernel<128, 8>), grid, block, 0, st, a);
  else if (head_dim == 64 && a.qbits == 8)
    hipLaunchKernelGGL((kv4_append_kernel<64, 8>), grid, block, 0, st, a);
  else
    return -1;
  return (int)hipGetLastError();
}

}  // namespace duo
