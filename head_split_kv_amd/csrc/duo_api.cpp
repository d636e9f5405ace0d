// The C ABI entry points that enqueue device work. Every argument and capacity check runs
// here on the host before anything is launched; on an error nothing is launched and neither
// the host mirror nor the device state changes.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "duo_internal.h"

namespace duo {
int copy_d2h_sync(void* dst, const void* src, uint64_t bytes, void* stream);
}

using namespace duo;

namespace {

// Rows are moved in 16-byte chunks, so every tensor must start on a 16-byte boundary.
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

bool layer_ok(const duo_cache* c, int32_t layer) {
  return c && layer >= 0 && layer < c->cfg.num_layers;
}

int32_t& len_of(duo_cache* c, int32_t layer, int32_t b) {
  return c->lens[(size_t)layer * c->cfg.batch + b];
}

// The pre-RoPE cos/sin tables (RopeGeom) of a cache, or nulls when its keys are appended as
// attended.
struct RopePtrs {
  const float* base = nullptr;
  const uint32_t* tau16 = nullptr;
};

RopePtrs rope_ptrs(const duo_cache* c) {
  RopePtrs r;
  if (c->cfg.rope_theta > 0.f) {
    const RopeGeom g = rope_geom(c->cfg.capacity, c->cfg.head_dim);
    const char* t = c->arena + c->lay.rope_off;
    r.base = (const float*)(t + g.base);
    r.tau16 = (const uint32_t*)(t + g.tau16);
  }
  return r;
}

struct LayerPtrs {
  char* full_k;
  char* full_v;
  char* str_k;
  char* str_v;
  int32_t* slot_pos;
  int32_t* seq_len;
};

LayerPtrs layer_ptrs(duo_cache* c, int32_t layer) {
  const LayerInfo& li = c->layers[layer];
  const uint64_t SR = (uint64_t)c->cfg.sink + c->cfg.recent;
  LayerPtrs p;
  p.full_k = c->arena + c->lay.full_k_off + li.full_off;
  p.full_v = c->arena + c->lay.full_v_off + li.full_off;
  p.str_k = c->arena + c->lay.str_k_off + li.str_off;
  p.str_v = c->arena + c->lay.str_v_off + li.str_off;
  p.slot_pos = (int32_t*)(c->arena + c->lay.slot_pos_off) + (uint64_t)layer * c->cfg.batch * SR;
  p.seq_len = (int32_t*)(c->arena + c->lay.seq_len_off) + (uint64_t)layer * c->cfg.batch;
  return p;
}

// Split-K partials of the decode kernel: o [B][Hq][max_splits][D], then (m, l) pairs.
struct Workspace {
  float* part_o;
  float* part_ml;
};

Workspace workspace(duo_cache* c) {
  const uint64_t B = c->cfg.batch, Hq = c->cfg.num_q_heads, D = c->cfg.head_dim;
  const uint64_t S = c->cfg.max_splits;
  char* base = c->arena + c->lay.workspace_off;
  Workspace w;
  w.part_o = (float*)base;
  w.part_ml = (float*)(base + (B * Hq * S * D * 4 + kAlign - 1) / kAlign * kAlign);
  return w;
}

}  // namespace

namespace {

// The next event pair of a kernel timer, or none when the timer is off or full.
KernelMarks next_marks(duo_cache* c, int kind) {
  KernelMarks m;
  duo_cache::Timer& t = c->timers[kind];
  if (2 * (t.used + 1) <= (int)t.ev.size()) {
    m.begin = t.ev[2 * t.used];
    m.end = t.ev[2 * t.used + 1];
    ++t.used;
  }
  return m;
}

// Bytes of split-K partials for `stride` partials per (sequence, query head): o [B][Hq]
// [stride][D] floats, then, 256-byte aligned, (m, l) [B][Hq][stride][2].
uint64_t partial_bytes(const duo_cache* c, uint64_t stride) {
  const uint64_t rows = (uint64_t)c->cfg.batch * c->cfg.num_q_heads * stride;
  return (rows * c->cfg.head_dim * 4 + kAlign - 1) / kAlign * kAlign + rows * 2 * 4;
}

// Shared by duo_attn_decode (k == v == null), duo_decode_step and, with use_static,
// duo_attn_decode_noalloc (partials in the static scratch instead of the arena's workspace).
duo_status decode_impl(duo_cache* c, int32_t layer, const void* q, const void* k, const void* v,
                       void* out, float* lse, void* stream, bool use_static = false) {
  if (!layer_ok(c, layer) || !q || !out || !aligned16(q) || !aligned16(out) || !aligned4(lse))
    return DUO_ERR_INVALID;
  const bool fused = k != nullptr;
  if (fused && (!v || !aligned16(k) || !aligned16(v))) return DUO_ERR_INVALID;
  int32_t n_max = 0;
  for (int32_t b = 0; b < c->cfg.batch; ++b) {
    const int64_t n = (int64_t)len_of(c, layer, b) + (fused ? 1 : 0);
    if (n < 1) return DUO_ERR_INVALID;
    if (n > c->cfg.capacity) return DUO_ERR_CAPACITY;
    n_max = std::max(n_max, (int32_t)n);
  }
  const LayerInfo& li = c->layers[layer];
  const LayerPtrs p = layer_ptrs(c, layer);
  const Workspace w = workspace(c);
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.full_k = p.full_k;
  a.full_v = p.full_v;
  a.str_k = p.str_k;
  a.str_v = p.str_v;
  for (int32_t b = 0; b < c->cfg.batch; ++b) a.n[b] = len_of(c, layer, b) + (fused ? 1 : 0);
  a.part_o = w.part_o;
  a.part_ml = w.part_ml;
  a.new_k = k;
  a.new_v = v;
  a.slot_pos = p.slot_pos;
  a.seq_len = p.seq_len;
  a.B = c->cfg.batch;
  a.Hq = c->cfg.num_q_heads;
  a.Hkv = c->cfg.num_kv_heads;
  a.Hr = li.n_ret;
  a.Hs = li.n_str;
  a.cap = c->cfg.capacity;
  a.S = c->cfg.sink;
  a.R = c->cfg.recent;
  a.max_splits = c->cfg.max_splits;
  const int group = c->cfg.num_q_heads / c->cfg.num_kv_heads;
  const int32_t qbits = (c->cfg.kv_bits == 4 || c->cfg.kv_bits == 8) ? c->cfg.kv_bits : 0;
  const bool quant = qbits != 0;  // 4- or 8-bit full caches
  // 4- and 8-bit caches: a streaming head's window is cut over up to 8 blocks of ~128 slots, so that
  // it is done long before the retrieval groups
  a.nss = 1;
  if (quant && a.Hs > 0) {
    const int32_t rows = std::min(n_max, c->cfg.sink + c->cfg.recent);
    a.nss = std::max(1, std::min({8, (rows + 127) / 128, (int)c->cfg.max_splits}));
  }
  // 4- and 8-bit caches: one more block and one more partial per retrieval head (its residual rows)
  const int32_t split_cap = quant ? a.max_splits - 1 : a.max_splits;
  // One round of splits: two blocks per CU for a batch, whose sequences' unequal lengths then
  // share each CU (the second block takes up the bandwidth a short sequence's block leaves),
  // one block per CU for a single sequence, whose four waves then have the CU's memory
  // pipeline to themselves. Measured per layer-step: the 128K GQA layer 49.6-50.5 us with
  // 56-63 splits (one per CU) against 51.2-52.3 us with 126-127, its 4-bit cache 22.6 against
  // 23.3 us; the 32 layers of 8 ragged sequences 2,355 us at two blocks per CU against
  // 2,477 us at one.
  const RopePtrs rp = rope_ptrs(c);
  const int32_t resident = decode_resident_blocks(c->cfg.dtype, c->cfg.head_dim, group, qbits,
                                                  rp.base != nullptr, a.B == 1 ? 1 : 2);
  a.nsplit = c->force_splits
                 ? std::min(c->force_splits, split_cap)
                 : choose_decode_splits(n_max, a.B, a.Hr, a.Hs * a.nss + (quant ? a.Hr : 0),
                                        split_cap, resident);
  if (use_static) {
    // partials per (sequence, query head): the splits (plus the residual's on a quantized
    // cache) or a quantized cache's streaming window blocks; fewer splits until they fit the scratch
    const int32_t extra = quant ? 1 : 0;
    int32_t stride = std::max(a.nsplit + extra, a.nss);
    while (stride > 1 && partial_bytes(c, stride) > kScratchBytes) --stride;
    const bool fits = partial_bytes(c, stride) <= kScratchBytes;
    if (quant && (stride < 2 || !fits)) return DUO_ERR_CAPACITY;
    if (!fits) stride = 1;  // one split per head: outputs are written directly, no partials
    a.nsplit = std::max(1, std::min(a.nsplit, stride - extra));
    a.nss = std::min(a.nss, stride);
    void* base = nullptr;
    if (static_scratch(&base) != 0) return DUO_ERR_HIP;
    const uint64_t rows = (uint64_t)a.B * a.Hq * stride;
    a.max_splits = stride;
    a.part_o = (float*)base;
    a.part_ml = (float*)((char*)base + (rows * c->cfg.head_dim * 4 + kAlign - 1) / kAlign * kAlign);
  }
  a.scale_log2 = (float)((double)c->scale * 1.4426950408889634);
  a.out_f32 = c->cfg.out_dtype == DUO_F32;
  for (int k = 0; k < kMaxKvHeads; ++k) {
    a.ret_kv[k] = li.ret_kv[k];
    a.str_kv[k] = li.str_kv[k];
  }
  if (quant) {
    const Q4Geom g = q4_geom(c->cfg.capacity, c->cfg.head_dim, qbits);
    a.qbits = qbits;
    a.q4_stride = (int64_t)g.stride;
    a.q4_params = (int64_t)g.codes;
    a.q4_resid = (int64_t)(g.codes + g.params);
    a.rope_base = rp.base;
    a.rope_tau16 = rp.tau16;
  }
  if (launch_decode(a, c->cfg.dtype, c->cfg.head_dim, group, stream,
                    next_marks(c, DUO_TIMING_DECODE)) != 0)
    return DUO_ERR_HIP;
  if (fused)
    for (int32_t b = 0; b < c->cfg.batch; ++b) len_of(c, layer, b) += 1;
  return DUO_OK;
}

}  // namespace

extern "C" {

duo_status duo_cache_reset(duo_cache* c, void* stream) {
  if (!c) return DUO_ERR_INVALID;
  const uint64_t L = c->cfg.num_layers, B = c->cfg.batch;
  const uint64_t SR = (uint64_t)c->cfg.sink + c->cfg.recent;
  ResetArgs a;
  a.slot_pos = (int32_t*)(c->arena + c->lay.slot_pos_off);
  a.n_slot = (int64_t)(L * B * SR);
  a.seq_len = (int32_t*)(c->arena + c->lay.seq_len_off);
  a.n_len = (int64_t)(L * B);
  if (launch_reset(a, stream) != 0) return DUO_ERR_HIP;
  if (c->cfg.rope_theta > 0.f &&
      launch_rope_tables(c->arena + c->lay.rope_off, c->cfg.head_dim,
                         rope_geom(c->cfg.capacity, c->cfg.head_dim).nbase,
                         (double)c->cfg.rope_theta, stream) != 0)
    return DUO_ERR_HIP;
  std::fill(c->lens.begin(), c->lens.end(), 0);
  return DUO_OK;
}

duo_status duo_cache_init(const duo_config* cfg, void* arena, uint64_t arena_bytes,
                          void* stream, duo_cache** out) {
  duo_cache* c = nullptr;
  const duo_status st = duo_cache_create(cfg, arena, arena_bytes, &c);
  if (st != DUO_OK) return st;
  const duo_status rs = duo_cache_reset(c, stream);
  if (rs != DUO_OK) {
    duo_cache_destroy(c);
    return rs;
  }
  *out = c;
  return DUO_OK;
}

duo_status duo_cache_set_lengths(duo_cache* c, const int32_t* lens, void* stream) {
  if (!c || !lens) return DUO_ERR_INVALID;
  const int32_t L = c->cfg.num_layers, B = c->cfg.batch;
  for (int64_t i = 0; i < (int64_t)L * B; ++i)
    if (lens[i] < 0 || lens[i] > c->cfg.capacity) return DUO_ERR_INVALID;
  for (int32_t layer = 0; layer < L; ++layer) {
    const LayerPtrs p = layer_ptrs(c, layer);
    SetLenArgs a;
    std::memset(&a, 0, sizeof(a));
    a.slot_pos = p.slot_pos;
    a.seq_len = p.seq_len;
    a.B = B;
    a.S = c->cfg.sink;
    a.R = c->cfg.recent;
    std::memcpy(a.n, lens + (int64_t)layer * B, sizeof(int32_t) * B);
    if (launch_set_lengths(a, stream) != 0) return DUO_ERR_HIP;
    std::memcpy(&len_of(c, layer, 0), lens + (int64_t)layer * B, sizeof(int32_t) * B);
  }
  return DUO_OK;
}

duo_status duo_kv_append(duo_cache* c, int32_t layer, int32_t seq, const void* k,
                         const void* v, int32_t n_new, void* stream) {
  if (!layer_ok(c, layer) || seq < -1 || seq >= c->cfg.batch || n_new < 0)
    return DUO_ERR_INVALID;
  if (n_new == 0) return DUO_OK;
  if (!k || !v || !aligned16(k) || !aligned16(v)) return DUO_ERR_INVALID;
  const int32_t b0 = seq < 0 ? 0 : seq, nb = seq < 0 ? c->cfg.batch : 1;
  for (int32_t b = b0; b < b0 + nb; ++b)
    if ((int64_t)len_of(c, layer, b) + n_new > c->cfg.capacity) return DUO_ERR_CAPACITY;
  const LayerInfo& li = c->layers[layer];
  const LayerPtrs p = layer_ptrs(c, layer);
  AppendArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k = k;
  a.v = v;
  a.full_k = p.full_k;
  a.full_v = p.full_v;
  a.str_k = p.str_k;
  a.str_v = p.str_v;
  a.slot_pos = p.slot_pos;
  a.seq_len = p.seq_len;
  a.b0 = b0;
  a.nb = nb;
  a.m = n_new;
  a.Hkv = c->cfg.num_kv_heads;
  a.Hr = li.n_ret;
  a.Hs = li.n_str;
  a.cap = c->cfg.capacity;
  a.S = c->cfg.sink;
  a.R = c->cfg.recent;
  a.row_bytes = c->cfg.head_dim * c->esize;
  std::memcpy(a.cls_idx, li.cls_idx, sizeof(a.cls_idx));
  std::memcpy(a.ret_kv, li.ret_kv, sizeof(a.ret_kv));
  for (int32_t i = 0; i < nb; ++i) a.n_old[i] = len_of(c, layer, b0 + i);
  const bool quant = c->cfg.kv_bits == 4 || c->cfg.kv_bits == 8;
  if (quant) {
    const Q4Geom g = q4_geom(c->cfg.capacity, c->cfg.head_dim, c->cfg.kv_bits);
    a.qbits = c->cfg.kv_bits;
    a.q4_stride = (int64_t)g.stride;
    a.q4_params = (int64_t)g.codes;
    a.q4_resid = (int64_t)(g.codes + g.params);
    for (int32_t i = 0; i < nb; ++i) {
      const int32_t n0 = a.n_old[i], n1 = n0 + n_new;
      const int32_t first_new = n0 / kQ4Group + (n0 % kQ4Group != 0 ? 1 : 0);
      a.q4_mid = std::max(a.q4_mid, n1 / kQ4Group - first_new);
    }
  }
  if (launch_append(a, c->cfg.dtype, stream) != 0) return DUO_ERR_HIP;
  if (quant && a.Hr > 0 && launch_append_kv4(a, c->cfg.head_dim, stream) != 0) return DUO_ERR_HIP;
  for (int32_t b = b0; b < b0 + nb; ++b) len_of(c, layer, b) += n_new;
  return DUO_OK;
}

duo_status duo_attn_decode(duo_cache* c, int32_t layer, const void* q, void* out, float* lse,
                           void* stream) {
  return decode_impl(c, layer, q, nullptr, nullptr, out, lse, stream);
}

duo_status duo_attn_decode_noalloc(duo_cache* c, int32_t layer, const void* q, void* out,
                                   float* lse, void* stream) {
  return decode_impl(c, layer, q, nullptr, nullptr, out, lse, stream, true);
}

duo_status duo_decode_step(duo_cache* c, int32_t layer, const void* q, const void* k,
                           const void* v, void* out, float* lse, void* stream) {
  if (!k || !v) return DUO_ERR_INVALID;
  if (c && (c->cfg.kv_bits == 4 || c->cfg.kv_bits == 8) && layer_ok(c, layer)) {
    // 4- and 8-bit full caches: a token that completes a group of some sequence needs the
    // group's quantization, so that step runs as append + decode; otherwise the token only
    // lands in the bf16 residual and the step is fused like the bf16 one
    bool completes = false;
    for (int32_t b = 0; b < c->cfg.batch; ++b)
      completes |= (len_of(c, layer, b) + 1) % kQ4Group == 0;
    if (completes) {
      if (!q || !out || !aligned16(q) || !aligned16(out) || !aligned4(lse)) return DUO_ERR_INVALID;
      const duo_status st = duo_kv_append(c, layer, -1, k, v, 1, stream);
      if (st != DUO_OK) return st;
      return decode_impl(c, layer, q, nullptr, nullptr, out, lse, stream);
    }
  }
  return decode_impl(c, layer, q, k, v, out, lse, stream);
}

namespace {

// Staging of duo_attn_prefill_staged, byte offsets: the retrieval prefix as bf16 rows, K at 0
// and V at pv, [nb][Hr][c_max][D] each; with pre-RoPE keys also the chunk's keys turned at
// `chunk`, [nb][m][Hkv][D], and the layer's streaming keys turned at `str`, [B][Hs][S+R][D]
// (indexed by sequence like the cache; only the call's sequences are written).
// Staging of duo_attn_prefill_staged (byte offsets). On a 4- or 8-bit cache: the retrieval
// prefix read back, keys (bf16) at 0 and values (fp16) at pv, both [nb][Hr][c_max][d]; with
// pre-RoPE keys the chunk's keys turned at `chunk` and the streaming keys turned at `str`.
// On every staged bf16 path: the chunk's values in fp16 at cv ([nb][m][Hkv][d]) and the
// streaming values in fp16 at sv ([B][Hs][S+R][d]); on a bf16 cache the prefix values in fp16
// at pv = 0 ([nb][Hr][c_max][d]). Regions start on 256-byte boundaries.
struct StagingPlan {
  uint64_t pv = 0, chunk = 0, str = 0, cv = 0, sv = 0, bytes = 0;
  int32_t c_max = 0;
};
StagingPlan staging_plan(const duo_cache* c, int32_t layer, int32_t seq, int32_t n_chunk) {
  auto up = [](uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; };
  const int32_t b0 = seq < 0 ? 0 : seq, nb = seq < 0 ? c->cfg.batch : 1;
  StagingPlan p;
  for (int32_t b = b0; b < b0 + nb; ++b)
    p.c_max = std::max(p.c_max, c->lens[(size_t)layer * c->cfg.batch + b]);
  const uint64_t row = (uint64_t)c->cfg.head_dim * 2;
  const LayerInfo& li = c->layers[layer];
  const uint64_t pre = (uint64_t)nb * li.n_ret * (uint64_t)p.c_max * row;
  const uint64_t chunk_bytes = (uint64_t)nb * n_chunk * c->cfg.num_kv_heads * row;
  const uint64_t str_bytes =
      (uint64_t)c->cfg.batch * li.n_str * ((uint64_t)c->cfg.sink + c->cfg.recent) * row;
  uint64_t end;
  if (c->cfg.kv_bits != 4 && c->cfg.kv_bits != 8) {
    p.pv = 0;
    end = pre;
  } else {
    p.pv = pre;
    end = 2 * pre;
    if (c->cfg.rope_theta > 0.f) {
      p.chunk = up(end);
      p.str = p.chunk + up(chunk_bytes);
      end = p.str + str_bytes;
    }
  }
  p.cv = up(end);
  p.sv = p.cv + up(chunk_bytes);
  p.bytes = p.sv + str_bytes;
  return p;
}

// Checks and launch arguments of one prefill chunk (shared by duo_attn_prefill and
// duo_attn_gate_mixed). Returns DUO_OK with `a` filled, or the error to report.
// staged: the caller has a bf16 read-back of a quantized layer's retrieval caches to offer
// (duo_attn_prefill_staged); otherwise prefill over a quantized layer is unsupported.
duo_status prefill_args(duo_cache* c, int32_t layer, int32_t seq, const void* q, const void* k,
                        const void* v, int32_t n_chunk, void* out, float* lse, PrefillArgs& a,
                        bool staged = false) {
  // quantized retrieval caches, and pre-RoPE keys on any head, are read through staging
  if ((c->cfg.kv_bits == 4 || c->cfg.kv_bits == 8) &&
      (c->layers[layer].n_ret > 0 || c->cfg.rope_theta > 0.f) && !staged)
    return DUO_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
      !aligned16(out) || !aligned4(lse))
    return DUO_ERR_INVALID;
  const int32_t b0 = seq < 0 ? 0 : seq, nb = seq < 0 ? c->cfg.batch : 1;
  for (int32_t b = b0; b < b0 + nb; ++b)
    if ((int64_t)len_of(c, layer, b) + n_chunk > c->cfg.capacity) return DUO_ERR_CAPACITY;
  const LayerInfo& li = c->layers[layer];
  const LayerPtrs p = layer_ptrs(c, layer);
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.full_k = p.full_k;
  a.full_v = p.full_v;
  a.str_k = p.str_k;
  a.str_v = p.str_v;
  a.slot_pos = p.slot_pos;
  a.b0 = b0;
  a.nb = nb;
  a.m = n_chunk;
  a.Hq = c->cfg.num_q_heads;
  a.Hkv = c->cfg.num_kv_heads;
  a.Hr = li.n_ret;
  a.Hs = li.n_str;
  a.cap = c->cfg.capacity;
  a.S = c->cfg.sink;
  a.R = c->cfg.recent;
  a.scale_log2 = (float)((double)c->scale * 1.4426950408889634);
  a.out_f32 = c->cfg.out_dtype == DUO_F32;
  a.chunk_mode = c->cfg.streaming_prefill == DUO_PREFILL_CHUNK;
  std::memcpy(a.cls_idx, li.cls_idx, sizeof(a.cls_idx));
  std::memcpy(a.ret_kv, li.ret_kv, sizeof(a.ret_kv));
  std::memcpy(a.str_kv, li.str_kv, sizeof(a.str_kv));
  int32_t c_max = 0, c_sum = 0;
  for (int32_t i = 0; i < nb; ++i) {
    a.c0[i] = len_of(c, layer, b0 + i);
    c_max = std::max(c_max, a.c0[i]);
    c_sum += a.c0[i];
  }
  const int group = c->cfg.num_q_heads / c->cfg.num_kv_heads;
  const int qpb = kPrefillRows / group;
  a.n_qt = (n_chunk + qpb - 1) / qpb;
  a.nsplit = choose_prefill_splits(nb, n_chunk, c_max, c_sum, a.Hr, a.Hs, a.S, a.R, group,
                                   c->cfg.prefill_tiles,
                                   prefill_resident_blocks(c->cfg.head_dim, group),
                                   a.chunk_mode != 0);
  const uint64_t D = c->cfg.head_dim;
  char* ws = c->arena + c->lay.workspace_off;
  a.part_o = (float*)ws;
  a.part_ml = (float*)(ws + ((uint64_t)c->cfg.prefill_tiles * kPrefillTileRows * D * 4 + kAlign - 1) /
                                kAlign * kAlign);
  a.full_heads = li.n_ret;
  return DUO_OK;
}

duo_status launch_status(int rc) {
  if (rc == -1) return DUO_ERR_UNSUPPORTED;
  return rc != 0 ? DUO_ERR_HIP : DUO_OK;
}

}  // namespace

namespace {

// duo_attn_prefill_staged on a bf16 cache: the values the chunk reads are converted to fp16
// once into the staging (the prefix of every retrieval head [nb][Hr][c_max][d], the chunk's
// [nb][m][Hkv][d], the streaming caches [B][Hs][S+R][d]), and the prefill kernel reads them
// without converting each V tile in LDS. The products are the same: the kernel's conversion
// and the staging's are one function of each element.
duo_status prefill_v16(duo_cache* c, int32_t layer, int32_t seq, const void* q, const void* k,
                       const void* v, int32_t n_chunk, void* out, float* lse, void* staging,
                       uint64_t staging_bytes, void* stream) {
  const StagingPlan sp = staging_plan(c, layer, seq, n_chunk);
  if (!aligned16(staging) || staging_bytes < sp.bytes) return DUO_ERR_INVALID;
  if (n_chunk == 0) return DUO_OK;
  PrefillArgs a;
  const duo_status st = prefill_args(c, layer, seq, q, k, v, n_chunk, out, lse, a);
  if (st != DUO_OK) return st;
  char* stg = (char*)staging;
  V16StageArgs d;
  std::memset(&d, 0, sizeof(d));
  d.full_v = a.full_v;
  d.v = a.v;
  d.str_v = a.str_v;
  d.out_pv = stg + sp.pv;
  d.out_chunk = stg + sp.cv;
  d.out_str = stg + sp.sv;
  d.cap = a.cap;
  d.c_max = sp.c_max;
  d.b0 = a.b0;
  d.nb = a.nb;
  d.Hr = a.Hr;
  d.Hs = a.Hs;
  d.SR = a.S + a.R;
  d.m = n_chunk;
  d.Hkv = a.Hkv;
  d.D = c->cfg.head_dim;
  std::memcpy(d.c0, a.c0, sizeof(d.c0));
  if (launch_v16_stage(d, stream) != 0) return DUO_ERR_HIP;
  a.v16 = 1;
  a.full_v = stg + sp.pv;
  a.vcap = sp.c_max;
  a.v_b0 = a.b0;
  a.v = stg + sp.cv;
  a.str_v = stg + sp.sv;
  const int group = c->cfg.num_q_heads / c->cfg.num_kv_heads;
  return launch_status(launch_prefill(a, c->cfg.dtype, c->cfg.head_dim, group, stream,
                                      next_marks(c, DUO_TIMING_PREFILL)));
}

}  // namespace

duo_status duo_attn_prefill(duo_cache* c, int32_t layer, int32_t seq, const void* q,
                            const void* k, const void* v, int32_t n_chunk, void* out,
                            float* lse, void* stream) {
  if (!layer_ok(c, layer) || seq < -1 || seq >= c->cfg.batch || n_chunk < 0)
    return DUO_ERR_INVALID;
  if (n_chunk == 0) return DUO_OK;
  PrefillArgs a;
  const duo_status st = prefill_args(c, layer, seq, q, k, v, n_chunk, out, lse, a);
  if (st != DUO_OK) return st;
  const int group = c->cfg.num_q_heads / c->cfg.num_kv_heads;
  return launch_status(launch_prefill(a, c->cfg.dtype, c->cfg.head_dim, group, stream,
                                      next_marks(c, DUO_TIMING_PREFILL)));
}

duo_status duo_prefill_staging_bytes(const duo_cache* c, int32_t layer, int32_t seq,
                                     int32_t n_chunk, uint64_t* bytes) {
  if (!layer_ok(c, layer) || seq < -1 || seq >= c->cfg.batch || n_chunk < 0 || !bytes)
    return DUO_ERR_INVALID;
  *bytes = 0;
  const bool quant = c->cfg.kv_bits == 4 || c->cfg.kv_bits == 8;
  if (!quant && c->cfg.dtype != DUO_BF16) return DUO_OK;
  *bytes = staging_plan(c, layer, seq, n_chunk).bytes;
  return DUO_OK;
}

duo_status duo_attn_prefill_staged(duo_cache* c, int32_t layer, int32_t seq, const void* q,
                                   const void* k, const void* v, int32_t n_chunk, void* out,
                                   float* lse, void* staging, uint64_t staging_bytes,
                                   void* stream) {
  if (!layer_ok(c, layer) || seq < -1 || seq >= c->cfg.batch || n_chunk < 0)
    return DUO_ERR_INVALID;
  const bool quant = c->cfg.kv_bits == 4 || c->cfg.kv_bits == 8;
  if (!quant && (c->cfg.dtype != DUO_BF16 || !staging))
    return duo_attn_prefill(c, layer, seq, q, k, v, n_chunk, out, lse, stream);
  if (!quant) return prefill_v16(c, layer, seq, q, k, v, n_chunk, out, lse, staging,
                                 staging_bytes, stream);
  const bool rope = c->cfg.rope_theta > 0.f;
  const StagingPlan sp = staging_plan(c, layer, seq, n_chunk);
  if (sp.bytes > 0 && (!staging || !aligned16(staging) || staging_bytes < sp.bytes))
    return DUO_ERR_INVALID;
  if (n_chunk == 0) return DUO_OK;
  PrefillArgs a;
  const duo_status st = prefill_args(c, layer, seq, q, k, v, n_chunk, out, lse, a, true);
  if (st != DUO_OK) return st;
  char* stg = (char*)staging;
  const Q4Geom g = q4_geom(c->cfg.capacity, c->cfg.head_dim, c->cfg.kv_bits);
  DequantArgs d;
  std::memset(&d, 0, sizeof(d));
  d.full_k = a.full_k;
  d.full_v = a.full_v;
  d.out_k = stg;
  d.out_v = stg + sp.pv;
  d.q4_stride = (int64_t)g.stride;
  d.q4_params = (int64_t)g.codes;
  d.q4_resid = (int64_t)(g.codes + g.params);
  d.qbits = c->cfg.kv_bits;
  d.b0 = a.b0;
  d.nb = a.nb;
  d.Hr = a.Hr;
  d.cap_s = sp.c_max;
  d.v_f16 = 1;
  std::memcpy(d.c0, a.c0, sizeof(d.c0));
  if (rope) {
    d.rope_base = rope_ptrs(c).base;
    d.log2_theta = (float)std::log2((double)c->cfg.rope_theta);
    d.chunk_k = k;
    d.out_chunk_k = stg + sp.chunk;
    d.m = n_chunk;
    d.Hkv = a.Hkv;
    d.str_k = a.str_k;
    d.out_str_k = stg + sp.str;
    d.Hs = a.Hs;
    d.S = a.S;
    d.R = a.R;
  }
  // the prefix of every retrieval head read back as bf16 rows (values only with pre-RoPE
  // keys), then, with pre-RoPE keys, every key the chunk attends to turned at its position
  if (a.Hr > 0 && sp.c_max > 0 && launch_dequant_kv4(d, c->cfg.head_dim, stream) != 0)
    return DUO_ERR_HIP;
  if (rope && launch_rope_stage(d, c->cfg.head_dim, stream) != 0) return DUO_ERR_HIP;
  // the chunk's and the streaming caches' values as fp16 copies too (the prefix values were
  // read back in fp16), so the prefill kernel reads every V tile as it is
  V16StageArgs v16;
  std::memset(&v16, 0, sizeof(v16));
  v16.v = a.v;
  v16.str_v = a.str_v;
  v16.out_chunk = stg + sp.cv;
  v16.out_str = stg + sp.sv;
  v16.b0 = a.b0;
  v16.nb = a.nb;
  v16.Hr = 0;  // no prefix groups
  v16.Hs = a.Hs;
  v16.SR = a.S + a.R;
  v16.m = n_chunk;
  v16.Hkv = a.Hkv;
  v16.D = c->cfg.head_dim;
  if (launch_v16_stage(v16, stream) != 0) return DUO_ERR_HIP;
  a.full_k = stg;
  a.full_v = stg + sp.pv;
  a.cap = sp.c_max;
  a.full_b0 = a.b0;
  a.v16 = 1;
  a.vcap = sp.c_max;
  a.v_b0 = a.b0;
  a.v = stg + sp.cv;
  a.str_v = stg + sp.sv;
  if (rope) {
    a.k = stg + sp.chunk;
    a.str_k = stg + sp.str;
  }
  const int group = c->cfg.num_q_heads / c->cfg.num_kv_heads;
  return launch_status(launch_prefill(a, c->cfg.dtype, c->cfg.head_dim, group, stream,
                                      next_marks(c, DUO_TIMING_PREFILL)));
}

duo_status duo_attn_gate_mixed(duo_cache* c, int32_t layer, int32_t seq, const void* q,
                               const void* k, const void* v, int32_t n_chunk,
                               const float* alpha, void* out, void* stream) {
  if (!layer_ok(c, layer) || seq < -1 || seq >= c->cfg.batch || n_chunk < 0 || !alpha)
    return DUO_ERR_INVALID;
  const LayerInfo& li = c->layers[layer];
  if (li.n_ret != c->cfg.num_kv_heads) return DUO_ERR_INVALID;  // every head needs a full cache
  for (int32_t j = 0; j < c->cfg.num_kv_heads; ++j)
    if (!(alpha[j] >= 0.f && alpha[j] <= 1.f)) return DUO_ERR_INVALID;
  if (n_chunk == 0) return DUO_OK;
  PrefillArgs a;
  duo_status st = prefill_args(c, layer, seq, q, k, v, n_chunk, out, nullptr, a);
  if (st != DUO_OK) return st;
  const int group = c->cfg.num_q_heads / c->cfg.num_kv_heads;
  // full attention of every head into out (the layer is all retrieval heads)
  a.chunk_mode = 0;
  st = launch_status(launch_prefill(a, c->cfg.dtype, c->cfg.head_dim, group, stream, {}));
  if (st != DUO_OK) return st;
  // sink + recent attention of every head over the same full caches, blended into out
  PrefillArgs s = a;
  s.Hr = 0;
  s.Hs = c->cfg.num_kv_heads;
  for (int32_t j = 0; j < s.Hs; ++j) s.str_kv[j] = (uint8_t)j;
  s.nsplit = 1;
  s.mixed = 1;
  for (int32_t j = 0; j < s.Hs; ++j) s.alpha[j] = alpha[j];
  return launch_status(launch_prefill(s, c->cfg.dtype, c->cfg.head_dim, group, stream, {}));
}

duo_status duo_timing_enable(duo_cache* c, int32_t max_records) {
  if (!c || max_records < 0 || max_records > kMaxTimingRecords) return DUO_ERR_INVALID;
  for (duo_cache::Timer& t : c->timers) {
    destroy_events(&t.ev);
    t.used = 0;
    if (max_records > 0 && create_events(2 * max_records, &t.ev) != 0) {
      for (duo_cache::Timer& u : c->timers) destroy_events(&u.ev);
      return DUO_ERR_HIP;
    }
  }
  return DUO_OK;
}

duo_status duo_timing_read(duo_cache* c, int32_t kind, double* total_ms, int32_t* records) {
  if (!c || kind < DUO_TIMING_DECODE || kind > DUO_TIMING_PREFILL || !total_ms || !records)
    return DUO_ERR_INVALID;
  duo_cache::Timer& t = c->timers[kind];
  *records = t.used;
  if (pairs_elapsed_ms(t.ev, t.used, total_ms) != 0) return DUO_ERR_HIP;
  t.used = 0;
  return DUO_OK;
}

duo_status duo_read_probe(const void* src, uint64_t bytes, uint32_t* flag, int32_t blocks,
                          void* stream) {
  if (!src || !flag || !aligned16(src) || !aligned4(flag) || bytes == 0 || bytes % 16 != 0 ||
      blocks < 0 || blocks > (1 << 20))
    return DUO_ERR_INVALID;
  return launch_read_probe(src, bytes, flag, blocks, stream) != 0 ? DUO_ERR_HIP : DUO_OK;
}

duo_status duo_slot_positions(duo_cache* c, int32_t layer, int32_t* host_out, void* stream) {
  if (!layer_ok(c, layer) || !host_out) return DUO_ERR_INVALID;
  const uint64_t SR = (uint64_t)c->cfg.sink + c->cfg.recent;
  const LayerPtrs p = layer_ptrs(c, layer);
  if (copy_d2h_sync(host_out, p.slot_pos, (uint64_t)c->cfg.batch * SR * 4, stream) != 0)
    return DUO_ERR_HIP;
  return DUO_OK;
}

}  // extern "C"
