// Host-side logic of libduo: configuration checks, the arena layout, the host object and the
// KV byte model. Plain C++ with no HIP dependency; every function here runs without a GPU.
#include <cmath>
#include <cstring>
#include <new>

#include "duo_internal.h"

namespace duo {

int element_size(int32_t dtype) {
  switch (dtype) {
    case DUO_F32: return 4;
    case DUO_BF16: return 2;
    default: return 0;
  }
}

static uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

duo_status check_config(const duo_config* cfg) {
  if (!cfg) return DUO_ERR_INVALID;
  if (cfg->num_layers < 1 || cfg->num_layers > 4096) return DUO_ERR_INVALID;
  if (cfg->batch < 1 || cfg->batch > kMaxBatch) return DUO_ERR_INVALID;
  if (cfg->num_kv_heads < 1 || cfg->num_kv_heads > kMaxKvHeads) return DUO_ERR_INVALID;
  if (cfg->num_q_heads < cfg->num_kv_heads || cfg->num_q_heads % cfg->num_kv_heads != 0)
    return DUO_ERR_INVALID;
  if (cfg->head_dim < 1) return DUO_ERR_INVALID;
  if (cfg->sink < 0 || cfg->recent < 1) return DUO_ERR_INVALID;
  if ((int64_t)cfg->sink + cfg->recent > (1 << 20)) return DUO_ERR_INVALID;
  if (cfg->capacity < 1) return DUO_ERR_INVALID;
  if (cfg->max_splits < 0 || cfg->max_splits > kMaxSplits) return DUO_ERR_INVALID;
  if (cfg->prefill_tiles < 0 || cfg->prefill_tiles > kMaxPrefillTiles) return DUO_ERR_INVALID;
  if (!cfg->retrieval_mask) return DUO_ERR_INVALID;
  if (cfg->streaming_prefill != DUO_PREFILL_WINDOW && cfg->streaming_prefill != DUO_PREFILL_CHUNK)
    return DUO_ERR_INVALID;
  if (cfg->kv_bits != 0 && cfg->kv_bits != 16 && cfg->kv_bits != 4 && cfg->kv_bits != 8)
    return DUO_ERR_INVALID;
  if (element_size(cfg->dtype) == 0 || element_size(cfg->out_dtype) == 0)
    return DUO_ERR_INVALID;
  if (!(std::isfinite(cfg->softmax_scale))) return DUO_ERR_INVALID;
  if (!(std::isfinite(cfg->rope_theta))) return DUO_ERR_INVALID;
  // Built variants: head_dim 64/128, group 1/2/4/8, out either fp32 or the input dtype.
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return DUO_ERR_UNSUPPORTED;
  const int g = cfg->num_q_heads / cfg->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return DUO_ERR_UNSUPPORTED;
  if (cfg->out_dtype != DUO_F32 && cfg->out_dtype != cfg->dtype) return DUO_ERR_UNSUPPORTED;
  const bool quantized = cfg->kv_bits == 4 || cfg->kv_bits == 8;
  if (quantized && cfg->dtype != DUO_BF16) return DUO_ERR_UNSUPPORTED;
  // a quantized retrieval head decodes into its splits' partials plus one for the residual rows
  if (quantized && cfg->max_splits == 1) return DUO_ERR_INVALID;
  // pre-RoPE keys: the rotation is built into the quantized caches' decode only
  if (cfg->rope_theta > 0.f && !quantized) return DUO_ERR_UNSUPPORTED;
  return DUO_OK;
}

duo_status build_layout(const duo_config* cfg, duo_layout* lay, std::vector<LayerInfo>* layers) {
  duo_status st = check_config(cfg);
  if (st != DUO_OK) return st;
  const uint64_t es = (uint64_t)element_size(cfg->dtype);
  const uint64_t L = cfg->num_layers, B = cfg->batch, Hkv = cfg->num_kv_heads;
  const uint64_t Hq = cfg->num_q_heads, D = cfg->head_dim;
  const uint64_t cap = cfg->capacity, SR = (uint64_t)cfg->sink + cfg->recent;
  const uint64_t splits = cfg->max_splits ? cfg->max_splits : kDefaultSplits;

  // Sizes in long double first so that absurd configurations are rejected, not wrapped.
  long double full_total = 0, str_total = 0;
  if (layers) layers->assign(L, LayerInfo{});
  uint64_t full_off = 0, str_off = 0;
  for (uint64_t l = 0; l < L; ++l) {
    int nr = 0, ns = 0;
    LayerInfo info;
    for (uint64_t j = 0; j < Hkv; ++j) {
      if (cfg->retrieval_mask[l * Hkv + j]) {
        info.cls_idx[j] = (int16_t)nr;
        info.ret_kv[nr++] = (uint8_t)j;
      } else {
        info.cls_idx[j] = (int16_t)(-(ns + 1));
        info.str_kv[ns++] = (uint8_t)j;
      }
    }
    info.n_ret = nr;
    info.n_str = ns;
    const long double per_head = (cfg->kv_bits == 4 || cfg->kv_bits == 8)
                                     ? (long double)q4_geom(cap, D, cfg->kv_bits).stride
                                     : (long double)cap * D * es;
    const long double fb = (long double)B * nr * per_head;
    const long double sb = (long double)B * ns * SR * D * es;
    full_total += fb;
    str_total += sb;
    if (full_total > 4.0e18L || str_total > 4.0e18L) return DUO_ERR_INVALID;
    info.full_off = full_off;
    info.str_off = str_off;
    full_off += align_up((uint64_t)fb);
    str_off += align_up((uint64_t)sb);
    if (layers) (*layers)[l] = info;
  }
  duo_layout out{};
  uint64_t off = 0;
  out.full_k_off = off;  off = align_up(off + full_off);
  out.full_v_off = off;  off = align_up(off + full_off);
  out.str_k_off = off;   off = align_up(off + str_off);
  out.str_v_off = off;   off = align_up(off + str_off);
  out.slot_pos_off = off; off = align_up(off + L * B * SR * 4);
  out.seq_len_off = off;  off = align_up(off + L * B * 4);
  out.workspace_off = off;
  const uint64_t ptiles = cfg->prefill_tiles ? cfg->prefill_tiles : kDefaultPrefillTiles;
  const uint64_t ws_decode = align_up(B * Hq * splits * D * 4) + align_up(B * Hq * splits * 2 * 4);
  const uint64_t ws_prefill = align_up(ptiles * kPrefillTileRows * D * 4) +
                              align_up(ptiles * kPrefillTileRows * 2 * 4);
  const uint64_t ws = ws_decode > ws_prefill ? ws_decode : ws_prefill;
  out.workspace_bytes = ws;
  off = align_up(off + ws);
  if (cfg->rope_theta > 0.f) {
    out.rope_off = off;
    out.rope_bytes = rope_geom(cap, D).bytes;
    off = align_up(off + out.rope_bytes);
  }
  out.arena_bytes = off;
  if (lay) *lay = out;
  return DUO_OK;
}

int choose_decode_splits(int32_t n_max, int32_t batch, int32_t n_ret, int32_t n_str,
                         int32_t max_splits, int32_t resident_blocks) {
  // One round of resident blocks: the streaming items take one block each and the retrieval
  // heads share the rest evenly, so no block waits for a second round; no split is made
  // shorter than kMinTokens (each split costs one partial write and one merge read).
  constexpr int64_t kMinTokens = 128;
  if (n_ret <= 0 || n_max <= 0) return 1;
  const int64_t ret_items = (int64_t)batch * n_ret;
  int64_t avail = (int64_t)resident_blocks - (int64_t)batch * n_str;
  if (avail < ret_items) avail = ret_items;
  int64_t s = avail / ret_items;
  const int64_t by_len = (n_max + kMinTokens - 1) / kMinTokens;
  if (s > by_len) s = by_len;
  if (s < 1) s = 1;
  if (s > max_splits) s = max_splits;
  return (int)s;
}

int choose_prefill_splits(int32_t nb, int32_t m, int32_t c_max, int32_t c_sum, int32_t n_ret,
                          int32_t n_str, int32_t sink, int32_t recent, int32_t group,
                          int32_t prefill_tiles, int32_t resident_blocks, bool chunk_mode) {
  // Retrieval query tiles see the whole cache prefix, streaming ones a constant window
  // (or, chunk-granular, the S + R cache rows and the chunk up to the tile).
  // Cut the retrieval key ranges so that the heaviest piece is about the size of a
  // streaming tile or of one resident round's share of the work, whichever is larger (half a
  // share took 2-3 % longer on the 32K prompt in 4K chunks: more partials and shorter blocks).
  constexpr int64_t kBN = 64;
  if (n_ret <= 0 || m <= 0) return 1;
  const int64_t qpb = kPrefillRows / group;
  const int64_t n_qt = (m + qpb - 1) / qpb;
  const int64_t chunk_tiles_avg = ((int64_t)m + 2 * kBN - 1) / (2 * kBN);
  const int64_t t_ret_max = (c_max + kBN - 1) / kBN + (m + kBN - 1) / kBN;
  const int64_t t_ret_avg = ((int64_t)c_sum / (nb > 0 ? nb : 1) + kBN - 1) / kBN + chunk_tiles_avg;
  const int64_t sr = (int64_t)sink + recent;
  int64_t t_str = (c_max > 0 ? (sr + kBN - 1) / kBN : 0) + (recent + qpb + kBN - 1) / kBN + 1;
  if (t_str > (m + kBN - 1) / kBN + (sr + kBN - 1) / kBN) t_str = (m + kBN - 1) / kBN + (sr + kBN - 1) / kBN;
  if (chunk_mode) t_str = (c_max > 0 ? (sr + kBN - 1) / kBN : 0) + chunk_tiles_avg;
  const int64_t work = (int64_t)nb * n_qt * ((int64_t)n_ret * t_ret_avg + (int64_t)n_str * t_str);
  int64_t target = work / (int64_t)(resident_blocks > 0 ? resident_blocks : 512);
  if (target < t_str) target = t_str;
  if (target < 4) target = 4;
  int64_t s = (t_ret_max + target - 1) / target;
  if (s > 32) s = 32;
  const int64_t items = (int64_t)nb * n_ret * n_qt;
  const int64_t capacity = (int64_t)prefill_tiles * kPrefillTileRows / kPrefillRows;
  if (s * items > capacity) s = capacity / items;
  if (s < 1) s = 1;
  return (int)s;
}

}  // namespace duo

using namespace duo;

extern "C" {

duo_status duo_layout_query(const duo_config* cfg, duo_layout* out) {
  if (!out) return DUO_ERR_INVALID;
  return build_layout(cfg, out, nullptr);
}

duo_status duo_cache_create(const duo_config* cfg, void* arena, uint64_t arena_bytes,
                            duo_cache** out) {
  if (!out) return DUO_ERR_INVALID;
  *out = nullptr;
  duo_layout lay;
  std::vector<LayerInfo> layers;
  duo_status st = build_layout(cfg, &lay, &layers);
  if (st != DUO_OK) return st;
  if (!arena || ((uintptr_t)arena % kAlign) != 0 || arena_bytes < lay.arena_bytes)
    return DUO_ERR_INVALID;
  duo_cache* c = new (std::nothrow) duo_cache();
  if (!c) return DUO_ERR_INVALID;
  c->cfg = *cfg;
  if (c->cfg.max_splits == 0) c->cfg.max_splits = kDefaultSplits;
  if (c->cfg.prefill_tiles == 0) c->cfg.prefill_tiles = kDefaultPrefillTiles;
  const size_t nm = (size_t)cfg->num_layers * cfg->num_kv_heads;
  c->mask.assign(cfg->retrieval_mask, cfg->retrieval_mask + nm);
  for (auto& x : c->mask) x = x ? 1 : 0;
  c->cfg.retrieval_mask = c->mask.data();
  c->layers = std::move(layers);
  c->lay = lay;
  c->arena = (char*)arena;
  c->lens.assign((size_t)cfg->num_layers * cfg->batch, 0);
  c->esize = element_size(cfg->dtype);
  c->scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale
                                      : (float)(1.0 / std::sqrt((double)cfg->head_dim));
  *out = c;
  return DUO_OK;
}

duo_status duo_cache_destroy(duo_cache* cache) {
  delete cache;
  return DUO_OK;
}

duo_status duo_cache_lengths(const duo_cache* cache, int32_t* host_out) {
  if (!cache || !host_out) return DUO_ERR_INVALID;
  std::memcpy(host_out, cache->lens.data(), cache->lens.size() * sizeof(int32_t));
  return DUO_OK;
}

duo_status duo_kv_bytes(const duo_config* cfg, const int32_t* seq_lens, int32_t layer,
                        uint64_t* full_attn_bytes, uint64_t* duo_bytes) {
  duo_status st = check_config(cfg);
  if (st != DUO_OK) return st;
  if (layer < 0 || layer >= cfg->num_layers || !seq_lens || !full_attn_bytes || !duo_bytes)
    return DUO_ERR_INVALID;
  const uint64_t es = element_size(cfg->dtype), D = cfg->head_dim;
  const uint64_t SR = (uint64_t)cfg->sink + cfg->recent;
  uint64_t nr = 0, ns = 0;
  for (int j = 0; j < cfg->num_kv_heads; ++j)
    (cfg->retrieval_mask[(size_t)layer * cfg->num_kv_heads + j] ? nr : ns) += 1;
  uint64_t full = 0, duo_b = 0;
  for (int b = 0; b < cfg->batch; ++b) {
    if (seq_lens[b] < 0) return DUO_ERR_INVALID;
    const uint64_t n = (uint64_t)seq_lens[b];
    full += 2 * (nr + ns) * n * D * es;
    duo_b += 2 * ns * (n < SR ? n : SR) * D * es;
    if (cfg->kv_bits == 4 || cfg->kv_bits == 8) {
      // complete groups: K and V codes (d * bits / 8 bytes each per token), the keys'
      // per-channel bf16 scale and zero per group, the values' per-token bf16 pair; then the
      // residual
      const uint64_t g = n / kQ4Group, t = g * kQ4Group;
      duo_b += nr * (t * D * cfg->kv_bits / 4 + g * 2 * D * 2 + t * 4 + 2 * (n - t) * D * es);
    } else {
      duo_b += 2 * nr * n * D * es;
    }
  }
  *full_attn_bytes = full;
  *duo_bytes = duo_b;
  return DUO_OK;
}

duo_status duo_set_decode_splits(duo_cache* cache, int32_t splits) {
  if (!cache || splits < 0 || splits > cache->cfg.max_splits) return DUO_ERR_INVALID;
  cache->force_splits = splits;
  return DUO_OK;
}

const char* duo_status_string(duo_status status) {
  switch (status) {
    case DUO_OK: return "DUO_OK";
    case DUO_ERR_INVALID: return "DUO_ERR_INVALID: invalid argument or configuration";
    case DUO_ERR_CAPACITY: return "DUO_ERR_CAPACITY: sequence would exceed the cache capacity";
    case DUO_ERR_UNSUPPORTED: return "DUO_ERR_UNSUPPORTED: head_dim, group size or dtype not built";
    case DUO_ERR_HIP: return "DUO_ERR_HIP: a HIP runtime call or kernel launch failed";
  }
  return "DUO_ERR_UNKNOWN";
}

}  // extern "C"
