// Internal declarations shared by the host logic (duo_host.cpp, plain C++) and the HIP
// kernel launchers. Nothing here is part of the C ABI.
#pragma once

#include <cstdint>
#include <vector>

#include "../../include/duo.h"

namespace duo {

constexpr int kMaxKvHeads = 64;
constexpr int kMaxBatch = 512;
constexpr int kDefaultSplits = 256;
constexpr int kMaxSplits = 1024;
constexpr int kDefaultPrefillTiles = 2048;
constexpr int kMaxPrefillTiles = 65536;
constexpr int kPrefillRows = 128;      // query rows per prefill block (and per partial tile)
constexpr int kPrefillTileRows = 128;  // rows of the workspace unit counted by prefill_tiles
constexpr uint64_t kAlign = 256;
constexpr int kMaxTimingRecords = 1 << 16;  // event pairs per kernel timer

// Byte geometry of one retrieval head's K (or V) region in a 4-bit or 8-bit cache: codes,
// then the parameter block, then the residual group in bf16 (layout in duo.h).
constexpr int kQ4Group = DUO_KV4_GROUP;
struct Q4Geom {
  uint64_t codes;   // bytes of codes (128 G rows of D * bits / 8)
  uint64_t params;  // bytes of the parameter block
  uint64_t resid;   // bytes of the residual group
  uint64_t stride;  // bytes per head
};
inline Q4Geom q4_geom(uint64_t cap, uint64_t D, uint64_t bits) {
  const uint64_t groups = (cap + kQ4Group - 1) / kQ4Group;
  Q4Geom g;
  g.codes = groups * kQ4Group * D * bits / 8;
  const uint64_t kp = groups * 2 * D * 2, vp = groups * kQ4Group * 4;  // bf16 parameters
  g.params = kp > vp ? kp : vp;
  g.resid = (uint64_t)kQ4Group * D * 2;
  g.stride = g.codes + g.params + g.resid;
  return g;
}

// cos/sin tables of a cache with pre-RoPE keys (cfg.rope_theta > 0), at layout.rope_off;
// f_i = theta^(-2 i / D) is the frequency of channel pair (i, i + D / 2):
//   tau16: [128] rows of D / 2 + 4 words, the decode kernel's LDS image: for each block of 8
//          pairs b, 4 words of fp16 (cos, cos) then 4 of (sin, sin) of pairs (8 b + w, 8 b + w + 4)
//          at angle tau f_i (w = 0..3), then 4 padding words that keep the LDS reads of
//          neighbouring rows on different banks;
//   base:  float [nbase][D / 2][2], (cos, sin) of 128 g f_i, nbase = cap / 128 + 1.
// A position t turns by base[t / 128] composed with tau[t % 128].
struct RopeGeom {
  uint64_t tau16, base, bytes;  // offsets from layout.rope_off, total bytes
  int32_t nbase;
};
inline RopeGeom rope_geom(uint64_t cap, uint64_t D) {
  auto up = [](uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; };
  RopeGeom g;
  g.nbase = (int32_t)(cap / kQ4Group + 1);
  g.tau16 = 0;
  g.base = up((uint64_t)kQ4Group * (D / 2 + 4) * 4);
  g.bytes = g.base + up((uint64_t)g.nbase * D * 4);
  return g;
}

// Per-layer head partition. For KV head j: cls_idx[j] >= 0 is its index among the layer's
// retrieval heads; cls_idx[j] < 0 encodes streaming index -(cls_idx[j] + 1).
struct LayerInfo {
  int32_t n_ret = 0, n_str = 0;
  uint64_t full_off = 0;  // bytes from layout.full_k_off (same offset in the V region)
  uint64_t str_off = 0;   // bytes from layout.str_k_off (same offset in the V region)
  int16_t cls_idx[kMaxKvHeads];
  uint8_t ret_kv[kMaxKvHeads];  // retrieval index -> KV head
  uint8_t str_kv[kMaxKvHeads];  // streaming index -> KV head
};

// ---------------------------------------------------------------------------------------
// Kernel argument blocks (plain data, passed by value)
// ---------------------------------------------------------------------------------------

struct ResetArgs {
  int32_t* slot_pos;   // [n_slot] -> -1
  int64_t n_slot;
  int32_t* seq_len;    // [n_len] -> 0
  int64_t n_len;
};

struct SetLenArgs {
  int32_t* slot_pos;  // this layer: [B][S+R]
  int32_t* seq_len;   // this layer: [B]
  int32_t B, S, R;
  int32_t n[kMaxBatch];
};

struct AppendArgs {
  const void* k;  // [nb][m][Hkv][D]
  const void* v;
  void* full_k;   // this layer: [B][Hr][cap][D]
  void* full_v;
  void* str_k;    // this layer: [B][Hs][S+R][D]
  void* str_v;
  int32_t* slot_pos;  // this layer: [B][S+R]
  int32_t* seq_len;   // this layer: [B]
  int32_t b0, nb, m, Hkv, Hr, Hs, cap, S, R;
  int32_t row_bytes;  // D * element size
  int32_t qbits;      // 4- or 8-bit full caches (else 0): append_kernel leaves retrieval
                      // heads to the quantizing append
  int64_t q4_stride, q4_params, q4_resid;  // Q4Geom: head stride, parameter and residual offsets
  int32_t q4_mid;     // complete groups of the widest sequence that need no residual rows
  int16_t cls_idx[kMaxKvHeads];
  uint8_t ret_kv[kMaxKvHeads];
  int32_t n_old[kMaxBatch];  // lengths before the append, for sequences b0 .. b0+nb-1
};

struct DecodeArgs {
  const void* q;   // [B][Hq][D]
  void* out;       // [B][Hq][D]
  float* lse;      // [B][Hq] or null
  const void* full_k;
  const void* full_v;
  const void* str_k;
  const void* str_v;
  float* part_o;           // [B][Hq][max_splits][D]
  float* part_ml;          // [B][Hq][max_splits][2]
  const void* new_k;       // fused step: the appended token [B][Hkv][D], else null
  const void* new_v;
  int32_t* slot_pos;       // fused step: this layer's slot table [B][S+R] and lengths [B]
  int32_t* seq_len;
  int32_t B, Hq, Hkv, Hr, Hs, cap, S, R, nsplit, max_splits;
  float scale_log2;        // softmax scale * log2(e)
  int32_t out_f32;
  int32_t qbits;           // full caches in 4 or 8 bits (Q4Geom offsets below), else 0
  int64_t q4_stride, q4_params, q4_resid;
  int32_t nss;             // blocks per streaming head (4-bit kernel; 1 otherwise)
  const float* rope_base;      // pre-RoPE keys (4-bit kernel): RopeGeom base and tau16
  const uint32_t* rope_tau16;  // tables, else null
  // KV head of each retrieval / streaming index, as 32-bit words: a block reads its entry with
  // a scalar load (a byte would take a vector load, whose latency delays every first load)
  int32_t ret_kv[kMaxKvHeads];
  int32_t str_kv[kMaxKvHeads];
  int32_t n[kMaxBatch];    // length of every sequence, the fused step's token included
};

struct PrefillArgs {
  const void* q;   // [nb][m][Hq][D]
  const void* k;   // [nb][m][Hkv][D]
  const void* v;
  void* out;       // [nb][m][Hq][D]
  float* lse;      // [nb][m][Hq] or null
  const void* full_k;
  const void* full_v;
  const void* str_k;
  const void* str_v;
  const int32_t* slot_pos;  // this layer: [B][S+R]
  float* part_o;            // retrieval split-K partials [item][split][128][D] (nsplit > 1)
  float* part_ml;           // [item][split][128][2]
  int32_t b0, nb, m, Hq, Hkv, Hr, Hs, cap, S, R;
  int32_t n_qt;             // query tiles of 128 rows per (sequence, KV head)
  int32_t nsplit;           // key-range splits of every retrieval query tile
  float scale_log2;
  int32_t out_f32;
  int32_t chunk_mode;       // streaming heads see the whole cache plus the chunk causally
  // Gate-mixed pass (its own kernel variant): streaming blocks read the full caches under
  // the sink + recent window and write alpha[j] * out + (1 - alpha[j]) * result.
  int32_t mixed;
  int32_t full_heads;       // full caches per sequence of this layer
  int32_t full_b0;          // sequence whose full caches start at full_k / full_v (0, or b0
                            // when they are a staging copy of sequences b0 .. b0 + nb - 1)
  // fp16 values (duo_attn_prefill_staged on a bf16 cache): v, str_v and the retrieval
  // prefix in full_v are fp16 copies, the prefix laid out [nb][Hr][vcap][D] from sequence
  // v_b0; the kernel then reads V tiles as they are instead of converting them in LDS
  int32_t v16, vcap, v_b0;
  float alpha[kMaxKvHeads];
  int16_t cls_idx[kMaxKvHeads];
  uint8_t ret_kv[kMaxKvHeads];
  uint8_t str_kv[kMaxKvHeads];
  int32_t c0[kMaxBatch];  // chunk start (current length) of each sequence b0 .. b0+nb-1
};

// A pair of HIP events (hipEvent_t, or null) that a launcher records on its stream right
// before and right after the main kernel of its family (kernel timing).
struct KernelMarks {
  void* begin = nullptr;
  void* end = nullptr;
};

// Launchers (one translation unit per kernel family). They return a hipError_t value as int.
int launch_reset(const ResetArgs& a, void* stream);
// Fills the RopeGeom tables at `tables` for head dimension D and base theta.
int launch_rope_tables(char* tables, int32_t D, int32_t nbase, double theta, void* stream);
int launch_append(const AppendArgs& a, int dtype, void* stream);
int launch_append_kv4(const AppendArgs& a, int head_dim, void* stream);
// Read-back of a layer's 4- or 8-bit retrieval caches into bf16 rows (kv4.hip): for each
// sequence b0 + i and retrieval head r, tokens 0 .. c0[i] - 1 into out_k / out_v
// [nb][Hr][cap_s][D], complete groups as bf16(float32(c * scale + zero)), residual rows copied.
struct DequantArgs {
  const void* full_k;  // this layer's quantized regions
  const void* full_v;
  void* out_k;         // staging rows, [nb][Hr][cap_s][D] bf16 each
  void* out_v;
  int64_t q4_stride, q4_params, q4_resid;  // Q4Geom of the regions
  int32_t qbits, b0, nb, Hr, cap_s;
  int32_t v_f16;       // value rows in fp16 (each the bf16 read-back, converted exactly)
  int32_t c0[kMaxBatch];
  // Pre-RoPE caches (rope_base set): launch_dequant_kv4 reads back the values only, and
  // launch_rope_stage writes every key the chunk attends to, turned at its position: the
  // retrieval prefix into out_k, the chunk's keys into out_chunk_k, the held streaming slots
  // into out_str_k.
  const float* rope_base;  // RopeGeom base table: (cos, sin) of 128 g f_i, float32
  float log2_theta;        // f_i = 2^(-(2 i / D) log2_theta)
  const void* chunk_k;     // the chunk's keys as given, [nb][m][Hkv][D]
  void* out_chunk_k;       // [nb][m][Hkv][D]
  const void* str_k;       // this layer's streaming keys, [B][Hs][S + R][D]
  void* out_str_k;         // [B][Hs][S + R][D], rows of sequences b0 .. b0 + nb - 1
  int32_t m, Hkv, Hs, S, R;
};
int launch_dequant_kv4(const DequantArgs& a, int head_dim, void* stream);

// fp16 copies of the values a bf16 prefill chunk reads (prefill.hip): the retrieval prefix
// rows [0, c0) of sequences b0 .. b0 + nb - 1 into out_pv ([nb][Hr][c_max][D]), the chunk's
// values v ([nb][m][Hkv][D]) into out_chunk, and the streaming values of those sequences into
// out_str at their places in [B][Hs][S + R][D]. Every element is converted exactly as the
// prefill kernel converts a V tile in LDS.
struct V16StageArgs {
  const void* full_v;  // this layer's retrieval values, [B][Hr][cap][D]
  const void* v;
  const void* str_v;   // this layer's streaming values, [B][Hs][S + R][D]
  void* out_pv;
  void* out_chunk;
  void* out_str;
  int64_t cap;
  int32_t c_max, b0, nb, Hr, Hs, SR, m, Hkv, D;
  int32_t c0[kMaxBatch];
};
int launch_v16_stage(const V16StageArgs& a, void* stream);
int launch_rope_stage(const DequantArgs& a, int head_dim, void* stream);
int launch_set_lengths(const SetLenArgs& a, void* stream);
int launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group, void* stream,
                  const KernelMarks& marks);
int launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int group, void* stream,
                   const KernelMarks& marks);

// Block permutation (reorder.hip): dst[o][i] = src[o][order[i]], blocks of 16-byte chunks.
constexpr int kMaxPermuteBlocks = 1024;
struct PermuteArgs {
  const void* src;
  void* dst;
  uint32_t n_chunks;        // outer * n_blocks * chunks_per_block (< 2^31)
  uint32_t chunks_per_block;
  uint32_t n_blocks;
  uint16_t order[kMaxPermuteBlocks];
};
int launch_permute(const PermuteArgs& a, void* stream);

// Streaming-read probe (probe.hip); blocks <= 0 selects two per compute unit.
int launch_read_probe(const void* src, uint64_t bytes, uint32_t* flag, int blocks, void* stream);

// HIP events of the kernel timers (cache_kernels.hip); hipError_t values as int.
int create_events(int n, std::vector<void*>* out);
void destroy_events(std::vector<void*>* ev);
int record_event(void* event, void* stream);
// Sum of the elapsed times of the pairs (ev[2i], ev[2i+1]), i < pairs, after waiting for
// the last one.
int pairs_elapsed_ms(const std::vector<void*>& ev, int pairs, double* total_ms);
// Static split-K scratch of duo_attn_decode_noalloc (decode.hip): its size, and the device
// address of the current device's copy, looked up on the first call on each device (a
// hipError_t value as int).
constexpr uint64_t kScratchBytes = 8ull << 20;
constexpr int kMaxDevices = 64;
int static_scratch(void** ptr);
// Decode blocks of this variant (the quantized kernel of qbits 4 or 8, its pre-RoPE form when
// rope) that are resident on the device at once, counting at most max_per_cu (1 or 2) per CU
// (512 if unknown): the size of one round of splits.
int decode_resident_blocks(int dtype, int head_dim, int group, int qbits, bool rope,
                           int max_per_cu);
// Prefill blocks of this variant that are resident on the device at once (512 if unknown).
int prefill_resident_blocks(int head_dim, int group);

// Host-side helpers (duo_host.cpp)
int element_size(int32_t dtype);
duo_status check_config(const duo_config* cfg);
duo_status build_layout(const duo_config* cfg, duo_layout* lay, std::vector<LayerInfo>* layers);
int choose_decode_splits(int32_t n_max, int32_t batch, int32_t n_ret, int32_t n_str,
                         int32_t max_splits, int32_t resident_blocks);
int choose_prefill_splits(int32_t nb, int32_t m, int32_t c_max, int32_t c_sum, int32_t n_ret,
                          int32_t n_str, int32_t sink, int32_t recent, int32_t group,
                          int32_t prefill_tiles, int32_t resident_blocks, bool chunk_mode);

}  // namespace duo

// The opaque cache object behind duo_cache*.
struct duo_cache {
  duo_config cfg;                       // retrieval_mask points into `mask`
  std::vector<uint8_t> mask;            // [L][Hkv]
  std::vector<duo::LayerInfo> layers;   // [L]
  duo_layout lay;
  char* arena = nullptr;
  std::vector<int32_t> lens;            // host mirror [L][B]
  int32_t force_splits = 0;
  int esize = 0;
  float scale = 0.f;
  // kernel timers, indexed by duo_timing_kind: 2 * capacity events and the pairs used
  struct Timer {
    std::vector<void*> ev;
    int32_t used = 0;
  } timers[2];
  ~duo_cache() {
    for (Timer& t : timers) duo::destroy_events(&t.ev);
  }
};
