// One-time preprocessing before deployment: the binarization of the trained gates into the
// retrieval mask, the head order that puts retrieval heads first, and the host side of the
// weight reordering (argument checks; the copy runs in reorder.hip).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <numeric>
#include <vector>

#include "duo_internal.h"

extern "C" {

duo_status duo_binarize_gates(const float* alpha, int32_t n_layers, int32_t n_kv_heads,
                              double ratio, uint8_t* mask_out, float* tau_out,
                              int32_t* n_retrieval_out) {
  if (!alpha || !mask_out || n_layers < 1 || n_kv_heads < 1) return DUO_ERR_INVALID;
  if (!(ratio >= 0.0 && ratio <= 1.0)) return DUO_ERR_INVALID;
  const int64_t n = (int64_t)n_layers * n_kv_heads;
  if (n > (int64_t)1 << 30) return DUO_ERR_INVALID;
  for (int64_t i = 0; i < n; ++i)
    if (!std::isfinite(alpha[i])) return DUO_ERR_INVALID;
  // count nearest to ratio * n, halves up (the product rounded to double first)
  int64_t k = (int64_t)std::floor(ratio * (double)n + 0.5);
  k = std::min<int64_t>(std::max<int64_t>(k, 0), n);
  // rank heads by decreasing gate; the flat index layer * H + head breaks ties in
  // (layer, head) order
  std::vector<int64_t> rank(n);
  std::iota(rank.begin(), rank.end(), 0);
  std::stable_sort(rank.begin(), rank.end(),
                   [&](int64_t x, int64_t y) { return alpha[x] > alpha[y]; });
  for (int64_t i = 0; i < n; ++i) mask_out[i] = 0;
  for (int64_t i = 0; i < k; ++i) mask_out[rank[i]] = 1;
  if (tau_out) *tau_out = k < n ? alpha[rank[k]] : -std::numeric_limits<float>::infinity();
  if (n_retrieval_out) *n_retrieval_out = (int32_t)k;
  return DUO_OK;
}

duo_status duo_head_order(const uint8_t* mask, int32_t n_kv_heads, int32_t group,
                          int32_t* kv_order_out, int32_t* q_order_out) {
  if (!mask || !kv_order_out || n_kv_heads < 1 || n_kv_heads > duo::kMaxPermuteBlocks ||
      group < 1 || (int64_t)n_kv_heads * group > ((int64_t)1 << 30))
    return DUO_ERR_INVALID;
  int32_t slot = 0;
  for (int pass = 0; pass < 2; ++pass)  // retrieval heads, then streaming heads
    for (int32_t j = 0; j < n_kv_heads; ++j)
      if ((mask[j] != 0) == (pass == 0)) kv_order_out[slot++] = j;
  if (q_order_out)
    for (int32_t i = 0; i < n_kv_heads; ++i)
      for (int32_t g = 0; g < group; ++g)
        q_order_out[i * group + g] = kv_order_out[i] * group + g;
  return DUO_OK;
}

duo_status duo_permute_blocks(const void* src, void* dst, int64_t outer, int32_t n_blocks,
                              int64_t block_bytes, const int32_t* order, void* stream) {
  if (!src || !dst || !order || outer < 0 || n_blocks < 1 ||
      n_blocks > duo::kMaxPermuteBlocks || block_bytes < 16 || block_bytes % 16 != 0)
    return DUO_ERR_INVALID;
  if ((uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0) return DUO_ERR_INVALID;
  // below 2^31 chunks, so that the kernel's 32-bit chunk indices (plus a few grid strides)
  // never wrap
  const uint64_t cpb = (uint64_t)block_bytes / 16;
  constexpr uint64_t kMaxChunks = (uint64_t)1 << 31;
  if (cpb >= kMaxChunks || (outer > 0 && cpb * (uint64_t)n_blocks >= kMaxChunks / (uint64_t)outer))
    return DUO_ERR_INVALID;
  const uint64_t n_chunks = (uint64_t)outer * n_blocks * cpb;
  if (n_chunks >= kMaxChunks) return DUO_ERR_INVALID;
  std::vector<uint8_t> seen(n_blocks, 0);
  for (int32_t i = 0; i < n_blocks; ++i) {
    if (order[i] < 0 || order[i] >= n_blocks || seen[order[i]]) return DUO_ERR_INVALID;
    seen[order[i]] = 1;
  }
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst, bytes = (uintptr_t)(n_chunks * 16);
  if (n_chunks > 0 && s0 < d0 + bytes && d0 < s0 + bytes) return DUO_ERR_INVALID;
  if (n_chunks == 0) return DUO_OK;
  duo::PermuteArgs a;
  a.src = src;
  a.dst = dst;
  a.n_chunks = (uint32_t)n_chunks;
  a.chunks_per_block = (uint32_t)cpb;
  a.n_blocks = (uint32_t)n_blocks;
  for (int32_t i = 0; i < duo::kMaxPermuteBlocks; ++i)
    a.order[i] = (uint16_t)(i < n_blocks ? order[i] : 0);
  return duo::launch_permute(a, stream) == 0 ? DUO_OK : DUO_ERR_HIP;
}

}  // extern "C"
