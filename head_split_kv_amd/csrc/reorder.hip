// Block permutation of a device tensor: the one-time reordering of the Q, K, V and output
// projection weights that puts the retrieval heads first (explainer, "Head Reordering
// Preprocessing"). A pure copy, bound by HBM bandwidth: every byte is read once and written
// once, 16 bytes per lane, consecutive lanes on consecutive destination chunks so that both
// the loads (inside a block) and the stores are coalesced.
#include <hip/hip_runtime.h>

#include "duo_internal.h"

namespace duo {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // chunks in flight per lane

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

__global__ void __launch_bounds__(kThreads) permute_kernel(PermuteArgs a) {
  const uint32_t stride = gridDim.x * kThreads;
  const u32x4_t* src = (const u32x4_t*)a.src;
  u32x4_t* dst = (u32x4_t*)a.dst;
  const uint32_t cpb = a.chunks_per_block;
  for (uint32_t base = blockIdx.x * kThreads + threadIdx.x; base < a.n_chunks;
       base += stride * kUnroll) {
    u32x4_t v[kUnroll];
    uint32_t at[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t c = base + u * stride;  // destination chunk
      at[u] = c;
      if (c < a.n_chunks) {
        const uint32_t row = c / cpb;           // o * n_blocks + i
        const uint32_t w = c - row * cpb;
        const uint32_t o = row / a.n_blocks;
        const uint32_t i = row - o * a.n_blocks;
        const uint32_t s = (o * a.n_blocks + a.order[i]) * cpb + w;
        v[u] = __builtin_nontemporal_load(src + s);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (at[u] < a.n_chunks) __builtin_nontemporal_store(v[u], dst + at[u]);
  }
}

}  // namespace

int launch_permute(const PermuteArgs& a, void* stream) {
  if (a.n_chunks == 0) return 0;
  const uint64_t per_block = (uint64_t)kThreads * kUnroll;
  uint64_t grid = (a.n_chunks + per_block - 1) / per_block;
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace duo
