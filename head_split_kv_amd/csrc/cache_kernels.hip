// Cache maintenance kernels: reset and append (sink fill, then ring overwrite).
#include <hip/hip_runtime.h>

#include "duo_internal.h"

namespace duo {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) reset_kernel(ResetArgs a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n_slot; i += stride)
    a.slot_pos[i] = -1;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n_len; i += stride)
    a.seq_len[i] = 0;
}

// Streaming slot of token t: sinks take slots 0..S-1, later tokens a ring of R slots after
// them (explainer, "Decoding Procedure", step 4: evict the oldest non-sink token).
__device__ __forceinline__ int32_t slot_of(int32_t t, int32_t S, int32_t R) {
  return t < S ? t : S + (t - S) % R;
}

// A new token t of an append that ends at n_end is still held by a streaming cache iff it
// is a sink or one of the last R tokens. Only those are written, so every slot is written
// at most once per launch.
__device__ __forceinline__ bool survives(int32_t t, int32_t n_end, int32_t S, int32_t R) {
  return t < S || t >= n_end - R;
}

// Lengths of one layer set to n[b], with the slot table rebuilt to match: slot s holds the
// latest token t < n that maps to it (t = s for a sink slot; for a ring slot, the latest
// t <= n - 1 with t = s (mod R), which is one of the last R tokens), or -1.
__global__ void __launch_bounds__(kThreads) set_lengths_kernel(SetLenArgs a) {
  const int32_t SR = a.S + a.R;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.B * SR) return;
  const int32_t b = (int32_t)(i / SR), s = (int32_t)(i % SR), n = a.n[b];
  int32_t pos = -1;
  if (s < a.S) pos = s < n ? s : -1;
  else if (n - 1 >= s) pos = s + a.R * ((n - 1 - s) / a.R);
  a.slot_pos[i] = pos;
  if (s == 0) a.seq_len[b] = n;
}

// RopeGeom tables, one work item per (row, pair) of tau (rows 0..127) and base (rows 128..),
// then the padding words of tau16: angles and their cos/sin in float64, rounded to float32
// (base) or through float32 to fp16 (tau16).
__global__ void __launch_bounds__(kThreads)
    rope_table_kernel(uint32_t* tau16, float* base, int32_t D, int32_t nbase, double theta) {
  const int half = D / 2;
  const int64_t n_val = (int64_t)(kQ4Group + nbase) * half;
  const int64_t total = n_val + kQ4Group * 4;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * blockDim.x) {
    if (u >= n_val) {
      const int64_t k = u - n_val;
      tau16[(k / 4) * (half + 4) + half + k % 4] = 0u;
      continue;
    }
    const int64_t r = u / half;
    const int i = (int)(u % half);
    const double f = pow(theta, -2.0 * i / D);
    const bool is_tau = r < kQ4Group;
    const double ang = (is_tau ? (double)r : (double)kQ4Group * (double)(r - kQ4Group)) * f;
    double sn, cs;
    sincos(ang, &sn, &cs);
    if (is_tau) {
      uint16_t* row = (uint16_t*)(tau16 + r * (half + 4));
      const int at = (i / 8) * 16 + 2 * (i % 4) + (i % 8) / 4;  // pair 8 b + w (+ 4): word w, half
      row[at] = __builtin_bit_cast(uint16_t, (_Float16)(float)cs);
      row[at + 8] = __builtin_bit_cast(uint16_t, (_Float16)(float)sn);
    } else {
      base[((r - kQ4Group) * half + i) * 2] = (float)cs;
      base[((r - kQ4Group) * half + i) * 2 + 1] = (float)sn;
    }
  }
}

// One thread moves one 16-byte chunk of one K or V row. Work index (outer to inner):
// tensor (K, V), sequence, token, KV head, chunk; consecutive threads read consecutive
// bytes of the input. The extra nb*m work items at the end write the slot table.
__global__ void __launch_bounds__(kThreads) append_kernel(AppendArgs a) {
  const int32_t nch = a.row_bytes / 16;
  const int64_t per_tensor = (int64_t)a.nb * a.m * a.Hkv * nch;
  const int64_t n_slot_items = (int64_t)a.nb * a.m;
  const int64_t total = 2 * per_tensor + n_slot_items;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int32_t SR = a.S + a.R;

  if (blockIdx.x == 0)
    for (int32_t i = threadIdx.x; i < a.nb; i += blockDim.x)
      a.seq_len[a.b0 + i] = a.n_old[i] + a.m;

  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += stride) {
    if (u >= 2 * per_tensor) {
      const int64_t w = u - 2 * per_tensor;
      const int32_t bi = (int32_t)(w / a.m), i = (int32_t)(w % a.m);
      const int32_t n0 = a.n_old[bi], t = n0 + i;
      if (survives(t, n0 + a.m, a.S, a.R))
        a.slot_pos[(int64_t)(a.b0 + bi) * SR + slot_of(t, a.S, a.R)] = t;
      continue;
    }
    const int tensor = u >= per_tensor;
    int64_t w = tensor ? u - per_tensor : u;
    const int32_t c = (int32_t)(w % nch); w /= nch;
    const int32_t j = (int32_t)(w % a.Hkv); w /= a.Hkv;
    const int32_t i = (int32_t)(w % a.m); w /= a.m;
    const int32_t bi = (int32_t)w;
    const int32_t b = a.b0 + bi;
    const int32_t n0 = a.n_old[bi], t = n0 + i;
    const char* src = (const char*)(tensor ? a.v : a.k) +
                      (((int64_t)bi * a.m + i) * a.Hkv + j) * a.row_bytes + c * 16;
    const int32_t ci = a.cls_idx[j];
    char* dst;
    if (ci >= 0) {
      if (a.qbits) continue;  // 4- or 8-bit full caches: written by the quantizing append
      dst = (char*)(tensor ? a.full_v : a.full_k) +
            (((int64_t)b * a.Hr + ci) * a.cap + t) * a.row_bytes + c * 16;
    } else {
      if (!survives(t, n0 + a.m, a.S, a.R)) continue;
      const int32_t s = -ci - 1;
      dst = (char*)(tensor ? a.str_v : a.str_k) +
            (((int64_t)b * a.Hs + s) * SR + slot_of(t, a.S, a.R)) * a.row_bytes + c * 16;
    }
    *(uint4*)dst = *(const uint4*)src;
  }
}

int grid_for(int64_t work) {
  int64_t g = (work + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > 8192) g = 8192;
  return (int)g;
}

}  // namespace

int launch_reset(const ResetArgs& a, void* stream) {
  const int64_t work = a.n_slot > a.n_len ? a.n_slot : a.n_len;
  hipLaunchKernelGGL(reset_kernel, dim3(grid_for(work)), dim3(kThreads), 0,
                     (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_rope_tables(char* tables, int32_t D, int32_t nbase, double theta, void* stream) {
  const RopeGeom g = rope_geom((uint64_t)(nbase - 1) * kQ4Group, (uint64_t)D);
  const int64_t work = (int64_t)(kQ4Group + nbase) * (D / 2) + kQ4Group * 4;
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(work)), dim3(kThreads), 0,
                     (hipStream_t)stream, (uint32_t*)(tables + g.tau16),
                     (float*)(tables + g.base), D, nbase, theta);
  return (int)hipGetLastError();
}

int launch_append(const AppendArgs& a, int /*dtype*/, void* stream) {
  const int64_t work = 2 * (int64_t)a.nb * a.m * a.Hkv * (a.row_bytes / 16) + (int64_t)a.nb * a.m;
  hipLaunchKernelGGL(append_kernel, dim3(grid_for(work)), dim3(kThreads), 0,
                     (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int create_events(int n, std::vector<void*>* out) {
  out->clear();
  for (int i = 0; i < n; ++i) {
    // timing only: no system-scope cache writeback and invalidation at each record, which
    // would slow the kernels that follow and count in the measured pairs
    hipEvent_t e;
    const hipError_t rc = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (rc != hipSuccess) {
      destroy_events(out);
      return (int)rc;
    }
    out->push_back((void*)e);
  }
  return 0;
}

void destroy_events(std::vector<void*>* ev) {
  for (void* e : *ev) (void)hipEventDestroy((hipEvent_t)e);
  ev->clear();
}

int record_event(void* event, void* stream) {
  return (int)hipEventRecord((hipEvent_t)event, (hipStream_t)stream);
}

int pairs_elapsed_ms(const std::vector<void*>& ev, int pairs, double* total_ms) {
  *total_ms = 0.0;
  if (pairs <= 0) return 0;
  hipError_t rc = hipEventSynchronize((hipEvent_t)ev[2 * pairs - 1]);
  if (rc != hipSuccess) return (int)rc;
  for (int i = 0; i < pairs; ++i) {
    float ms = 0.f;
    rc = hipEventElapsedTime(&ms, (hipEvent_t)ev[2 * i], (hipEvent_t)ev[2 * i + 1]);
    if (rc != hipSuccess) return (int)rc;
    *total_ms += ms;
  }
  return 0;
}

int launch_set_lengths(const SetLenArgs& a, void* stream) {
  const int64_t work = (int64_t)a.B * (a.S + a.R);
  hipLaunchKernelGGL(set_lengths_kernel, dim3((unsigned)((work + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int copy_d2h_sync(void* dst, const void* src, uint64_t bytes, void* stream) {
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e != hipSuccess) return (int)e;
  return (int)hipStreamSynchronize((hipStream_t)stream);
}

}  // namespace duo
