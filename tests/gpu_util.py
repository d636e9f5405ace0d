"""Helpers shared by the GPU parity tests: building caches from workloads, moving the seeded
inputs to the device, reading the split layout back, and the tolerance check."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

ATOL, RTOL = 2e-3, 1e-2  # |gpu - ref| <= ATOL + RTOL * |ref|, elementwise


def torch_dtype(w_dtype: str) -> torch.dtype:
    return torch.float32 if w_dtype == "f32" else torch.bfloat16


def to_dev(x: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    """float32 host values (exactly representable in ``dtype``) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return t.to(dtype) if dtype != torch.float32 else t


def make_cache(w: W.Workload, out_dtype=torch.float32, max_splits=0, capacity=None,
               layers=None, streaming_prefill="window"):
    import head_split_kv_amd as hsk
    mask = W.retrieval_mask(w)
    if layers is not None:
        mask = mask[:layers]
    return hsk.DuoCache(num_layers=mask.shape[0], batch=w.batch, num_q_heads=w.hq,
                        num_kv_heads=w.hkv, head_dim=w.d, sink=w.sink, recent=w.recent,
                        capacity=capacity or w.capacity, retrieval_mask=mask,
                        dtype=torch_dtype(w.dtype), out_dtype=out_dtype, max_splits=max_splits,
                        streaming_prefill=streaming_prefill)


def fill(cache, w: W.Workload, layer: int, lens, chunk: int = 1 << 16, mask_layer=None):
    """Bulk-append positions 0..lens[b]-1 of every sequence (no attention)."""
    dt = torch_dtype(w.dtype)
    gl = layer if mask_layer is None else mask_layer
    for b, n in enumerate(lens):
        for t0 in range(0, int(n), chunk):
            t1 = min(int(n), t0 + chunk)
            k = to_dev(W.tokens(w, "k", gl, b, t0, t1), dt)
            v = to_dev(W.tokens(w, "v", gl, b, t0, t1), dt)
            cache.kv_append(layer, k, v, seq=b)


def step_inputs(w: W.Workload, layer: int, pos):
    """q [B,Hq,d] and k, v [B,1,Hkv,d] of the token at position pos[b] of each sequence."""
    dt = torch_dtype(w.dtype)
    q = np.stack([W.tokens(w, "q", layer, b, p, p + 1)[0] for b, p in enumerate(pos)])
    k = np.stack([W.tokens(w, "k", layer, b, p, p + 1) for b, p in enumerate(pos)])
    v = np.stack([W.tokens(w, "v", layer, b, p, p + 1) for b, p in enumerate(pos)])
    return to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), q


def assert_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (ATOL + RTOL * np.abs(ref))), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r}; max abs err {err.max():.3e}")
    return float(err.max())


def layer_regions(cache, layer):
    """Device views of one layer's caches and tables, following the documented layout:
    layers are consecutive inside each region, each starting on a 256-byte boundary."""
    lay = cache.layout
    mask = cache.retrieval_mask
    es = 4 if cache.dtype == torch.float32 else 2
    B, D, cap, SR = cache.batch, cache.d, cache.capacity, cache.sink + cache.recent

    def al(x):
        return (x + 255) // 256 * 256

    full_off = sum(al(B * int(mask[l].sum()) * cap * D * es) for l in range(layer))
    str_off = sum(al(B * int((1 - mask[l]).sum()) * SR * D * es) for l in range(layer))
    hr = int(mask[layer].sum())
    hs = cache.hkv - hr
    a = cache.arena

    def view(off, n_heads, rows):
        nbytes = B * n_heads * rows * D * es
        t = a[off:off + nbytes].view(cache.dtype)
        return t.view(B, n_heads, rows, D)

    out = dict(
        full_k=view(lay.full_k_off + full_off, hr, cap),
        full_v=view(lay.full_v_off + full_off, hr, cap),
        str_k=view(lay.str_k_off + str_off, hs, SR),
        str_v=view(lay.str_v_off + str_off, hs, SR),
        ret_heads=np.nonzero(mask[layer])[0],
        str_heads=np.nonzero(1 - mask[layer])[0],
    )
    return out
