"""Python binding of libduo: attention over a head-partitioned KV cache on MI355X.

The functions below carry the names of the C ABI in ``include/duo.h`` and only marshal
arguments: they check tensor shapes, dtypes, devices and contiguity (the C side sees raw
pointers and cannot), pass data pointers and the current HIP stream, and raise
``DuoError`` on a non-zero status. PyTorch supplies device memory and streams; every step
of the computation runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import _native
from ._native import (DUO_BF16, DUO_ERR_CAPACITY, DUO_ERR_HIP, DUO_ERR_INVALID,  # noqa: F401
                      DUO_ERR_UNSUPPORTED, DUO_F32, DUO_OK, DuoConfig, DuoError, DuoLayout,
                      check, lib, status_string)

_DTYPES = {torch.float32: DUO_F32, torch.bfloat16: DUO_BF16}


def _dt(dtype: torch.dtype) -> int:
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}; use torch.float32 or torch.bfloat16")
    return _DTYPES[dtype]


_PREFILL_MODES = {"window": _native.PREFILL_WINDOW, "chunk": _native.PREFILL_CHUNK}


def make_config(*, num_layers: int, batch: int, num_q_heads: int, num_kv_heads: int,
                head_dim: int, sink: int, recent: int, capacity: int,
                retrieval_mask, dtype: torch.dtype = torch.bfloat16,
                out_dtype: Optional[torch.dtype] = None, softmax_scale: float = 0.0,
                max_splits: int = 0, prefill_tiles: int = 0, streaming_prefill: str = "window",
                kv_bits: int = 0, rope_theta: float = 0.0):
    """Build a ``DuoConfig``; returns ``(cfg, mask_array)`` (keep the array alive).

    ``streaming_prefill`` is ``"window"`` (streaming heads use the per-query sink + recent
    mask during pre-filling) or ``"chunk"`` (they see the whole pruned cache before the chunk
    plus the chunk causally). ``kv_bits=4`` (or 8) stores the full (retrieval) caches in 4
    (8) bits; with it, ``rope_theta > 0`` takes keys before RoPE (base ``rope_theta``, rotate-half
    pairs) and queries after it, and attention turns each key at its position."""
    if streaming_prefill not in _PREFILL_MODES:
        raise ValueError(f"streaming_prefill must be 'window' or 'chunk', not {streaming_prefill!r}")
    mask = np.ascontiguousarray(np.asarray(retrieval_mask, dtype=np.uint8)
                                .reshape(num_layers, num_kv_heads))
    cfg = DuoConfig(num_layers, batch, num_q_heads, num_kv_heads, head_dim, sink, recent,
                    capacity, _dt(dtype), _dt(out_dtype or dtype), float(softmax_scale),
                    max_splits, prefill_tiles,
                    mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                    _PREFILL_MODES[streaming_prefill], int(kv_bits), float(rope_theta))
    return cfg, mask


def duo_layout_query(cfg: DuoConfig) -> DuoLayout:
    lay = DuoLayout()
    check(lib().duo_layout_query(ctypes.byref(cfg), ctypes.byref(lay)), "duo_layout_query")
    return lay


def duo_kv_bytes(cfg: DuoConfig, seq_lens: Sequence[int], layer: int):
    """(full-attention bytes, split-layout bytes) one layer holds for these lengths."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    full = ctypes.c_uint64()
    duo = ctypes.c_uint64()
    check(lib().duo_kv_bytes(ctypes.byref(cfg),
                             lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), layer,
                             ctypes.byref(full), ctypes.byref(duo)), "duo_kv_bytes")
    return full.value, duo.value


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


class DuoCache:
    """A head-partitioned KV cache in one device arena (``torch.uint8`` tensor)."""

    def __init__(self, *, num_layers: int, batch: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, sink: int, recent: int, capacity: int, retrieval_mask,
                 dtype: torch.dtype = torch.bfloat16, out_dtype: Optional[torch.dtype] = None,
                 softmax_scale: float = 0.0, max_splits: int = 0, prefill_tiles: int = 0,
                 streaming_prefill: str = "window", kv_bits: int = 0, rope_theta: float = 0.0,
                 device="cuda", stream=None):
        self.cfg, self._mask = make_config(
            num_layers=num_layers, batch=batch, num_q_heads=num_q_heads,
            num_kv_heads=num_kv_heads, head_dim=head_dim, sink=sink, recent=recent,
            capacity=capacity, retrieval_mask=retrieval_mask, dtype=dtype, out_dtype=out_dtype,
            softmax_scale=softmax_scale, max_splits=max_splits, prefill_tiles=prefill_tiles,
            streaming_prefill=streaming_prefill, kv_bits=kv_bits, rope_theta=rope_theta)
        self.streaming_prefill = streaming_prefill
        self.kv_bits = kv_bits
        self.rope_theta = rope_theta
        self.layout = duo_layout_query(self.cfg)
        self.dtype = dtype
        self.out_dtype = out_dtype or dtype
        self.device = torch.device(device)
        self.num_layers, self.batch = num_layers, batch
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.sink, self.recent, self.capacity = sink, recent, capacity
        nbytes = int(self.layout.arena_bytes)
        self._arena_raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        off = (-self._arena_raw.data_ptr()) % 256
        self.arena = self._arena_raw[off:off + nbytes]
        h = ctypes.c_void_p()
        check(lib().duo_cache_init(ctypes.byref(self.cfg), ctypes.c_void_p(self.arena.data_ptr()),
                                   nbytes, _stream(stream), ctypes.byref(h)), "duo_cache_init")
        self.handle = h

    @property
    def retrieval_mask(self) -> np.ndarray:
        return self._mask.copy()

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib().duo_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # convenience wrappers
    def kv_append(self, layer, k, v, seq=-1, stream=None):
        return duo_kv_append(self, layer, seq, k, v, stream=stream)

    def attn_decode(self, layer, q, out=None, lse=None, stream=None):
        return duo_attn_decode(self, layer, q, out, lse, stream=stream)

    def decode_step(self, layer, q, k, v, out=None, lse=None, stream=None):
        return duo_decode_step(self, layer, q, k, v, out, lse, stream=stream)

    def attn_prefill(self, layer, q, k, v, seq=-1, out=None, lse=None, stream=None):
        return duo_attn_prefill(self, layer, seq, q, k, v, out, lse, stream=stream)

    def attn_prefill_staged(self, layer, q, k, v, seq=-1, out=None, lse=None, staging=None,
                            stream=None):
        return duo_attn_prefill_staged(self, layer, seq, q, k, v, out, lse, staging,
                                       stream=stream)

    def attn_gate_mixed(self, layer, q, k, v, alpha, seq=-1, out=None, stream=None):
        return duo_attn_gate_mixed(self, layer, seq, q, k, v, alpha, out, stream=stream)

    def slot_positions(self, layer, stream=None):
        return duo_slot_positions(self, layer, stream)

    def lengths(self):
        return duo_cache_lengths(self)

    def set_lengths(self, lens, stream=None):
        return duo_cache_set_lengths(self, lens, stream)


def _check_tensor(t: torch.Tensor, shape, dtype, device, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device and not (t.device.type == device.type == "cuda"
                                   and (device.index is None or t.device.index == device.index)):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")


def duo_cache_reset(cache: DuoCache, stream=None) -> None:
    check(lib().duo_cache_reset(cache.handle, _stream(stream)), "duo_cache_reset")


def duo_cache_set_lengths(cache: DuoCache, lens, stream=None) -> None:
    """Set every length (int ``[L, B]``) and rebuild the slot tables to match."""
    a = np.ascontiguousarray(np.asarray(lens, dtype=np.int32).reshape(cache.num_layers, cache.batch))
    check(lib().duo_cache_set_lengths(cache.handle, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      _stream(stream)), "duo_cache_set_lengths")


def duo_kv_append(cache: DuoCache, layer: int, seq: int, k: torch.Tensor, v: torch.Tensor,
                  n_new: Optional[int] = None, stream=None) -> None:
    """Append tokens; k, v ``[B, m, Hkv, d]`` (seq = -1) or ``[m, Hkv, d]`` (seq >= 0)."""
    m = k.shape[1] if seq < 0 else k.shape[0]
    if n_new is not None and n_new != m:
        raise ValueError("n_new does not match k")
    shape = ((cache.batch, m, cache.hkv, cache.d) if seq < 0 else (m, cache.hkv, cache.d))
    _check_tensor(k, shape, cache.dtype, cache.device, "k")
    _check_tensor(v, shape, cache.dtype, cache.device, "v")
    check(lib().duo_kv_append(cache.handle, layer, seq, ctypes.c_void_p(k.data_ptr()),
                              ctypes.c_void_p(v.data_ptr()), m, _stream(stream)),
          "duo_kv_append")


def duo_attn_decode(cache: DuoCache, layer: int, q: torch.Tensor, out=None, lse=None,
                    stream=None):
    """One decode step; q ``[B, Hq, d]`` -> out ``[B, Hq, d]`` (and lse ``[B, Hq]``)."""
    _check_tensor(q, (cache.batch, cache.hq, cache.d), cache.dtype, cache.device, "q")
    if out is None:
        out = torch.empty((cache.batch, cache.hq, cache.d), dtype=cache.out_dtype,
                          device=q.device)
    _check_tensor(out, (cache.batch, cache.hq, cache.d), cache.out_dtype, cache.device, "out")
    lse_ptr = None
    if lse is not None:
        _check_tensor(lse, (cache.batch, cache.hq), torch.float32, cache.device, "lse")
        lse_ptr = lse.data_ptr()
    check(lib().duo_attn_decode(cache.handle, layer, ctypes.c_void_p(q.data_ptr()),
                                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse_ptr),
                                _stream(stream)), "duo_attn_decode")
    return out


def duo_attn_decode_noalloc(cache: DuoCache, layer: int, q: torch.Tensor, out: torch.Tensor,
                            lse=None, stream=None):
    """``duo_attn_decode`` whose split-K partials live in the library's static device scratch
    (no allocation in the call); ``out`` must be given."""
    _check_tensor(q, (cache.batch, cache.hq, cache.d), cache.dtype, cache.device, "q")
    _check_tensor(out, (cache.batch, cache.hq, cache.d), cache.out_dtype, cache.device, "out")
    lse_ptr = None
    if lse is not None:
        _check_tensor(lse, (cache.batch, cache.hq), torch.float32, cache.device, "lse")
        lse_ptr = lse.data_ptr()
    check(lib().duo_attn_decode_noalloc(cache.handle, layer, ctypes.c_void_p(q.data_ptr()),
                                        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse_ptr),
                                        _stream(stream)), "duo_attn_decode_noalloc")
    return out


def duo_decode_step(cache: DuoCache, layer: int, q: torch.Tensor, k: torch.Tensor,
                    v: torch.Tensor, out=None, lse=None, stream=None):
    """Append one token per sequence and decode it in one pass: q ``[B, Hq, d]``,
    k, v ``[B, Hkv, d]`` -> out ``[B, Hq, d]`` (and lse ``[B, Hq]``)."""
    _check_tensor(q, (cache.batch, cache.hq, cache.d), cache.dtype, cache.device, "q")
    _check_tensor(k, (cache.batch, cache.hkv, cache.d), cache.dtype, cache.device, "k")
    _check_tensor(v, (cache.batch, cache.hkv, cache.d), cache.dtype, cache.device, "v")
    if out is None:
        out = torch.empty((cache.batch, cache.hq, cache.d), dtype=cache.out_dtype,
                          device=q.device)
    _check_tensor(out, (cache.batch, cache.hq, cache.d), cache.out_dtype, cache.device, "out")
    lse_ptr = None
    if lse is not None:
        _check_tensor(lse, (cache.batch, cache.hq), torch.float32, cache.device, "lse")
        lse_ptr = lse.data_ptr()
    check(lib().duo_decode_step(cache.handle, layer, ctypes.c_void_p(q.data_ptr()),
                                ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse_ptr),
                                _stream(stream)), "duo_decode_step")
    return out


def duo_attn_prefill(cache: DuoCache, layer: int, seq: int, q: torch.Tensor, k: torch.Tensor,
                     v: torch.Tensor, out=None, lse=None, stream=None):
    """Attention of one chunk; q ``[B, m, Hq, d]`` / k, v ``[B, m, Hkv, d]`` (seq = -1) or
    without the batch dimension (seq >= 0). Does not modify the cache."""
    m = q.shape[1] if seq < 0 else q.shape[0]
    lead = (cache.batch, m) if seq < 0 else (m,)
    _check_tensor(q, lead + (cache.hq, cache.d), cache.dtype, cache.device, "q")
    _check_tensor(k, lead + (cache.hkv, cache.d), cache.dtype, cache.device, "k")
    _check_tensor(v, lead + (cache.hkv, cache.d), cache.dtype, cache.device, "v")
    if out is None:
        out = torch.empty(lead + (cache.hq, cache.d), dtype=cache.out_dtype, device=q.device)
    _check_tensor(out, lead + (cache.hq, cache.d), cache.out_dtype, cache.device, "out")
    lse_ptr = None
    if lse is not None:
        _check_tensor(lse, lead + (cache.hq,), torch.float32, cache.device, "lse")
        lse_ptr = lse.data_ptr()
    check(lib().duo_attn_prefill(cache.handle, layer, seq, ctypes.c_void_p(q.data_ptr()),
                                 ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                 m, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse_ptr),
                                 _stream(stream)), "duo_attn_prefill")
    return out


def duo_prefill_staging_bytes(cache: DuoCache, layer: int, seq: int = -1,
                              n_chunk: int = 0) -> int:
    """Bytes of staging ``duo_attn_prefill_staged`` needs for a chunk of ``n_chunk`` tokens at
    the current lengths (bf16 read-backs on a 4- or 8-bit cache, fp16 values on a bf16
    cache, 0 on an fp32 cache)."""
    n = ctypes.c_uint64()
    check(lib().duo_prefill_staging_bytes(cache.handle, layer, seq, n_chunk, ctypes.byref(n)),
          "duo_prefill_staging_bytes")
    return n.value


def duo_attn_prefill_staged(cache: DuoCache, layer: int, seq: int, q: torch.Tensor,
                            k: torch.Tensor, v: torch.Tensor, out=None, lse=None, staging=None,
                            stream=None):
    """``duo_attn_prefill`` through caller staging (a ``torch.uint8`` device tensor of at
    least ``duo_prefill_staging_bytes`` bytes; allocated here when None). Over a 4- or 8-bit
    cache the retrieval heads' earlier tokens are read back as bf16 rows into it, then the
    chunk attends; with pre-RoPE keys (``rope_theta``) ``q`` is after RoPE and ``k`` before
    it, and the keys are staged turned. On a bf16 cache the values the chunk reads are staged
    as fp16 copies, and the result is bit-identical to ``duo_attn_prefill``. Shapes as in
    ``duo_attn_prefill``."""
    m = q.shape[1] if seq < 0 else q.shape[0]
    lead = (cache.batch, m) if seq < 0 else (m,)
    _check_tensor(q, lead + (cache.hq, cache.d), cache.dtype, cache.device, "q")
    _check_tensor(k, lead + (cache.hkv, cache.d), cache.dtype, cache.device, "k")
    _check_tensor(v, lead + (cache.hkv, cache.d), cache.dtype, cache.device, "v")
    if out is None:
        out = torch.empty(lead + (cache.hq, cache.d), dtype=cache.out_dtype, device=q.device)
    _check_tensor(out, lead + (cache.hq, cache.d), cache.out_dtype, cache.device, "out")
    lse_ptr = None
    if lse is not None:
        _check_tensor(lse, lead + (cache.hq,), torch.float32, cache.device, "lse")
        lse_ptr = lse.data_ptr()
    need = duo_prefill_staging_bytes(cache, layer, seq, m)
    if staging is None:
        staging = torch.empty(max(need, 16), dtype=torch.uint8, device=cache.device)
    check(lib().duo_attn_prefill_staged(cache.handle, layer, seq, ctypes.c_void_p(q.data_ptr()),
                                        ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                        m, ctypes.c_void_p(out.data_ptr()),
                                        ctypes.c_void_p(lse_ptr),
                                        ctypes.c_void_p(staging.data_ptr()), staging.numel(),
                                        _stream(stream)), "duo_attn_prefill_staged")
    return out


def duo_attn_gate_mixed(cache: DuoCache, layer: int, seq: int, q: torch.Tensor, k: torch.Tensor,
                        v: torch.Tensor, alpha, out=None, stream=None):
    """Gate-mixed attention of one chunk, ``alpha[j] * full + (1 - alpha[j]) * streaming`` per
    KV head j (every KV head of the layer must keep a full cache). Shapes as in
    ``duo_attn_prefill``; ``alpha`` has one gate per KV head. Does not modify the cache."""
    m = q.shape[1] if seq < 0 else q.shape[0]
    lead = (cache.batch, m) if seq < 0 else (m,)
    _check_tensor(q, lead + (cache.hq, cache.d), cache.dtype, cache.device, "q")
    _check_tensor(k, lead + (cache.hkv, cache.d), cache.dtype, cache.device, "k")
    _check_tensor(v, lead + (cache.hkv, cache.d), cache.dtype, cache.device, "v")
    if out is None:
        out = torch.empty(lead + (cache.hq, cache.d), dtype=cache.out_dtype, device=q.device)
    _check_tensor(out, lead + (cache.hq, cache.d), cache.out_dtype, cache.device, "out")
    a = np.ascontiguousarray(np.asarray(alpha, dtype=np.float32).reshape(-1))
    if a.size != cache.hkv:
        raise ValueError(f"alpha must hold {cache.hkv} gates")
    check(lib().duo_attn_gate_mixed(cache.handle, layer, seq, ctypes.c_void_p(q.data_ptr()),
                                    ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                    m, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                    ctypes.c_void_p(out.data_ptr()), _stream(stream)),
          "duo_attn_gate_mixed")
    return out


def duo_slot_positions(cache: DuoCache, layer: int, stream=None) -> np.ndarray:
    """Slot table of one layer, int32 ``[B, S+R]`` (synchronizes the stream)."""
    out = np.empty((cache.batch, cache.sink + cache.recent), dtype=np.int32)
    check(lib().duo_slot_positions(cache.handle, layer,
                                   out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   _stream(stream)), "duo_slot_positions")
    return out


def duo_cache_lengths(cache: DuoCache) -> np.ndarray:
    out = np.empty((cache.num_layers, cache.batch), dtype=np.int32)
    check(lib().duo_cache_lengths(cache.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
          "duo_cache_lengths")
    return out


def duo_set_decode_splits(cache: DuoCache, splits: int) -> None:
    check(lib().duo_set_decode_splits(cache.handle, splits), "duo_set_decode_splits")


def duo_timing_enable(cache: DuoCache, max_records: int) -> None:
    """Record HIP events around the attention kernel of the next ``max_records`` decode
    calls and, separately, prefill calls (0 switches timing off)."""
    check(lib().duo_timing_enable(cache.handle, max_records), "duo_timing_enable")


def duo_timing_read(cache: DuoCache, kind: str = "decode"):
    """(summed kernel milliseconds, recorded launches) of ``kind`` ("decode" or "prefill")
    since the last read; waits for the last recorded launch."""
    from ._native import TIMING_DECODE, TIMING_PREFILL
    k = {"decode": TIMING_DECODE, "prefill": TIMING_PREFILL}[kind]
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int32(0)
    check(lib().duo_timing_read(cache.handle, k, ctypes.byref(ms), ctypes.byref(n)),
          "duo_timing_read")
    return ms.value, n.value


def duo_read_probe(src: torch.Tensor, flag: torch.Tensor, blocks: int = 0, stream=None) -> None:
    """Measurement aid: read every byte of the device tensor ``src`` once with the decode
    kernels' non-temporal loads (``flag``: a device int32 tensor of at least one element)."""
    for t in (src, flag):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("src and flag must be contiguous device tensors")
    if flag.numel() * flag.element_size() < 4:
        raise ValueError("flag must hold at least 4 bytes")
    check(lib().duo_read_probe(ctypes.c_void_p(src.data_ptr()),
                               src.numel() * src.element_size(),
                               ctypes.c_void_p(flag.data_ptr()), int(blocks), _stream(stream)),
          "duo_read_probe")


def duo_binarize_gates(alpha, ratio: float):
    """Retrieval mask (uint8 ``[L, H_kv]``), threshold tau and retrieval count from the trained
    gates ``alpha [L, H_kv]`` for a target retrieval ratio (the quantile runs over all heads;
    equal gates go to the lower (layer, head))."""
    a = np.ascontiguousarray(np.asarray(alpha, dtype=np.float32))
    if a.ndim != 2:
        raise ValueError("alpha must be [layers, kv_heads]")
    mask = np.empty(a.shape, dtype=np.uint8)
    tau = ctypes.c_float()
    n = ctypes.c_int32()
    check(lib().duo_binarize_gates(a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), a.shape[0],
                                   a.shape[1], float(ratio),
                                   mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                   ctypes.byref(tau), ctypes.byref(n)), "duo_binarize_gates")
    return mask, tau.value, n.value


def duo_head_order(mask_layer, group: int = 1):
    """(kv_order, q_order): native KV / query head at each slot of the reordered layout of one
    layer, retrieval heads first."""
    m = np.ascontiguousarray(np.asarray(mask_layer, dtype=np.uint8).reshape(-1))
    kv = np.empty(m.size, dtype=np.int32)
    q = np.empty(m.size * group, dtype=np.int32)
    check(lib().duo_head_order(m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), m.size, group,
                               kv.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                               q.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
          "duo_head_order")
    return kv, q


def duo_permute_blocks(src: torch.Tensor, dst: torch.Tensor, outer: int, n_blocks: int,
                       block_bytes: int, order, stream=None) -> None:
    """``dst[o][i] = src[o][order[i]]`` over blocks of ``block_bytes`` bytes (device tensors)."""
    for t in (src, dst):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("src and dst must be contiguous device tensors")
    if src.numel() * src.element_size() != outer * n_blocks * block_bytes or \
            dst.numel() * dst.element_size() != outer * n_blocks * block_bytes:
        raise ValueError("tensor sizes do not match outer * n_blocks * block_bytes")
    o = np.ascontiguousarray(np.asarray(order, dtype=np.int32).reshape(-1))
    if o.size != n_blocks:
        raise ValueError("order must have n_blocks entries")
    check(lib().duo_permute_blocks(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                   outer, n_blocks, block_bytes,
                                   o.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   _stream(stream)), "duo_permute_blocks")


def reorder_output_rows(w: torch.Tensor, order, rows_per_head: int, stream=None) -> torch.Tensor:
    """A Q, K or V projection weight ``[heads * rows_per_head, hidden]`` with its head blocks
    in ``order`` (block i of the result is block ``order[i]`` of ``w``)."""
    heads = len(order)
    if w.dim() != 2 or w.shape[0] != heads * rows_per_head:
        raise ValueError("w must be [heads * rows_per_head, hidden]")
    w = w.contiguous()
    out = torch.empty_like(w)
    duo_permute_blocks(w, out, 1, heads, rows_per_head * w.shape[1] * w.element_size(), order,
                       stream)
    return out


def reorder_input_cols(w: torch.Tensor, order, cols_per_head: int, stream=None) -> torch.Tensor:
    """The output projection ``[hidden, heads * cols_per_head]`` with its per-head column
    blocks in ``order``."""
    heads = len(order)
    if w.dim() != 2 or w.shape[1] != heads * cols_per_head:
        raise ValueError("w must be [hidden, heads * cols_per_head]")
    w = w.contiguous()
    out = torch.empty_like(w)
    duo_permute_blocks(w, out, w.shape[0], heads, cols_per_head * w.element_size(), order, stream)
    return out


def duo_status_string(status: int) -> str:
    return status_string(status)
