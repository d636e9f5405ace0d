"""Seeded synthetic inputs for head-partitioned KV attention.

This module only draws numbers and rounds them once to the storage dtype. It holds none of
the attention arithmetic, so both the CPU oracle and the GPU path can take their inputs from
it without sharing any of the method's code.

Shapes follow the models the DuoAttention pages measure on (Llama-2-7B: 32 heads, MHA;
Llama-3-8B: 32 query heads over 8 KV heads; head_dim 128, bf16) with the sink/recent sizes
and retrieval fractions stated for this hot path. No benchmark data is used: every value is a
seeded N(0, 1) draw.

Draw recipe (fixed, so any token range can be regenerated on its own):

* Every token stream is cut into blocks of ``BLOCK`` positions. Block ``i`` of stream
  ``(kind, layer, seq)`` comes from ``numpy.random.Generator(PCG64(SeedSequence([seed, tag,
  layer, seq, i])))`` with ``tag`` = 1 (q), 2 (k), 3 (v), 4 (per-position K scale).
  A block holds ``[BLOCK, heads, head_dim]`` float32 standard normals.
* Where a workload scales K per position, ``s_t = 1 + 0.5 * |z_t|`` with ``z_t`` the
  tag-4 stream, one value per position shared by all KV heads and dims, applied before the
  rounding.
* bf16 workloads round each float32 draw once to bf16 (round to nearest even); the values
  stay stored as float32 arrays that are exactly representable in bf16, so the GPU side can
  cast them to bf16 without a second rounding and the oracle can widen them to float64.
* Retrieval masks: per layer, ``sorted(permutation(H_kv)[:H_r])`` from
  ``SeedSequence([seed, 5, layer])``.
* Ragged initial lengths: ``integers(lo, hi + 1, size=batch)`` from
  ``SeedSequence([seed, 6])``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

BLOCK = 1024
TAG_Q, TAG_K, TAG_V, TAG_KSCALE, TAG_MASK, TAG_LENS = 1, 2, 3, 4, 5, 6


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32 values.

    Inputs are finite normal draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclass(frozen=True)
class Workload:
    """One synthetic configuration: shapes, cache policy and draw recipe."""

    name: str
    layers: int
    batch: int
    hq: int
    hkv: int
    d: int
    dtype: str  # "f32" or "bf16"
    sink: int
    recent: int
    context: int  # initial length (upper bound when ragged)
    decode_steps: int
    n_retrieval: int  # retrieval KV heads per layer
    fixed_mask: Optional[Tuple[Tuple[int, ...], ...]] = None  # per-layer retrieval heads
    ragged: Optional[Tuple[int, int]] = None  # (lo, hi) inclusive initial lengths
    k_scale: bool = False
    prefill_len: int = 0
    prefill_chunk: int = 0
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def capacity(self) -> int:
        """Full-cache rows per sequence: the initial context plus every decode step."""
        return max(self.context, self.prefill_len) + self.decode_steps

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _c(*heads):
    return (tuple(heads),)


WORKLOADS = {
    # Tiny GQA decode (fp32): oracle finishes in seconds.
    "c1": Workload("c1-tiny-gqa-fp32", 1, 1, 8, 2, 64, "f32", 4, 32, 1024, 16, 1,
                   fixed_mask=_c(0)),
    # Llama-2-7B-shaped MHA layer: decode at 32K and chunked prefill of a 32K prompt.
    "c2": Workload("c2-mha-llama2-7b-32k", 1, 1, 32, 32, 128, "bf16", 16, 512, 32768, 64, 8,
                   prefill_len=32768, prefill_chunk=4096),
    # Llama-3-8B-shaped GQA layer at 128K context, K scaled per position.
    "c3": Workload("c3-gqa-llama3-8b-128k", 1, 1, 32, 8, 128, "bf16", 16, 512, 131072, 128, 4,
                   k_scale=True),
    # Full-depth GQA decode: 32 layers, batch 8, ragged 16K..32K.
    "c4": Workload("c4-gqa-llama3-8b-32layer-b8-ragged", 32, 8, 32, 8, 128, "bf16", 16, 512,
                   32768, 16, 4, ragged=(16384, 32768)),
    # Extreme context: 1M tokens, 50% and 25% retrieval KV heads.
    "c5": Workload("c5-gqa-llama3-8b-1m-r50", 1, 1, 32, 8, 128, "bf16", 16, 512, 1 << 20, 16, 4),
    "c5q": Workload("c5-gqa-llama3-8b-1m-r25", 1, 1, 32, 8, 128, "bf16", 16, 512, 1 << 20, 16,
                    2),
}


def workload(key: str) -> Workload:
    return WORKLOADS[key]


def retrieval_mask(w: Workload) -> np.ndarray:
    """uint8 ``[layers][hkv]``, 1 = retrieval KV head."""
    m = np.zeros((w.layers, w.hkv), dtype=np.uint8)
    for layer in range(w.layers):
        if w.fixed_mask is not None:
            heads = w.fixed_mask[layer % len(w.fixed_mask)]
        else:
            rng = np.random.default_rng(np.random.SeedSequence([w.seed, TAG_MASK, layer]))
            heads = sorted(rng.permutation(w.hkv)[: w.n_retrieval].tolist())
        m[layer, list(heads)] = 1
    return m


def initial_lengths(w: Workload) -> np.ndarray:
    """int32 ``[batch]`` initial context length of each sequence."""
    if w.ragged is None:
        return np.full(w.batch, w.context, dtype=np.int32)
    lo, hi = w.ragged
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, TAG_LENS]))
    return rng.integers(lo, hi + 1, size=w.batch).astype(np.int32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _block(w: Workload, tag: int, layer: int, seq: int, i: int, heads: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, tag, layer, seq, i]))
    x = rng.standard_normal((BLOCK, heads, w.d), dtype=np.float32)
    if tag == TAG_K and w.k_scale:
        srng = np.random.default_rng(np.random.SeedSequence([w.seed, TAG_KSCALE, layer, seq, i]))
        z = srng.standard_normal(BLOCK, dtype=np.float32)
        s = (1.0 + 0.5 * np.abs(z)).astype(np.float32)
        x *= s[:, None, None]
    if w.dtype == "bf16":
        x = bf16_round(x)
    return x


def tokens(w: Workload, kind: str, layer: int, seq: int, t0: int, t1: int) -> np.ndarray:
    """float32 ``[t1 - t0, heads, d]`` for positions ``t0 .. t1-1`` of one stream.

    ``kind`` is ``"q"`` (heads = hq), ``"k"`` or ``"v"`` (heads = hkv). The values are exactly
    representable in the workload dtype. Any sub-range gives the same values as the
    corresponding slice of a longer range.
    """
    tag = {"q": TAG_Q, "k": TAG_K, "v": TAG_V}[kind]
    heads = w.hq if kind == "q" else w.hkv
    t0, t1 = int(t0), int(t1)
    out = np.empty((max(0, t1 - t0), heads, w.d), dtype=np.float32)
    if t1 <= t0:
        return out
    b0, b1 = t0 // BLOCK, (t1 - 1) // BLOCK

    def fill(i):
        blk = _block(w, tag, layer, seq, i, heads)
        s0 = max(t0, i * BLOCK)
        s1 = min(t1, (i + 1) * BLOCK)
        out[s0 - t0 : s1 - t0] = blk[s0 - i * BLOCK : s1 - i * BLOCK]

    idx = range(b0, b1 + 1)
    if b1 - b0 >= 4:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, idx))
    else:
        for i in idx:
            fill(i)
    return out


def tokens_batched(w: Workload, kind: str, layer: int, t0s, m: int) -> np.ndarray:
    """float32 ``[batch, m, heads, d]``: positions ``t0s[b] .. t0s[b]+m-1`` of each sequence."""
    return np.stack([tokens(w, kind, layer, b, int(t0s[b]), int(t0s[b]) + m)
                     for b in range(w.batch)])
