"""CPU float64 oracle for DuoAttention's deployment hot path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module. It shares no code with the HIP library under
``head_split_kv_amd/`` and imports nothing from it; the product path never calls it.

Every function is written from the text of these pages (all about arXiv 2410.10819,
"DuoAttention: Efficient Long-Context LLM Inference with Retrieval and Streaming Heads"):

* *explainer*: the paper-graph-ui.vercel.app walkthrough of the paper;
* *OpenReview thread*: the paperhub.cn page with the authors' rebuttal;
* *abstract*: the arXiv abstract quoted on the mlsanity.com index page.

What it computes is a plain definition, so the oracle is that definition written out with no
blocking, splitting or reordering: per query head, softmax over the logits of the visible
keys (masked positions get a logit of -inf), times V, all in float64 from the exact input
values. The visible set is built from token positions only, never from a cache or a slot
table. Readings taken where the pages are silent or garbled are marked "Reading:" below.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against something other
than itself (brute force, library routines, special cases, the worked example of the chunked
pre-filling figure and the pages' printed memory numbers). Nothing is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------------------------
# Head classes and visibility
# --------------------------------------------------------------------------------------------

def kv_head_of(h: int, group: int) -> int:
    """KV head serving query head ``h`` when ``group`` query heads share one KV head.

    OpenReview thread, reply on the proportion of retrieval heads: in Llama-3-8B four query
    heads share one KV head; the gate (and so the retrieval/streaming class) is per KV head
    (explainer, "Gate Parameterization"). Reading: groups are contiguous, head h -> h // G.
    """
    return h // group


def visible_mask(q_pos, k_pos, retrieval: bool, sink: int, recent: int) -> np.ndarray:
    """Boolean ``[len(q_pos), len(k_pos)]``: may query position p attend to key position t?

    Explainer, "The Full and Streaming Attention Masks": the causal mask keeps t <= p; the
    Lambda-shaped streaming mask keeps only the first ``sink`` tokens of the sequence and the
    ``recent`` most recent tokens, every other logit being set to -inf before the softmax.

    Reading: the recent window counts the query's own token, so it is t in [p-R+1, p]. The
    decoding procedure (explainer, "Decoding Procedure", step 3-4) keeps at most S+R tokens
    in the streaming cache, which is exactly this set after the new token is appended.
    """
    p = np.asarray(q_pos, dtype=np.int64)[:, None]
    t = np.asarray(k_pos, dtype=np.int64)[None, :]
    causal = (t <= p) & (t >= 0)
    if retrieval:
        return causal
    return causal & ((t < sink) | (t >= p - recent + 1))


def chunk_visible_mask(q_pos, k_pos, start: int, retrieval: bool, sink: int,
                       recent: int) -> np.ndarray:
    """The chunk-granular reading of chunked pre-filling, for a chunk starting at ``start``.

    Explainer, "Chunked Pre-filling" (Figure 5): after each chunk the streaming heads' cache is
    pruned to the sinks and the most recent tokens, and the next chunk attends to that pruned
    cache together with itself. Reading: a streaming head's query p in the chunk sees the
    tokens the cache holds when the chunk starts (t < start with t < S or t >= start - R, the
    same set as ``streaming_valid_tokens(start)``) and the chunk's tokens t in [start, p];
    a retrieval head keeps the causal mask. Unlike ``visible_mask`` this depends on where
    the chunks start.
    """
    p = np.asarray(q_pos, dtype=np.int64)[:, None]
    t = np.asarray(k_pos, dtype=np.int64)[None, :]
    causal = (t <= p) & (t >= 0)
    if retrieval:
        return causal
    held = (t >= 0) & (t < start) & ((t < sink) | (t >= start - recent))
    return held | ((t >= start) & (t <= p))


# --------------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------------

def default_scale(d: int) -> float:
    """Reading: the pages' mask equations omit the softmax temperature; standard Transformer
    attention (which the explainer says Q, K, V are) uses 1/sqrt(head_dim)."""
    return 1.0 / math.sqrt(d)


def masked_softmax_attention(q, k, v, mask, scale):
    """One head: ``q [P, d]``, ``k, v [T, d]``, ``mask [P, T]`` -> ``out [P, d]``, ``lse [P]``.

    softmax(scale * q k^T with masked logits = -inf) v, in float64, max-subtracted.
    ``lse`` is the natural log of the softmax denominator of the unshifted logits.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    z = scale * (q @ k.T)
    z = np.where(mask, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    den = w.sum(axis=1, keepdims=True)
    out = (w @ v) / den
    lse = (m + np.log(den))[:, 0]
    return out, lse


def attention(q, k, v, q_pos, k_pos, retrieval, sink, recent, scale=None, chunk_start=None):
    """All heads of one layer and one sequence.

    ``q [P, Hq, d]``, ``k, v [T, Hkv, d]``, ``q_pos [P]``, ``k_pos [T]``,
    ``retrieval [Hkv]`` (1 = retrieval KV head) -> ``out [P, Hq, d]``, ``lse [P, Hq]``.

    Retrieval heads use the causal mask, streaming heads the Lambda mask (explainer,
    "Decoding Procedure", steps 2-3); the outputs are returned in the native head order,
    which is the concatenation of step 5 undone by the head permutation of "Head Reordering
    Preprocessing" (heads are permutation-invariant there). No KV head is repeated for GQA:
    each query head reads its own group's K and V (OpenReview thread, GQA compatibility).
    With ``chunk_start`` set, streaming heads use ``chunk_visible_mask`` for a chunk that
    starts there instead of the per-query Lambda mask.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    P, Hq, d = q.shape
    T, Hkv, _ = k.shape
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(d)
    out = np.empty((P, Hq, d), dtype=np.float64)
    lse = np.empty((P, Hq), dtype=np.float64)
    masks = {}
    for h in range(Hq):
        j = kv_head_of(h, G)
        r = bool(retrieval[j])
        if r not in masks:
            masks[r] = (visible_mask(q_pos, k_pos, r, sink, recent) if chunk_start is None else
                        chunk_visible_mask(q_pos, k_pos, chunk_start, r, sink, recent))
        out[:, h, :], lse[:, h] = masked_softmax_attention(q[:, h, :], k[:, j, :], v[:, j, :],
                                                           masks[r], scale)
    return out, lse


def gate_mixed_attention(q, k, v, q_pos, k_pos, alpha, sink, recent, scale=None):
    """Attention of the identification phase: for KV head j with gate ``alpha[j]``, each of
    its query heads returns alpha_j * full_attn + (1 - alpha_j) * streaming_attn.

    Explainer, "Gate Parameterization" (the mixing equation) and "The Full and Streaming
    Attention Masks": full_attn is softmax attention under the causal mask and
    streaming_attn the same under the Lambda mask, over the same keys; the two normalized
    outputs are blended, not their logits or weights. Shapes as in ``attention``;
    ``alpha [Hkv]``. Returns ``out [P, Hq, d]``.
    """
    Hkv = np.asarray(k).shape[1]
    full, _ = attention(q, k, v, q_pos, k_pos, np.ones(Hkv, dtype=np.uint8), sink, recent, scale)
    stream, _ = attention(q, k, v, q_pos, k_pos, np.zeros(Hkv, dtype=np.uint8), sink, recent,
                          scale)
    a = np.asarray(alpha, dtype=np.float64)
    G = np.asarray(q).shape[1] // Hkv
    w = np.array([a[kv_head_of(h, G)] for h in range(np.asarray(q).shape[1])])[None, :, None]
    return w * full + (1.0 - w) * stream


def decode_step(q, k_hist, v_hist, retrieval, sink, recent, scale=None):
    """Decode one token for one sequence.

    ``k_hist, v_hist [n, Hkv, d]`` hold tokens 0..n-1, the newest (position n-1) included;
    ``q [Hq, d]`` is that token's query. Returns ``out [Hq, d]``, ``lse [Hq]``.

    Reading: the cache is updated before attending (explainer, "Decoding Procedure" lists the
    update as step 4), so the query sees its own key, as the causal mask requires. For a
    one-token step the token overwritten in the ring is p-R, outside the window, so the order
    does not change the result.
    """
    n = k_hist.shape[0]
    out, lse = attention(np.asarray(q)[None], k_hist, v_hist, [n - 1], np.arange(n),
                         retrieval, sink, recent, scale)
    return out[0], lse[0]


def prefill_chunk(q, k_hist, v_hist, start, retrieval, sink, recent, scale=None,
                  chunk_granular=False):
    """Chunked pre-filling of positions ``start .. start+m-1`` for one sequence.

    ``q [m, Hq, d]``; ``k_hist, v_hist [start+m, Hkv, d]`` (all earlier tokens plus the
    chunk). Returns ``out [m, Hq, d]``, ``lse [m, Hq]``.

    Explainer, "Chunked Pre-filling": retrieval heads attend to every earlier token plus the
    chunk causally. Reading: streaming heads apply the same per-query Lambda mask as in
    decoding, so the result does not depend on the chunk size and equals token-by-token
    decoding; the pruned cache after each chunk still holds every key this mask can reach.
    ``chunk_granular=True`` takes the other reading instead (``chunk_visible_mask``).
    """
    m = np.asarray(q).shape[0]
    T = start + m
    assert k_hist.shape[0] >= T
    return attention(q, k_hist[:T], v_hist[:T], np.arange(start, T), np.arange(T),
                     retrieval, sink, recent, scale,
                     chunk_start=start if chunk_granular else None)


# --------------------------------------------------------------------------------------------
# Streaming cache state (sink fill, then ring overwrite)
# --------------------------------------------------------------------------------------------

def slot_of(t: int, sink: int, recent: int) -> int:
    """Streaming-cache slot of token t.

    Explainer, "Decoding Procedure", step 4: the streaming cache keeps the sink tokens and
    evicts the oldest non-sink token once it holds more than S+R tokens. Reading: sinks take
    slots 0..S-1 in order; later tokens go round a ring of R slots starting at slot S.
    """
    return t if t < sink else sink + (t - sink) % recent


def streaming_valid_tokens(n: int, sink: int, recent: int) -> np.ndarray:
    """Positions held by a streaming cache after ``n`` tokens: the first min(S, n) tokens and
    the last R non-sink tokens (explainer, "Decoding Procedure" step 3 and "Chunked
    Pre-filling": the pruned cache keeps only attention sinks and recent tokens)."""
    sinks = np.arange(min(sink, n))
    recent_part = np.arange(max(sink, n - recent), n)
    return np.concatenate([sinks, recent_part]).astype(np.int64)


def slot_table(n: int, sink: int, recent: int) -> np.ndarray:
    """int32 ``[S+R]``: the position held by each slot after ``n`` tokens, -1 if empty."""
    table = np.full(sink + recent, -1, dtype=np.int32)
    for t in streaming_valid_tokens(n, sink, recent):
        table[slot_of(int(t), sink, recent)] = t
    return table


def streaming_cache_rows(x_hist, n, sink, recent):
    """Expected streaming-cache contents ``[S+R, ...]`` of one head after ``n`` tokens:
    slot s holds row ``x_hist[slot_table[s]]``; empty slots are returned as NaN."""
    x_hist = np.asarray(x_hist)
    table = slot_table(n, sink, recent)
    rows = np.full((sink + recent,) + x_hist.shape[1:], np.nan, dtype=np.float64)
    ok = table >= 0
    rows[ok] = x_hist[table[ok]]
    return rows, table


# --------------------------------------------------------------------------------------------
# KV memory model
# --------------------------------------------------------------------------------------------

def full_kv_elements(layers: int, kv_heads: int, length: int, d: int) -> int:
    """Full-attention KV cache size in elements: 2 * D * H * L * d (explainer, "Context and
    Motivation": K and V for every head of every layer and every token). For a GQA model H
    counts KV heads."""
    return 2 * layers * kv_heads * length * d


def duo_kv_elements_layer(n_retrieval: int, n_streaming: int, length: int, sink: int,
                          recent: int, d: int) -> int:
    """Elements of K (or of V) held by one layer: (H_r * L + H_s * (S + R)) * d (explainer,
    "Decoding Procedure", memory formula). Reading: a streaming cache holds min(L, S+R)
    tokens, since it holds at most S+R and never a token that does not exist yet."""
    return (n_retrieval * length + n_streaming * min(length, sink + recent)) * d


def budget_ratio(retrieval_fraction: float, length: int, sink: int, recent: int) -> float:
    """Retained KV over full KV for a retrieval fraction r: (r L + (1 - r)(S + R)) / L.

    This is the memory formula above divided by H * L * d. The OpenReview thread's worked
    budget ratios (64K tokens, 50 % retrieval, 64 sinks + 256 recent) use the same terms.
    """
    r = retrieval_fraction
    return (r * length + (1.0 - r) * min(length, sink + recent)) / length


# --------------------------------------------------------------------------------------------
# From trained gates to the deployed head split
# --------------------------------------------------------------------------------------------

def retrieval_count(n_heads: int, ratio: float) -> int:
    """Number of retrieval heads for a target retrieval ratio over ``n_heads`` KV heads.

    Explainer, "Binarization: From Continuous Gates to Hard Assignments": the threshold is set
    so that a target fraction of the heads (25 % for the MHA model, 50 % for the GQA models)
    become retrieval heads. Reading: the count nearest to ratio * n_heads, halves rounded up,
    clamped to [0, n_heads], the product being taken in double precision (so 0.7 * 5, which
    rounds to 3.5, gives 4).
    """
    if not (0.0 <= ratio <= 1.0):
        raise ValueError("ratio must lie in [0, 1]")
    return max(0, min(n_heads, int(math.floor(ratio * n_heads + 0.5))))


def binarize_gates(alpha, ratio: float):
    """Hard retrieval/streaming assignment from the gate values ``alpha [L][H_kv]``.

    Explainer, same section, Equation 4: head (i, j) keeps full attention when its gate
    exceeds a threshold tau, and streaming attention otherwise, with tau placed at the
    quantile that leaves the target fraction of all heads of the model as retrieval heads.

    Reading: the quantile runs over every KV head of every layer together. Heads are ranked
    by decreasing gate value; equal values are ranked by layer, then head, ascending (the
    pages leave ties open). The first ``retrieval_count`` heads of that ranking are the
    retrieval heads, and tau is the gate of the first head left out (-inf when every head is
    kept), so that "alpha > tau" is exactly the retrieval set whenever no other head shares
    tau's value. Returns ``(mask uint8 [L][H_kv], tau)``.
    """
    a = np.asarray(alpha, dtype=np.float64)
    if a.ndim != 2 or not np.all(np.isfinite(a)):
        raise ValueError("alpha must be a finite [layers][kv_heads] array")
    L, H = a.shape
    k = retrieval_count(L * H, ratio)
    ranking = sorted(((layer, head) for layer in range(L) for head in range(H)),
                     key=lambda lh: (-a[lh], lh[0], lh[1]))
    mask = np.zeros((L, H), dtype=np.uint8)
    for lh in ranking[:k]:
        mask[lh] = 1
    tau = a[ranking[k]] if k < L * H else -math.inf
    return mask, float(tau)


def head_order(mask_layer) -> np.ndarray:
    """Native KV head at each position of the reordered layout of one layer.

    Explainer, "Head Reordering Preprocessing": the projection weights are permuted so that
    the retrieval heads take the first H_r head slots and the streaming heads the remaining
    H_s. Reading: each class keeps its native order (a stable partition).
    """
    m = np.asarray(mask_layer).astype(bool)
    return np.array([j for j in range(m.size) if m[j]] + [j for j in range(m.size) if not m[j]],
                    dtype=np.int64)


def query_head_order(kv_order, group: int) -> np.ndarray:
    """Native query head at each reordered query position: the G query heads of a KV head
    move with it, in their own order (same section; the same permutation must hold across Q,
    K and V, and a KV head serves the contiguous group of ``kv_head_of``)."""
    return np.array([j * group + g for j in kv_order for g in range(group)], dtype=np.int64)


def reorder_output_rows(w, order, rows_per_head: int) -> np.ndarray:
    """Rows of a Q, K or V projection weight ``[heads * rows_per_head][hidden]`` with head
    blocks in the reordered layout: block i of the result is block ``order[i]`` of ``w``."""
    w = np.asarray(w)
    return np.concatenate([w[h * rows_per_head:(h + 1) * rows_per_head] for h in order], axis=0)


def reorder_input_cols(w, order, cols_per_head: int) -> np.ndarray:
    """Columns of the output projection ``[hidden][heads * cols_per_head]`` permuted the same
    way, so that it reads the concatenated head outputs of the reordered layout (explainer,
    same section: reordering the heads and the output projection together leaves the layer's
    output unchanged)."""
    w = np.asarray(w)
    return np.concatenate([w[:, h * cols_per_head:(h + 1) * cols_per_head] for h in order],
                          axis=1)


# --------------------------------------------------------------------------------------------
# 4-bit (and 8-bit) retrieval caches
# --------------------------------------------------------------------------------------------
#
# Explainer, "Combination with Quantization" and the OpenReview reply on KV quantization:
# DuoAttention's full caches combine with 4-bit KV quantization (per-channel, as in KIVI);
# the explainer's "Category 3: KV Cache Quantization" names 4-bit or 8-bit storage. The pages
# fix the bit width only. Readings taken here, each a plain choice (L = 2^bits - 1 levels
# above zero: 15 for 4 bits, 255 for 8):
#   * asymmetric codes 0..L with a scale and zero point stored in bfloat16 (round to
#     nearest even of the float32 scale (max - min) / L and of the minimum);
#   * keys per channel over aligned groups of KV4_GROUP = 128 tokens (positions g*128 ..
#     g*128+127), values per token over the channels;
#   * the tokens of the last, incomplete group are kept exactly (bf16) until it completes;
#   * the code decision is taken in float32 against the stored values: c = rint((x - zero) /
#     scale) clamped to 0..L, and c = 0 when scale is 0 (IEEE float32 division, round half to
#     even), so that any float32 implementation takes the same decision;
#   * a stored token reads back as c * scale + zero with the stored scale and zero.

KV4_GROUP = 128


def to_bf16(x) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), returned as float32."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def kv4_codes(x, axis: int, bits: int = 4):
    """``bits``-bit codes (4 or 8) of a float32 block over ``axis`` (the reduction axis of
    min and max). Returns ``(codes uint8, scale, zero)``: the stored bfloat16 scale and zero
    (as float32), reduced over ``axis``."""
    levels = np.float32((1 << bits) - 1)
    x = np.asarray(x, dtype=np.float32)
    mn = to_bf16(x.min(axis=axis, keepdims=True))
    mx = x.max(axis=axis, keepdims=True)
    scale = to_bf16((mx - x.min(axis=axis, keepdims=True)) / levels)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.rint((x - mn) / scale)
    c = np.where(scale == 0, np.float32(0.0), c)
    codes = np.clip(c, 0, levels).astype(np.uint8)
    return codes, np.squeeze(scale, axis), np.squeeze(mn, axis)


def kv4_history(x_hist, n: int, is_key: bool, bits: int = 4) -> np.ndarray:
    """What a ``bits``-bit full cache reads back for tokens 0..n-1 of one head,
    ``x_hist [>=n, d]`` (float64 of the stored values): complete groups dequantized (keys per
    channel over the group, values per token), the incomplete last group exact."""
    x = np.asarray(x_hist, dtype=np.float32)[:n]
    out = x.astype(np.float64).copy()
    full = (n // KV4_GROUP) * KV4_GROUP
    for g0 in range(0, full, KV4_GROUP):
        blk = x[g0:g0 + KV4_GROUP]
        if is_key:
            codes, scale, zero = kv4_codes(blk, axis=0, bits=bits)  # per channel
            out[g0:g0 + KV4_GROUP] = (codes.astype(np.float64) * scale.astype(np.float64)[None, :]
                                      + zero.astype(np.float64)[None, :])
        else:
            codes, scale, zero = kv4_codes(blk, axis=1, bits=bits)  # per token
            out[g0:g0 + KV4_GROUP] = (codes.astype(np.float64) * scale.astype(np.float64)[:, None]
                                      + zero.astype(np.float64)[:, None])
    return out


def decode_step_kv4(q, k_hist, v_hist, retrieval, sink, recent, scale=None, rope_theta=None,
                    bits: int = 4):
    """``decode_step`` with the retrieval heads' full caches stored in ``bits`` bits (4 or 8):
    every retrieval KV head attends over ``kv4_history`` of its keys and values; streaming
    heads (constant-size caches, kept exact) as before.

    With ``rope_theta`` the keys of every head are pre-RoPE: the 4-bit codes are taken of the
    keys as given, and each key that attention reads (dequantized on retrieval heads, exact on
    streaming heads) is rotated at its own position by ``rope`` (see below); ``q`` is the
    query after its own rotation."""
    k = np.asarray(k_hist, dtype=np.float64).copy()
    v = np.asarray(v_hist, dtype=np.float64).copy()
    n = k.shape[0]
    for j in range(k.shape[1]):
        if retrieval[j]:
            k[:, j] = kv4_history(k_hist[:, j], n, True, bits)
            v[:, j] = kv4_history(v_hist[:, j], n, False, bits)
    if rope_theta:
        k = rope(k, np.arange(n), rope_theta)
    return decode_step(q, k, v, retrieval, sink, recent, scale)


def kv4_history_f32(x_hist, n: int, is_key: bool, bits: int = 4) -> np.ndarray:
    """``kv4_history`` as a float32 dequantizer computes it: every dequantized value is
    ``float32(c * scale + zero)`` (c * scale is exact in float32: at most 8 + 8 significant
    bits; one float32 rounding for the sum), the residual tokens exact. float32 ``[n, d]``."""
    x = np.asarray(x_hist, dtype=np.float32)[:n]
    out = x.copy()
    full = (n // KV4_GROUP) * KV4_GROUP
    for g0 in range(0, full, KV4_GROUP):
        blk = x[g0:g0 + KV4_GROUP]
        codes, scale, zero = kv4_codes(blk, axis=0 if is_key else 1, bits=bits)
        c = codes.astype(np.float32)
        if is_key:
            y = c * scale[None, :] + zero[None, :]
        else:
            y = c * scale[:, None] + zero[:, None]
        out[g0:g0 + KV4_GROUP] = y.astype(np.float32)
    return out


def kv4_history_bf16(x_hist, n: int, is_key: bool, bits: int = 4) -> np.ndarray:
    """``kv4_history`` read back in the cache dtype: ``kv4_history_f32`` rounded to the nearest
    bfloat16 (ties to even); the residual tokens, bf16 already, stay exact. float64 ``[n, d]``."""
    return to_bf16(kv4_history_f32(x_hist, n, is_key, bits)).astype(np.float64)


def prefill_chunk_kv4(q, k_hist, v_hist, start, retrieval, sink, recent, scale=None,
                      chunk_granular=False, bits: int = 4, rope_theta=None):
    """``prefill_chunk`` over a cache whose retrieval heads are stored in ``bits`` bits (4 or
    8). Reading (the pages pair quantized caches with serving the whole context, explainer,
    "Combination with Quantization"): the chunk's queries see the cache as it stands before
    the chunk, so a retrieval head's earlier tokens 0..start-1 read back as
    ``kv4_history_bf16(.., start)``: complete groups dequantized into the cache dtype, as a
    dequantize-then-attend kernel computes them, the last incomplete group exact. The chunk's
    own keys and values are exact (they are not in the cache yet; the caller appends them
    afterwards). Streaming heads are exact, as in decoding.

    With ``rope_theta`` the cache holds pre-RoPE keys (the 4-bit reading of the OpenReview
    thread, below) and ``k_hist`` holds every key as appended, before RoPE; ``q`` is the
    chunk's queries after their own rotation. Reading: every key the chunk attends to is
    turned at its own position and read in the cache dtype, as a kernel that stages the keys
    for a bf16 prefill computes them: ``to_bf16(rope(x, t))`` of the float32 dequantized key
    (``kv4_history_f32``) for a retrieval head's earlier tokens, and of the key as given for
    the chunk's own keys and for every streaming head. Values are as without RoPE."""
    k = np.asarray(k_hist, dtype=np.float64).copy()
    v = np.asarray(v_hist, dtype=np.float64).copy()
    if rope_theta:
        pos = np.arange(k.shape[0])
        k = to_bf16(rope(k, pos, rope_theta)).astype(np.float64)
    for j in range(k.shape[1]):
        if retrieval[j] and start > 0:
            if rope_theta:
                kd = kv4_history_f32(k_hist[:, j], start, True, bits)
                k[:start, j] = to_bf16(rope(kd, np.arange(start), rope_theta)).astype(np.float64)
            else:
                k[:start, j] = kv4_history_bf16(k_hist[:, j], start, True, bits)
            v[:start, j] = kv4_history_bf16(v_hist[:, j], start, False, bits)
    return prefill_chunk(q, k, v, start, retrieval, sink, recent, scale, chunk_granular)


# --------------------------------------------------------------------------------------------
# Pre-RoPE keys in 4-bit caches
# --------------------------------------------------------------------------------------------
#
# OpenReview thread, the authors' reply on combining DuoAttention with KV quantization: their
# 4-bit results quantize the keys before the rotary position embedding (RoPE) is applied. The
# pages name the technique only. Readings taken here:
#   * the caller appends every key of the layer before RoPE and passes each query after RoPE
#     at its own position (its usual form); attention rotates each key at its own position t:
#     after dequantization on a retrieval head, the exact stored key on a streaming head (at
#     its original position, as for the caller-rotated keys of the other caches);
#   * RoPE in its rotate-half form: channel i < d/2 pairs with channel i + d/2, and the pair
#     turns by the angle t * theta^(-2i/d), angles taken exactly (here in float64).

def rope_angles(pos, d: int, theta: float) -> np.ndarray:
    """float64 ``[len(pos), d/2]``: the angle of channel pair i at position t,
    t * theta**(-2 i / d)."""
    i = np.arange(d // 2, dtype=np.float64)
    inv = np.power(float(theta), -2.0 * i / d)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope(x, pos, theta: float) -> np.ndarray:
    """Rows ``x [n, ..., d]`` rotated at positions ``pos [n]``: channels (i, i + d/2) of row t
    turn by ``rope_angles`` (x_i cos - x_{i+d/2} sin, x_i sin + x_{i+d/2} cos)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    a = rope_angles(pos, d, theta)
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (h,)
    c = np.cos(a).reshape(shape)
    s = np.sin(a).reshape(shape)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)
