"""4-bit and 8-bit full caches (cfg.kv_bits = 4 or 8) on the GPU against the CPU oracle.

Append: the stored codes, bf16 scales and zeros, and the bf16 residual rows are compared
bit for bit with the oracle's kv4_codes, through the byte layout documented in duo.h.
Decode: outputs against decode_step_kv4 (retrieval heads attend over what the quantized
caches read back), |gpu - ref| <= 2e-3 + 1e-2 |ref|.
"""
import numpy as np
import pytest
import torch

import head_split_kv_amd as hsk
import workloads as W
from oracle import duo_oracle as O

from gpu_util import assert_close, step_inputs, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

QG = O.KV4_GROUP


def kv4_cache(w, capacity, out_dtype=torch.float32, mask=None, rope_theta=0.0, bits=4):
    mask = W.retrieval_mask(w) if mask is None else mask
    return hsk.DuoCache(num_layers=mask.shape[0], batch=w.batch, num_q_heads=w.hq,
                        num_kv_heads=w.hkv, head_dim=w.d, sink=w.sink, recent=w.recent,
                        capacity=capacity, retrieval_mask=mask, dtype=torch.bfloat16,
                        out_dtype=out_dtype, kv_bits=bits, rope_theta=rope_theta)


def geom(cap, D, bits=4):
    groups = -(-cap // QG)
    codes = groups * QG * D * bits // 8
    params = max(groups * 2 * D * 2, groups * QG * 4)
    resid = QG * D * 2
    return codes, params, resid, codes + params + resid


def head_region(cache, is_v, b, r):
    """Raw bytes of retrieval head r of sequence b (layer 0) as a numpy uint8 array."""
    codes, params, resid, stride = geom(cache.capacity, cache.d, cache.kv_bits)
    hr = int(cache.retrieval_mask[0].sum())
    off = (cache.layout.full_v_off if is_v else cache.layout.full_k_off) + (b * hr + r) * stride
    return cache.arena[off:off + stride].cpu().numpy(), codes, params


def nibbles(words):
    """uint32 words -> their 8 codes each (element e in bits 4e .. 4e + 3)."""
    w = np.asarray(words, dtype=np.uint32)
    return ((w[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 15).astype(np.uint8)


def unpack_keys(code_bytes, rows, D, bits=4):
    """Key codes [rows][D]. 4 bits: row words in slot KC j + kc hold channels 32 kc + 8 j ..
    + 7. 8 bits: slot 2 KC j + 2 kc + h holds channels 32 kc + 8 j + 4 h .. + 3, one a byte."""
    KC = D // 32
    out = np.empty((rows, D), dtype=np.uint8)
    if bits == 4:
        w = code_bytes[:rows * D // 2].view(np.uint32).reshape(rows, D // 8)
        for slot in range(D // 8):
            c0 = 32 * (slot % KC) + 8 * (slot // KC)
            out[:, c0:c0 + 8] = nibbles(w[:, slot])
        return out
    b = code_bytes[:rows * D].reshape(rows, D // 4, 4)
    for slot in range(D // 4):
        j, kc, h = slot // (2 * KC), (slot % (2 * KC)) // 2, slot % 2
        c0 = 32 * kc + 8 * j + 4 * h
        out[:, c0:c0 + 4] = b[:, slot]
    return out


def unpack_values(code_bytes, groups, D, bits=4):
    """Value codes [groups * QG][D]. 4 bits: word ((s (D / 64) + h) 64 + 16 j + c % 16) 4 + w
    of a group, with c / 16 = 4 h + w, holds channel c; its element e is token 32 s +
    16 (e / 4) + 4 j + e % 4. 8 bits: word ((s (D / 32) + h) 64 + 16 j + c % 16) 4 + u, with
    c / 16 = 2 h + u / 2, holds channel c; its byte e is token 32 s + 16 (u % 2) + 4 j + e."""
    if bits == 8:
        chunks = D // 32
        b = code_bytes[:groups * QG * D].reshape(groups, 4, chunks, 4, 16, 4, 4)
        out = np.empty((groups, QG, D), dtype=np.uint8)
        for s_ in range(4):
            for h in range(chunks):
                for j in range(4):
                    for cl in range(16):
                        for u in range(4):
                            c = 16 * (2 * h + u // 2) + cl
                            t0 = 32 * s_ + 16 * (u % 2) + 4 * j
                            out[:, t0:t0 + 4, c] = b[:, s_, h, j, cl, u]
        return out.reshape(groups * QG, D)
    halves = D // 64
    w = code_bytes[:groups * QG * D // 2].view(np.uint32).reshape(groups, 4, halves, 4, 16, 4)
    out = np.empty((groups, QG, D), dtype=np.uint8)
    e = np.arange(8)
    for s in range(4):
        for h in range(halves):
            for j in range(4):
                toks = 32 * s + 16 * (e // 4) + 4 * j + e % 4
                for cl in range(16):
                    for ww in range(4):
                        out[:, toks, 16 * (4 * h + ww) + cl] = nibbles(w[:, s, h, j, cl, ww])
    return out.reshape(groups * QG, D)


def check_stored(cache, w, lens):
    """Every retrieval head of every sequence: complete groups' codes and parameters equal
    the oracle's, residual rows equal the input bits."""
    D, bits = w.d, cache.kv_bits
    ret = np.nonzero(cache.retrieval_mask[0])[0]
    for b, n in enumerate(lens):
        ng = n // QG
        for r, j in enumerate(ret):
            for is_v in (False, True):
                x = W.tokens(w, "v" if is_v else "k", 0, b, 0, n)[:, j].astype(np.float32)
                raw, codes_b, params_b = head_region(cache, is_v, b, r)
                codes = (unpack_values(raw, ng, D, bits) if is_v
                         else unpack_keys(raw, ng * QG, D, bits))
                par = raw[codes_b:codes_b + params_b]
                for g in range(ng):
                    blk = x[g * QG:(g + 1) * QG]
                    c, s, z = O.kv4_codes(blk, axis=1 if is_v else 0, bits=bits)
                    assert np.array_equal(codes[g * QG:(g + 1) * QG], c), (b, j, is_v, g)
                    hi16 = lambda f: (f.view(np.uint32) >> 16).astype(np.uint16)  # noqa: E731
                    if is_v:  # one word per token: bf16 scale low, bf16 zero high
                        got = par.view(np.uint16)[2 * g * QG:2 * (g + 1) * QG].reshape(QG, 2)
                    else:     # bf16 [2][D] per group
                        got = par.view(np.uint16)[g * 2 * D:(g + 1) * 2 * D].reshape(2, D).T
                    assert np.array_equal(got[:, 0], hi16(s)), (b, j, is_v, g)
                    assert np.array_equal(got[:, 1], hi16(z)), (b, j, is_v, g)
                res = raw[codes_b + params_b:].view(np.uint16).reshape(QG, D)
                want = (x[ng * QG:n].view(np.uint32) >> 16).astype(np.uint16)
                got_rows = res[np.arange(ng * QG, n) % QG]
                assert np.array_equal(got_rows, want), (b, j, is_v, "residual")


def append_tokens(cache, w, b, t0, t1):
    dt = torch_dtype(w.dtype)
    k = to_dev(W.tokens(w, "k", 0, b, t0, t1), dt)
    v = to_dev(W.tokens(w, "v", 0, b, t0, t1), dt)
    cache.kv_append(0, k, v, seq=b)


def test_kv4_append_patterns_bit_exact():
    """Bulk appends, single tokens across a group boundary, chunks that complete a group
    holding residual rows and leave a new tail, and ragged sequences."""
    w = W.Workload("kv4-append", 1, 3, 8, 4, 128, "bf16", 4, 32, 0, 0, 2,
                   fixed_mask=((0, 2),), seed=101)
    cache = kv4_cache(w, 1200)
    lens = [0, 0, 0]
    plan = [(0, 300), (1, 1), (2, 128), (0, 1), (0, 83), (1, 126), (1, 1), (1, 1), (2, 257),
            (0, 5), (1, 500), (2, 1)]
    for b, m in plan:
        append_tokens(cache, w, b, lens[b], lens[b] + m)
        lens[b] += m
        torch.cuda.synchronize()
        check_stored(cache, w, lens)
    assert list(cache.lengths()[0]) == lens


@pytest.mark.parametrize("d", [64, 128])
def test_kv4_append_batch_calls(d):
    """Appends to every sequence at once (seq = -1), chunk sizes that straddle groups."""
    w = W.Workload("kv4-append-batch", 1, 2, 4, 2, d, "bf16", 2, 16, 0, 0, 1,
                   fixed_mask=((1,),), seed=103)
    cache = kv4_cache(w, 1000)
    dt = torch_dtype(w.dtype)
    n = 0
    for m in (1, 126, 2, 127, 128, 300, 1):
        k = to_dev(np.stack([W.tokens(w, "k", 0, b, n, n + m) for b in range(2)]), dt)
        v = to_dev(np.stack([W.tokens(w, "v", 0, b, n, n + m) for b in range(2)]), dt)
        cache.kv_append(0, k, v)
        n += m
        torch.cuda.synchronize()
        check_stored(cache, w, [n, n])


def run_decode_kv4(w, lens0, steps, check_steps=None, splits=None, out_dtype=torch.float32,
                   fused=False, heads=None, rope_theta=None, bits=4):
    cache = kv4_cache(w, max(lens0) + steps, out_dtype=out_dtype, rope_theta=rope_theta or 0.0,
                      bits=bits)
    for b, n in enumerate(lens0):
        for t0 in range(0, n, 1 << 16):
            append_tokens(cache, w, b, t0, min(n, t0 + (1 << 16)))
    if splits is not None:
        hsk.duo_set_decode_splits(cache, splits)
    mask = W.retrieval_mask(w)[0]
    lens = list(lens0)
    for s in range(steps):
        q, k, v, qh = step_inputs(w, 0, lens)
        lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device="cuda")
        if fused:
            out = cache.decode_step(0, q, k[:, 0], v[:, 0], lse=lse)
        else:
            cache.kv_append(0, k, v)
            out = cache.attn_decode(0, q, lse=lse)
        lens = [n + 1 for n in lens]
        if check_steps is not None and s not in check_steps:
            continue
        torch.cuda.synchronize()
        got, got_lse = out.float().cpu().numpy(), lse.cpu().numpy()
        for b, n in enumerate(lens):
            kh, vh = W.tokens(w, "k", 0, b, 0, n), W.tokens(w, "v", 0, b, 0, n)
            if heads is None:
                ref, ref_lse = O.decode_step_kv4(qh[b], kh, vh, mask, w.sink, w.recent,
                                                 rope_theta=rope_theta, bits=bits)
                assert_close(got[b], ref, f"step {s} seq {b} n {n} out")
                assert_close(got_lse[b], ref_lse, f"step {s} seq {b} n {n} lse")
            else:
                G = w.group
                for j in heads:
                    hq = slice(j * G, (j + 1) * G)
                    ref, ref_lse = O.decode_step_kv4(qh[b][hq], kh[:, j:j + 1], vh[:, j:j + 1],
                                                     mask[j:j + 1], w.sink, w.recent,
                                                     rope_theta=rope_theta, bits=bits)
                    assert_close(got[b][hq], ref, f"step {s} seq {b} kv {j}")
                    assert_close(got_lse[b][hq], ref_lse, f"step {s} seq {b} kv {j} lse")
    return cache


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_kv4_decode_variants(d, G):
    """Every (head_dim, group) variant; a context crossing several groups, steps across the
    next group boundary (the completing append re-quantizes the residual)."""
    w = W.Workload("kv4-variant", 1, 2, 2 * G, 2, d, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=105 + G)
    run_decode_kv4(w, [3 * QG - 2, 2 * QG + 40], 4)


@pytest.mark.parametrize("n0", [1, QG - 1, QG, QG + 1, 5 * QG + 17])
def test_kv4_decode_lengths(n0):
    """Contexts inside the first group (residual only), at group edges and past several."""
    w = W.Workload("kv4-len", 1, 1, 16, 4, 128, "bf16", 16, 64, 0, 0, 2,
                   fixed_mask=((1, 2),), seed=107)
    run_decode_kv4(w, [n0], 3)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
def test_kv4_decode_split_counts(splits):
    """Groups dealt to 1..16 splits: some splits with no group, leftover groups by steps (1
    and 2 splits) or whole (3 and more), the residual rows in a block of their own."""
    w = W.Workload("kv4-splits", 1, 1, 32, 8, 128, "bf16", 16, 64, 0, 0, 4, seed=109)
    run_decode_kv4(w, [9 * QG + 50], 2, splits=splits)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("n0", [300, 1000])
def test_kv4_decode_streaming_slices(fused, n0):
    """A streaming window of 4 + 500 slots is cut over several blocks (merged like retrieval
    splits): before the ring wraps and after, the fused step's token taken by the last block
    and the evicted slot skipped by every block."""
    w = W.Workload("kv4-slices", 1, 1, 16, 4, 64, "bf16", 4, 500, 0, 0, 2,
                   fixed_mask=((1, 2),), seed=119)
    run_decode_kv4(w, [n0], 3, fused=fused)


def test_kv4_decode_ragged_batch_bf16_out_and_streaming_only():
    w = W.Workload("kv4-ragged", 1, 3, 32, 8, 128, "bf16", 16, 64, 0, 0, 4, seed=111)
    run_decode_kv4(w, [700, 129, 1500], 2, out_dtype=torch.bfloat16)
    w2 = W.Workload("kv4-streaming", 1, 2, 8, 2, 128, "bf16", 4, 32, 0, 0, 0,
                    fixed_mask=((),), seed=113)
    run_decode_kv4(w2, [300, 40], 2)


def test_kv4_decode_step_from_empty():
    """duo_decode_step on a 4-bit cache from an empty cache through two group completions,
    every step checked."""
    w = W.Workload("kv4-step", 1, 1, 8, 2, 64, "bf16", 4, 16, 0, 0, 1,
                   fixed_mask=((1,),), seed=115)
    run_decode_kv4(w, [0], 2 * QG + 5, fused=True, check_steps=set(range(0, 2 * QG + 5, 7)) |
                   {QG - 1, QG, 2 * QG - 1, 2 * QG})


def test_kv4_rejects_prefill_and_gate_mixed():
    w = W.Workload("kv4-reject", 1, 1, 8, 2, 128, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=117)
    cache = kv4_cache(w, 256)
    dt = torch_dtype(w.dtype)
    q, k, v = (to_dev(W.tokens(w, t, 0, 0, 0, 16)[None], dt) for t in "qkv")
    with pytest.raises(hsk.DuoError) as e:
        cache.attn_prefill(0, q, k, v)
    assert e.value.status == hsk.DUO_ERR_UNSUPPORTED
    w2 = W.Workload("kv4-reject2", 1, 1, 8, 2, 128, "bf16", 4, 32, 0, 0, 2,
                    fixed_mask=((0, 1),), seed=117)
    cache2 = kv4_cache(w2, 256)
    with pytest.raises(hsk.DuoError) as e:
        cache2.attn_gate_mixed(0, q, k, v, [0.5, 0.5])
    assert e.value.status == hsk.DUO_ERR_UNSUPPORTED
    assert cache.lengths()[0][0] == 0 and cache2.lengths()[0][0] == 0


@pytest.mark.timeout(900)
def test_kv4_decode_gqa_128k():
    """Llama-3-8B-shaped GQA layer at a 128K context in 4 bits (the benchmark's shape): the
    steps cross the group boundary at 131,072 tokens."""
    w = W.workload("c3")
    run_decode_kv4(w, [w.context - 2], 4)


# ---- pre-RoPE keys (cfg.rope_theta > 0) ---------------------------------------------------
# Keys are appended before RoPE, queries are taken as already turned; the oracle turns each
# key at its position after dequantization (decode_step_kv4 with rope_theta).

THETA = 10000.0


def streaming_keys(cache, b, s):
    """bf16 slots [S + R][D] of streaming head index s of sequence b (layer 0) as float32."""
    lay, D, SR = cache.layout, cache.d, cache.sink + cache.recent
    hs = int((1 - cache.retrieval_mask[0]).sum())
    off = lay.str_k_off + ((b * hs + s) * SR) * D * 2
    raw = cache.arena[off:off + SR * D * 2].cpu().numpy().view(np.uint16).astype(np.uint32)
    return (raw << 16).view(np.float32).reshape(SR, D)


@pytest.mark.parametrize("d", [64, 128])
def test_kv4_rope_tables(d):
    """The cos/sin tables duo_cache_reset writes at layout.rope_off, against the oracle's
    angles: tau16 (fp16 pairs (8 b + w, 8 b + w + 4) of cos then sin of tau f_i, rows of
    d/2 + 4 words) and the base rows (float32 (cos, sin) of 128 g f_i)."""
    theta, cap = 500000.0, 3000
    w = W.Workload("kv4-rope-tables", 1, 1, 4, 2, d, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=243)
    cache = kv4_cache(w, cap, rope_theta=theta)
    torch.cuda.synchronize()
    lay = cache.layout
    raw = cache.arena[lay.rope_off:lay.rope_off + lay.rope_bytes].cpu().numpy()
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    half, nbase = d // 2, cap // QG + 1
    ob = al(QG * (half + 4) * 4)
    base = raw[ob:ob + nbase * d * 4].view(np.float32).reshape(nbase, half, 2)
    ang_t = O.rope_angles(np.arange(QG), d, theta)
    ang_b = O.rope_angles(QG * np.arange(nbase), d, theta)
    assert np.abs(base[..., 0] - np.cos(ang_b)).max() < 1e-6
    assert np.abs(base[..., 1] - np.sin(ang_b)).max() < 1e-6
    t16 = raw[:QG * (half + 4) * 4].view(np.float16).reshape(QG, 2 * (half + 4))
    i = np.arange(half)
    at = (i // 8) * 16 + 2 * (i % 4) + (i % 8) // 4
    assert np.abs(t16[:, at].astype(np.float64) - np.cos(ang_t)).max() <= 2.0 ** -11
    assert np.abs(t16[:, at + 8].astype(np.float64) - np.sin(ang_t)).max() <= 2.0 ** -11
    assert np.all(t16[:, 2 * half:] == 0)
    cache.close()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("path", ["residual", "groups", "streaming"])
def test_kv4_rope_each_path(d, path):
    """Each path alone with pre-RoPE keys: only bf16 residual rows (99 + 1 tokens), only
    complete groups (255 + 1 tokens), only streaming heads."""
    mask = ((),) if path == "streaming" else ((0, 1),)
    w = W.Workload("kv4-rope-path", 1, 1, 4, 2, d, "bf16", 4, 32, 0, 0, 0 if mask == ((),) else 2,
                   fixed_mask=mask, seed=241)
    n0 = {"residual": 99, "groups": 255, "streaming": 200}[path]
    run_decode_kv4(w, [n0], 1, rope_theta=THETA)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_kv4_rope_decode_variants(d, G):
    """Every (head_dim, group) variant with pre-RoPE keys: the MFMA path (dequantize, turn
    by the offset in the group, the query turned by the group base), the residual rows and
    the streaming heads, steps across a group boundary."""
    w = W.Workload("kv4-rope-variant", 1, 2, 2 * G, 2, d, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=205 + G)
    run_decode_kv4(w, [3 * QG - 2, 2 * QG + 40], 4, rope_theta=THETA)


def test_kv4_rope_append_keeps_keys_as_given():
    """With pre-RoPE keys every cache keeps the keys as given: the retrieval caches hold the
    oracle's codes of them, and every streaming slot the input bits of its position."""
    w = W.Workload("kv4-rope-append", 1, 2, 8, 4, 128, "bf16", 4, 64, 0, 0, 2,
                   fixed_mask=((0, 2),), seed=211)
    cache = kv4_cache(w, 3000, rope_theta=500000.0)
    lens = [2500, 300]
    for b, n in enumerate(lens):
        append_tokens(cache, w, b, 0, n - 7)
        for t in range(n - 7, n):  # single-token appends through the ring
            append_tokens(cache, w, b, t, t + 1)
    torch.cuda.synchronize()
    check_stored(cache, w, lens)
    str_heads = np.nonzero(1 - cache.retrieval_mask[0])[0]
    for b, n in enumerate(lens):
        table = O.slot_table(n, w.sink, w.recent)
        for s, j in enumerate(str_heads):
            got = streaming_keys(cache, b, s)
            kh = W.tokens(w, "k", 0, b, 0, n)[:, j].astype(np.float32)
            ok = table >= 0
            assert np.array_equal(got[ok], kh[table[ok]]), (b, j)


@pytest.mark.parametrize("fused", [False, True])
def test_kv4_rope_streaming_ring_and_fused(fused):
    """Streaming windows cut over several blocks before and after the ring wraps, each slot
    turned at the position it holds; the fused step's token is turned at its own position
    and stored as given (later steps read it back)."""
    w = W.Workload("kv4-rope-ring", 1, 1, 16, 4, 128, "bf16", 4, 500, 0, 0, 2,
                   fixed_mask=((1, 2),), seed=219)
    run_decode_kv4(w, [1000], 6, fused=fused, rope_theta=THETA)
    run_decode_kv4(w, [300], 3, fused=fused, rope_theta=THETA)


def test_kv4_rope_ragged_batch_splits_bf16_out():
    w = W.Workload("kv4-rope-ragged", 1, 3, 32, 8, 128, "bf16", 16, 64, 0, 0, 4, seed=223)
    run_decode_kv4(w, [700, 129, 1500], 2, out_dtype=torch.bfloat16, rope_theta=500000.0)
    w2 = W.Workload("kv4-rope-splits", 1, 1, 32, 8, 128, "bf16", 16, 64, 0, 0, 4, seed=227)
    for splits in (1, 3, 16):
        run_decode_kv4(w2, [9 * QG + 50], 1, splits=splits, rope_theta=THETA)


def test_kv4_rope_step_from_empty():
    """duo_decode_step with pre-RoPE keys from an empty cache through two group
    completions (append + decode), every few steps checked."""
    w = W.Workload("kv4-rope-step", 1, 1, 8, 2, 64, "bf16", 4, 16, 0, 0, 1,
                   fixed_mask=((1,),), seed=229)
    run_decode_kv4(w, [0], 2 * QG + 5, fused=True, rope_theta=THETA,
                   check_steps=set(range(0, 2 * QG + 5, 9)) | {QG - 1, QG, 2 * QG - 1, 2 * QG})


def test_kv4_rope_far_positions():
    """Positions near 20,000 with base 10,000: the group base angles are far from zero (the
    lowest pair turns by about 3,000 full turns)."""
    w = W.Workload("kv4-rope-far", 1, 1, 8, 2, 128, "bf16", 16, 64, 0, 0, 1,
                   fixed_mask=((0,),), seed=231)
    run_decode_kv4(w, [20000 - 3], 4, rope_theta=THETA)


@pytest.mark.timeout(900)
def test_kv4_rope_gqa_128k():
    """The Llama-3-8B-shaped GQA layer at a 128K context in 4 bits with pre-RoPE keys (base
    500,000, as that model's): steps across the group boundary at 131,072 tokens."""
    w = W.workload("c3")
    run_decode_kv4(w, [w.context - 2], 4, rope_theta=500000.0)


# ---- 8-bit caches (cfg.kv_bits = 8) --------------------------------------------------------

def test_kv8_append_patterns_bit_exact():
    """The 8-bit layouts bit for bit: bulk appends, single tokens across a group boundary,
    chunks that complete a group holding residual rows, ragged sequences, both head dims."""
    for d in (128, 64):
        w = W.Workload("kv8-append", 1, 3, 8, 4, d, "bf16", 4, 32, 0, 0, 2,
                       fixed_mask=((0, 2),), seed=301)
        cache = kv4_cache(w, 1200, bits=8)
        dt = torch_dtype(w.dtype)
        lens = [0, 0, 0]
        for b, chunks in enumerate(((300,), (127, 1, 1, 200), (1, 128, 500))):
            for m in chunks:
                k = to_dev(W.tokens(w, "k", 0, b, lens[b], lens[b] + m), dt)
                v = to_dev(W.tokens(w, "v", 0, b, lens[b], lens[b] + m), dt)
                cache.kv_append(0, k, v, seq=b)
                lens[b] += m
        torch.cuda.synchronize()
        check_stored(cache, w, lens)
        cache.close()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_kv8_decode_variants(d, G):
    """Every (head_dim, group) variant of the 8-bit kernel, steps across a group boundary."""
    w = W.Workload("kv8-variant", 1, 2, 2 * G, 2, d, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=305 + G)
    run_decode_kv4(w, [3 * QG - 2, 2 * QG + 40], 4, bits=8)


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_kv8_decode_split_counts_and_streaming(splits):
    w = W.Workload("kv8-splits", 1, 1, 32, 8, 128, "bf16", 16, 64, 0, 0, 4, seed=309)
    run_decode_kv4(w, [9 * QG + 50], 2, splits=splits, bits=8)
    w2 = W.Workload("kv8-slices", 1, 1, 16, 4, 64, "bf16", 4, 500, 0, 0, 2,
                    fixed_mask=((1, 2),), seed=311)
    run_decode_kv4(w2, [1000], 3, fused=splits == 3, bits=8)


def test_kv8_ragged_bf16_out_and_step_from_empty():
    w = W.Workload("kv8-ragged", 1, 3, 32, 8, 128, "bf16", 16, 64, 0, 0, 4, seed=313)
    run_decode_kv4(w, [700, 129, 1500], 2, out_dtype=torch.bfloat16, bits=8)
    w2 = W.Workload("kv8-step", 1, 1, 8, 2, 64, "bf16", 4, 16, 0, 0, 1,
                    fixed_mask=((1,),), seed=315)
    run_decode_kv4(w2, [0], QG + 5, fused=True, bits=8,
                   check_steps=set(range(0, QG + 5, 9)) | {QG - 1, QG})


@pytest.mark.parametrize("d", [64, 128])
def test_kv8_rope(d):
    """8-bit caches with pre-RoPE keys: quantized groups, residual rows and streaming heads."""
    w = W.Workload("kv8-rope", 1, 2, 8, 2, d, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=317)
    run_decode_kv4(w, [3 * QG - 2, 2 * QG + 40], 3, bits=8, rope_theta=THETA)


@pytest.mark.timeout(900)
def test_kv8_decode_gqa_128k():
    """The Llama-3-8B-shaped GQA layer at a 128K context in 8 bits."""
    w = W.workload("c3")
    run_decode_kv4(w, [w.context - 2], 3, bits=8)
