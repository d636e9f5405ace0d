"""duo_attn_prefill_staged: pre-filling over 4-bit and 8-bit caches on the GPU against the CPU
float64 oracle (prefill_chunk_kv4: a retrieval head's earlier tokens as the quantized cache
reads them back in bf16, the chunk's own keys and values exact; with pre-RoPE keys every key
turned at its position and read in bf16).

A prompt is processed in chunks: staged prefill of the chunk (compared with the oracle), then
the append of the same K/V, which quantizes every group the chunk completes.
|gpu - ref| <= 2e-3 + 1e-2 |ref| elementwise.
"""
import numpy as np
import pytest
import torch

import head_split_kv_amd as hsk
import workloads as W
from oracle import duo_oracle as O

from gpu_util import assert_close, to_dev

pytestmark = pytest.mark.gpu


def kvq_cache(w, capacity, bits, mode="window", out_dtype=torch.float32, rope_theta=0.0):
    return hsk.DuoCache(num_layers=1, batch=w.batch, num_q_heads=w.hq, num_kv_heads=w.hkv,
                        head_dim=w.d, sink=w.sink, recent=w.recent, capacity=capacity,
                        retrieval_mask=W.retrieval_mask(w)[:1], dtype=torch.bfloat16,
                        out_dtype=out_dtype, kv_bits=bits, streaming_prefill=mode,
                        rope_theta=rope_theta)


def staging_need(w, mask, nb, c_max, m, rope):
    """duo_prefill_staging_bytes as the header states it: the prefix keys and values, with
    pre-RoPE keys the chunk's and the streaming keys, then the chunk's and the streaming
    values (fp16), each region but the last rounded up to 256 bytes."""
    row = w.d * 2
    up = lambda x: (x + 255) // 256 * 256
    chunk = nb * m * w.hkv * row
    streaming = w.batch * int((mask == 0).sum()) * (w.sink + w.recent) * row
    end = 2 * nb * int(mask.sum()) * c_max * row
    if rope:
        end = up(end) + up(chunk) + streaming
    return up(end) + up(chunk) + streaming


def run_prefill_kvq(w, lens, chunks, bits, mode="window", seqwise=False, heads=None,
                    out_dtype=torch.float32, rope_theta=None):
    """Prefill prompts of lengths ``lens`` in chunks of the sizes ``chunks`` (cycled), each
    checked on every row (on the KV heads ``heads`` and their query heads when given). With
    ``rope_theta`` the cache holds pre-RoPE keys: the keys drawn are taken as before RoPE and
    the queries as after it."""
    cache = kvq_cache(w, max(lens) + 1, bits, mode, out_dtype, rope_theta or 0.0)
    dt = torch.bfloat16
    mask = W.retrieval_mask(w)[0]
    heads = list(range(w.hkv)) if heads is None else heads
    qh_idx = [j * w.group + g for j in heads for g in range(w.group)]

    def plan_for(n):
        out, c0, i = [], 0, 0
        while c0 < n:
            c1 = min(n, c0 + chunks[i % len(chunks)])
            out.append((c0, c1))
            c0, i = c1, i + 1
        return out

    if seqwise:
        plan = [(b, c0, c1) for b, n in enumerate(lens) for c0, c1 in plan_for(n)]
    else:
        assert len(set(lens)) == 1
        plan = [(-1, c0, c1) for c0, c1 in plan_for(lens[0])]
    for b, c0, c1 in plan:
        seqs = range(w.batch) if b < 0 else [b]
        q = np.stack([W.tokens(w, "q", 0, s, c0, c1) for s in seqs])
        k = np.stack([W.tokens(w, "k", 0, s, c0, c1) for s in seqs])
        v = np.stack([W.tokens(w, "v", 0, s, c0, c1) for s in seqs])
        dq, dk, dv = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
        if b >= 0:
            dq, dk, dv = dq[0], dk[0], dv[0]
        shape = (dq.shape[0], c1 - c0, w.hq) if b < 0 else (c1 - c0, w.hq)
        lse = torch.empty(shape, dtype=torch.float32, device="cuda")
        need = hsk.duo_prefill_staging_bytes(cache, 0, b, c1 - c0)
        c_max = max(cache.lengths()[0][s] for s in seqs)
        assert need == staging_need(w, mask, len(seqs), c_max, c1 - c0, bool(rope_theta))
        out = cache.attn_prefill_staged(0, dq, dk, dv, seq=b, lse=lse)
        cache.kv_append(0, dk, dv, seq=b)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        got_lse = lse.cpu().numpy()
        if b >= 0:
            got, got_lse = got[None], got_lse[None]
        for si, s in enumerate(seqs):
            kh = W.tokens(w, "k", 0, s, 0, c1)[:, heads]
            vh = W.tokens(w, "v", 0, s, 0, c1)[:, heads]
            qc = W.tokens(w, "q", 0, s, c0, c1)[:, qh_idx]
            ref, ref_lse = O.prefill_chunk_kv4(qc, kh, vh, c0, mask[heads], w.sink, w.recent,
                                               chunk_granular=mode == "chunk", bits=bits,
                                               rope_theta=rope_theta)
            assert_close(got[si][:, qh_idx], ref, f"{bits}-bit chunk [{c0},{c1}) seq {s} out")
            assert_close(got_lse[si][:, qh_idx], ref_lse,
                         f"{bits}-bit chunk [{c0},{c1}) seq {s} lse")
    return cache


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_prefill_kvq_variants(bits, d, G):
    """Chunks whose earlier tokens hold complete groups and residual rows (prefixes 0, 170,
    340), both head classes."""
    w = W.Workload("kvq-prefill", 1, 2, 2 * G, 2, d, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=401 + G)
    run_prefill_kvq(w, [500, 500], [170], bits)


@pytest.mark.parametrize("bits", [4, 8])
def test_prefill_kvq_ragged_seqwise_and_group_edges(bits):
    """Ragged prompts pre-filled one sequence at a time, with chunks ending on group edges
    (prefix 128 and 256: no residual rows), one token past them, and single tokens."""
    w = W.Workload("kvq-ragged", 1, 3, 16, 4, 128, "bf16", 16, 64, 0, 0, 2, seed=411)
    run_prefill_kvq(w, [300, 521, 129], [128, 1, 127, 1, 120], bits, seqwise=True)


def test_prefill_kvq_chunk_mode_and_bf16_out():
    w = W.Workload("kvq-chunkmode", 1, 2, 8, 4, 128, "bf16", 4, 64, 0, 0, 2,
                   fixed_mask=((1, 2),), seed=413)
    run_prefill_kvq(w, [600, 600], [200], 4, mode="chunk")
    run_prefill_kvq(w, [400, 400], [150], 8, out_dtype=torch.bfloat16)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("bits", [4, 8])
def test_prefill_kvq_mha_8k(bits):
    """The Llama-2-7B-shaped MHA layer (32 heads, 8 retrieval) over an 8K prompt in 2K chunks,
    checked on two retrieval heads and one streaming head."""
    w = W.workload("c2")
    mask = W.retrieval_mask(w)[0]
    ret = [int(j) for j in np.nonzero(mask)[0]]
    heads = [ret[0], ret[-1], int(np.nonzero(mask == 0)[0][0])]
    run_prefill_kvq(w, [8192], [2048], bits, heads=heads)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4])
def test_prefill_kvq_rope_variants(bits, d, G):
    """Pre-RoPE keys: the retrieval prefix (complete groups and residual rows), the chunk's
    keys and the streaming slots (sinks, and a ring that wraps: prompts of 500 against
    S + R = 36) are staged turned."""
    w = W.Workload("kvq-rope", 1, 2, 2 * G, 2, d, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=421 + G)
    run_prefill_kvq(w, [500, 500], [170], bits, rope_theta=10000.0)


def test_prefill_kvq_rope_ragged_seqwise_and_chunk_mode():
    """Ragged prompts one sequence at a time (chunks on and past group edges, single tokens),
    then chunk-granular streaming heads, both with pre-RoPE keys."""
    w = W.Workload("kvq-rope-ragged", 1, 3, 16, 4, 128, "bf16", 16, 64, 0, 0, 2, seed=431)
    run_prefill_kvq(w, [300, 521, 129], [128, 1, 127, 1, 120], 4, seqwise=True,
                    rope_theta=500000.0)
    w = W.Workload("kvq-rope-chunkmode", 1, 2, 8, 4, 128, "bf16", 4, 64, 0, 0, 2,
                   fixed_mask=((1, 2),), seed=433)
    run_prefill_kvq(w, [600, 600], [200], 8, mode="chunk", rope_theta=10000.0)


def test_prefill_kvq_rope_streaming_only_layer():
    """A layer whose KV heads are all streaming: no prefix to read back, the chunk's keys and
    the streaming slots still turned (duo_attn_prefill refuses such a layer of a pre-RoPE
    cache)."""
    w = W.Workload("kvq-rope-str", 1, 1, 8, 2, 64, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((),), seed=437)
    run_prefill_kvq(w, [300], [100], 4, rope_theta=10000.0)


@pytest.mark.timeout(600)
def test_prefill_kvq_rope_gqa_16k():
    """The Llama-3-8B-shaped GQA layer (32 q / 8 KV heads, 4 retrieval, base 500,000) over a
    16K prompt in 4K chunks with pre-RoPE 4-bit keys, checked on two retrieval heads and one
    streaming head."""
    w = W.workload("c3")
    mask = W.retrieval_mask(w)[0]
    ret = [int(j) for j in np.nonzero(mask)[0]]
    heads = [ret[0], ret[-1], int(np.nonzero(mask == 0)[0][0])]
    run_prefill_kvq(w, [16384], [4096], 4, heads=heads, rope_theta=500000.0)
