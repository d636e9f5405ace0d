"""duo_attn_prefill on the GPU against the CPU float64 oracle.

A prompt is processed in chunks: prefill attention of the chunk (compared with the oracle),
then the append of the same K/V. |gpu - ref| <= 2e-3 + 1e-2 |ref| elementwise.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import duo_oracle as O

from gpu_util import assert_close, make_cache, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def run_prefill(w, lens, chunk, layer=0, check_rows=None, cache=None, seqwise=False,
                out_dtype=torch.float32, rng_seed=0, mode="window"):
    """Prefill prompts of lengths ``lens`` in chunks of ``chunk``; returns the outputs.

    ``mode`` is the streaming-head prefill mode: "window" (per-query sink + recent mask) or
    "chunk" (the pruned cache before the chunk plus the chunk causally).

    ``check_rows``: None = every row, int = that many random rows per chunk and sequence.
    With ``seqwise`` every sequence is prefilled by its own calls (ragged prompts);
    otherwise all sequences share the chunk calls (equal lengths).
    """
    if cache is None:
        cache = make_cache(w, out_dtype=out_dtype, capacity=max(lens) + 1, streaming_prefill=mode)
    dt = torch_dtype(w.dtype)
    mask = W.retrieval_mask(w)[layer]
    rng = np.random.default_rng(rng_seed)
    outs = [np.zeros((n, w.hq, w.d)) for n in lens]
    lses = [np.zeros((n, w.hq)) for n in lens]
    if seqwise:
        plan = [(b, c0, min(n, c0 + chunk)) for b, n in enumerate(lens) for c0 in range(0, n, chunk)]
    else:
        assert len(set(lens)) == 1
        plan = [(-1, c0, min(lens[0], c0 + chunk)) for c0 in range(0, lens[0], chunk)]
    for b, c0, c1 in plan:
        seqs = range(w.batch) if b < 0 else [b]
        q = np.stack([W.tokens(w, "q", layer, s, c0, c1) for s in seqs])
        k = np.stack([W.tokens(w, "k", layer, s, c0, c1) for s in seqs])
        v = np.stack([W.tokens(w, "v", layer, s, c0, c1) for s in seqs])
        dq, dk, dv = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
        if b >= 0:
            dq, dk, dv = dq[0], dk[0], dv[0]
        shape = (dq.shape[0], c1 - c0, w.hq) if b < 0 else (c1 - c0, w.hq)
        lse = torch.empty(shape, dtype=torch.float32, device="cuda")
        out = cache.attn_prefill(layer, dq, dk, dv, seq=b, lse=lse)
        cache.kv_append(layer, dk, dv, seq=b)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        got_lse = lse.cpu().numpy()
        if b >= 0:
            got, got_lse = got[None], got_lse[None]
        for si, s in enumerate(seqs):
            outs[s][c0:c1] = got[si]
            lses[s][c0:c1] = got_lse[si]
            kh = W.tokens(w, "k", layer, s, 0, c1)
            vh = W.tokens(w, "v", layer, s, 0, c1)
            if check_rows is None:
                rows = np.arange(c0, c1)
            else:
                rows = np.unique(rng.integers(c0, c1, size=min(check_rows, c1 - c0)))
            qa = W.tokens(w, "q", layer, s, 0, c1)[rows]
            ref, ref_lse = O.attention(qa, kh, vh, rows, np.arange(c1), mask, w.sink, w.recent,
                                       chunk_start=c0 if mode == "chunk" else None)
            assert_close(got[si][rows - c0], ref, f"chunk [{c0},{c1}) seq {s} out")
            assert_close(got_lse[si][rows - c0], ref_lse, f"chunk [{c0},{c1}) seq {s} lse")
    return outs, lses, cache


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_prefill_variants(d, G):
    """Every built (head_dim, group) variant; chunks that straddle the sink and the window."""
    w = W.Workload("prefill-variant", 1, 2, 2 * G, 2, d, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((1,),), seed=21 + G)
    run_prefill(w, [300, 300], 70)


@pytest.mark.parametrize("S,R", [(0, 1), (4, 32), (16, 64), (16, 512), (70, 5)])
@pytest.mark.parametrize("chunk", [1, 7, 64, 200])
def test_prefill_sink_recent_chunks(S, R, chunk):
    w = W.Workload("prefill-sr", 1, 1, 8, 4, 128, "bf16", S, R, 0, 0, 2, fixed_mask=((0, 3),),
                   seed=23)
    run_prefill(w, [260], chunk, check_rows=None if chunk >= 64 else 40)


def test_prefill_ragged_sequences_seqwise():
    w = W.Workload("prefill-ragged", 1, 3, 16, 4, 128, "bf16", 16, 64, 0, 0, 2,
                   fixed_mask=((1, 2),), seed=25)
    run_prefill(w, [400, 37, 129], 100, seqwise=True)


def test_prefill_bf16_output():
    w = W.Workload("prefill-bf16-out", 1, 1, 8, 2, 128, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=27)
    run_prefill(w, [500], 128, out_dtype=torch.bfloat16)


def test_prefill_chunk_size_invariance():
    """Outputs do not depend on the chunk size (within rounding)."""
    w = W.Workload("prefill-inv", 1, 1, 8, 2, 128, "bf16", 8, 48, 0, 0, 1,
                   fixed_mask=((1,),), seed=29)
    a, la, _ = run_prefill(w, [600], 600, check_rows=64)
    b, lb, _ = run_prefill(w, [600], 37, check_rows=16)
    assert np.max(np.abs(a[0] - b[0])) < 4e-3
    assert np.max(np.abs(la[0] - lb[0])) < 4e-3


def test_prefill_equals_decode_sequence():
    """Chunked prefill of a prompt gives the outputs of decoding it token by token."""
    w = W.Workload("prefill-vs-decode", 1, 1, 8, 2, 128, "bf16", 4, 16, 0, 0, 1,
                   fixed_mask=((0,),), seed=31)
    n = 120
    outs, _, _ = run_prefill(w, [n], 50)
    cache = make_cache(w, capacity=n)
    dt = torch_dtype(w.dtype)
    dec = np.zeros((n, w.hq, w.d))
    for p in range(n):
        cache.kv_append(0, to_dev(W.tokens(w, "k", 0, 0, p, p + 1)[None], dt),
                        to_dev(W.tokens(w, "v", 0, 0, p, p + 1)[None], dt))
        dec[p] = cache.attn_decode(0, to_dev(W.tokens(w, "q", 0, 0, p, p + 1), dt)).float().cpu().numpy()[0]
    assert np.max(np.abs(outs[0] - dec)) < 4e-3


def test_prefill_c2_mha_32k_in_4k_chunks():
    """Llama-2-7B-shaped MHA layer: 32,768-token prompt in 8 chunks of 4,096 (the launch
    configuration of the benchmark); 64 sampled query rows per chunk, all 32 heads."""
    w = W.workload("c2")
    run_prefill(w, [w.prefill_len], w.prefill_chunk, check_rows=64)


def test_prefill_gqa_8k_in_2k_chunks():
    """Llama-3-8B-shaped GQA layer, 8,192-token prompt in 2,048-token chunks."""
    w = W.workload("c3").with_(context=8192)
    run_prefill(w, [8192], 2048, check_rows=64)
