"""duo_attn_prefill with chunk-granular streaming heads on the GPU against the CPU oracle.

In this mode a streaming head's query in a chunk starting at c sees every token the pruned
cache holds at c (the sinks and the R tokens before c) and the chunk up to itself
(explainer, "Chunked Pre-filling", Figure 5: the second chunk attends to the kept tokens
0, 2, 3 and to itself). Retrieval heads are unchanged. |gpu - ref| <= 2e-3 + 1e-2 |ref|.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import duo_oracle as O

from gpu_util import make_cache, to_dev, torch_dtype
from test_gpu_prefill import prefill_every_row, run_prefill

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_chunk_mode_variants(d, G):
    """Built (head_dim, group) variants; chunks that straddle the sinks and the window."""
    w = W.Workload("prefill-chunk-variant", 1, 2, 2 * G, 2, d, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((1,),), seed=41 + G)
    run_prefill(w, [300, 300], 70, mode="chunk")


@pytest.mark.parametrize("S,R", [(0, 1), (4, 32), (16, 512), (70, 5), (64, 100)])
@pytest.mark.parametrize("chunk", [1, 7, 64, 200])
def test_chunk_mode_sink_recent(S, R, chunk):
    """Every streaming head (all four KV heads of a GQA layer), ring sizes below, across and
    above the tile size of 64 keys, chunks from one token to several tiles."""
    w = W.Workload("prefill-chunk-sr", 1, 1, 8, 4, 128, "bf16", S, R, 0, 0, 0,
                   fixed_mask=((),), seed=43)
    run_prefill(w, [260], chunk, check_rows=None if chunk >= 64 else 40, mode="chunk")


def test_chunk_mode_ragged_sequences_seqwise():
    w = W.Workload("prefill-chunk-ragged", 1, 3, 16, 4, 128, "bf16", 16, 64, 0, 0, 2,
                   fixed_mask=((1, 2),), seed=45)
    run_prefill(w, [400, 37, 129], 100, seqwise=True, mode="chunk")


def test_chunk_mode_bf16_output():
    w = W.Workload("prefill-chunk-bf16-out", 1, 1, 8, 2, 128, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=47)
    run_prefill(w, [500], 128, out_dtype=torch.bfloat16, mode="chunk")


def test_chunk_mode_differs_from_window_only_on_streaming_heads():
    """The two modes agree on retrieval heads, and on streaming heads while the chunk is
    within the first S + R tokens; past that, streaming outputs differ."""
    w = W.Workload("prefill-chunk-vs-window", 1, 1, 8, 2, 128, "bf16", 4, 28, 0, 0, 1,
                   fixed_mask=((0,),), seed=49)
    a, la, _ = run_prefill(w, [320], 160, check_rows=64, mode="window")
    b, lb, _ = run_prefill(w, [320], 160, check_rows=64, mode="chunk")
    ret = slice(0, 4)  # query heads of KV head 0 (retrieval)
    assert np.max(np.abs(a[0][:, ret] - b[0][:, ret])) < 4e-3
    # the first chunk starts at 0: nothing is held, both are causal up to S + R - 1
    sr = w.sink + w.recent
    assert np.max(np.abs(a[0][:sr, 4:] - b[0][:sr, 4:])) < 4e-3
    assert np.max(np.abs(a[0][200:, 4:] - b[0][200:, 4:])) > 1e-2


def test_chunk_mode_gather_equivalence():
    """Chunk-granular prefill equals the same kernel in window mode run on nothing but the
    pruned cache: a streaming head over [held ; chunk] with R at least the chunk span is
    plain causal attention over those keys."""
    w = W.Workload("prefill-chunk-gather", 1, 1, 4, 1, 128, "bf16", 2, 30, 0, 0, 0,
                   fixed_mask=((),), seed=51)
    n, chunk = 190, 60
    outs, _, _ = run_prefill(w, [n], chunk, mode="chunk", check_rows=16)
    dt = torch_dtype(w.dtype)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        held = sorted(O.streaming_valid_tokens(c0, w.sink, w.recent).tolist())
        keys = held + list(range(c0, c1))
        # a retrieval-only cache holding the gathered keys in order, then the chunk's queries
        wg = W.Workload("gather", 1, 1, 4, 1, 128, "bf16", 2, 30, 0, 0, 1,
                        fixed_mask=((0,),), seed=51)
        cache = make_cache(wg, capacity=len(keys) + 1)
        kk = W.tokens(w, "k", 0, 0, 0, c1)[keys[:len(held)]]
        vv = W.tokens(w, "v", 0, 0, 0, c1)[keys[:len(held)]]
        if held:
            cache.kv_append(0, to_dev(kk[None], dt), to_dev(vv[None], dt))
        q = to_dev(W.tokens(w, "q", 0, 0, c0, c1)[None], dt)
        k = to_dev(W.tokens(w, "k", 0, 0, c0, c1)[None], dt)
        v = to_dev(W.tokens(w, "v", 0, 0, c0, c1)[None], dt)
        got = cache.attn_prefill(0, q, k, v).float().cpu().numpy()[0]
        assert np.max(np.abs(got - outs[0][c0:c1])) < 4e-3, c0


@pytest.mark.timeout(900)
def test_chunk_mode_c2_mha_32k_in_4k_chunks():
    """Llama-2-7B-shaped MHA layer: 32,768-token prompt in 8 chunks of 4,096 in the
    benchmark's launch configuration: every output row and log-sum-exp of all 32 heads."""
    prefill_every_row(W.workload("c2"), mode="chunk")


def test_chunk_mode_gqa_8k_in_2k_chunks():
    w = W.workload("c3").with_(context=8192)
    run_prefill(w, [8192], 2048, check_rows=64, mode="chunk", edges=True)
