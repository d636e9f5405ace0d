"""duo_attn_prefill on the GPU against the CPU float64 oracle.

A prompt is processed in chunks: prefill attention of the chunk (compared with the oracle),
then the append of the same K/V. |gpu - ref| <= 2e-3 + 1e-2 |ref| elementwise.
"""
import concurrent.futures as cf
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import duo_oracle as O

from gpu_util import assert_close, make_cache, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _progress(msg):
    print(msg, file=sys.stderr, flush=True)


def edge_rows(c0, c1, group, n_random, rng):
    """Query positions a full-size prefill chunk [c0, c1) is checked at: every position of a
    chunk that starts the sequence (where few keys are visible), otherwise the first and last
    position of every query tile of 128 / group positions (the tiles the kernel works in,
    counted from the chunk start; their rows meet the split key ranges' edges) plus
    ``n_random`` random positions."""
    if c0 == 0:
        return np.arange(c0, c1)
    qpb = 128 // group
    starts = np.arange(c0, c1, qpb)
    ends = np.minimum(starts + qpb, c1) - 1
    rnd = rng.integers(c0, c1, size=min(n_random, c1 - c0))
    return np.unique(np.concatenate([starts, ends, rnd]))


def run_prefill(w, lens, chunk, layer=0, check_rows=None, cache=None, seqwise=False,
                out_dtype=torch.float32, rng_seed=0, mode="window", edges=False,
                max_abs=None, staged=False):
    """Prefill prompts of lengths ``lens`` in chunks of ``chunk``; returns the outputs.

    ``mode`` is the streaming-head prefill mode: "window" (per-query sink + recent mask) or
    "chunk" (the pruned cache before the chunk plus the chunk causally).

    ``check_rows``: None = every row, int = that many random rows per chunk and sequence
    (with ``edges``: every row of the first chunk, the first and last row of every query
    tile of the others, plus that many random rows; see ``edge_rows``).
    With ``seqwise`` every sequence is prefilled by its own calls (ragged prompts);
    otherwise all sequences share the chunk calls (equal lengths). ``max_abs``: a tighter
    bound on the largest absolute error of every chunk (fp32 inputs). ``staged``: the chunks
    go through duo_attn_prefill_staged (on a bf16 cache: values staged as fp16 copies).
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
        call = cache.attn_prefill_staged if staged else cache.attn_prefill
        out = call(layer, dq, dk, dv, seq=b, lse=lse)
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
            elif edges:
                rows = edge_rows(c0, c1, w.group, check_rows, rng)
            else:
                rows = np.unique(rng.integers(c0, c1, size=min(check_rows, c1 - c0)))
            qa = W.tokens(w, "q", layer, s, 0, c1)[rows]
            ref, ref_lse = O.attention(qa, kh, vh, rows, np.arange(c1), mask, w.sink, w.recent,
                                       chunk_start=c0 if mode == "chunk" else None)
            err = assert_close(got[si][rows - c0], ref, f"chunk [{c0},{c1}) seq {s} out")
            assert_close(got_lse[si][rows - c0], ref_lse, f"chunk [{c0},{c1}) seq {s} lse")
            if max_abs is not None:
                assert err <= max_abs, f"chunk [{c0},{c1}) seq {s}: max abs err {err:.3e}"
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


def prefill_every_row(w, mode="window"):
    """The prompt of ``w`` (one sequence) in chunks of ``w.prefill_chunk`` through the GPU,
    then every output row and log-sum-exp of every head against the oracle. The oracle runs
    per chunk and KV head in a thread pool (its large-array numpy work releases the GIL); a
    streaming head is given only the keys its chunk can see in either mode (the sink, the R
    tokens before the chunk, the chunk) at their true positions, which leaves its explicit
    mask, and so its result, unchanged."""
    mask = W.retrieval_mask(w)[0]
    P, C, S, R, G = w.prefill_len, w.prefill_chunk, w.sink, w.recent, w.group
    cache = make_cache(w, out_dtype=torch.float32, capacity=P + 1, streaming_prefill=mode)
    dt = torch_dtype(w.dtype)
    q = W.tokens(w, "q", 0, 0, 0, P)
    k = W.tokens(w, "k", 0, 0, 0, P)
    v = W.tokens(w, "v", 0, 0, 0, P)
    got = np.empty((P, w.hq, w.d), dtype=np.float32)
    got_lse = np.empty((P, w.hq), dtype=np.float32)
    for c0 in range(0, P, C):
        c1 = min(P, c0 + C)
        dk, dv = to_dev(k[c0:c1][None], dt), to_dev(v[c0:c1][None], dt)
        lse = torch.empty((1, c1 - c0, w.hq), dtype=torch.float32, device="cuda")
        out = cache.attn_prefill(0, to_dev(q[c0:c1][None], dt), dk, dv, seq=-1, lse=lse)
        cache.kv_append(0, dk, dv, seq=-1)
        torch.cuda.synchronize()
        got[c0:c1] = out.float().cpu().numpy()[0]
        got_lse[c0:c1] = lse.cpu().numpy()[0]
    _progress(f"{w.name} prefill ({mode}): every chunk on the GPU")

    def check(c0, j):
        c1 = min(P, c0 + C)
        if mask[j]:
            keys = np.arange(c1)
        else:
            keys = np.unique(np.concatenate([np.arange(min(S, c1)),
                                             np.arange(max(S, c0 - R), c1)]))
        hq = slice(j * G, (j + 1) * G)
        ref, ref_lse = O.attention(q[c0:c1, hq], k[keys, j:j + 1], v[keys, j:j + 1],
                                   np.arange(c0, c1), keys, mask[j:j + 1], S, R,
                                   chunk_start=c0 if mode == "chunk" else None)
        assert_close(got[c0:c1, hq], ref, f"chunk [{c0},{c1}) kv {j} out")
        assert_close(got_lse[c0:c1, hq], ref_lse, f"chunk [{c0},{c1}) kv {j} lse")

    with cf.ThreadPoolExecutor(8) as ex:
        for c0 in range(0, P, C):
            for f in [ex.submit(check, c0, j) for j in range(w.hkv)]:
                f.result()
            _progress(f"{w.name} prefill ({mode}): chunk at {c0} checked, every row")
    cache.close()


@pytest.mark.timeout(900)
def test_prefill_c2_mha_32k_in_4k_chunks():
    """Llama-2-7B-shaped MHA layer: 32,768-token prompt in 8 chunks of 4,096 (the launch
    configuration of the benchmark): every output row and log-sum-exp of all 32 heads
    (32,768 x 32 rows)."""
    prefill_every_row(W.workload("c2"))


def test_prefill_gqa_8k_in_2k_chunks():
    """Llama-3-8B-shaped GQA layer, 8,192-token prompt in 2,048-token chunks: every row of the
    first chunk, tile edges and 64 random rows of the others."""
    w = W.workload("c3").with_(context=8192)
    run_prefill(w, [8192], 2048, check_rows=64, edges=True)


# ---- fp32 inputs (v_mfma_f32_16x16x4_f32 path) ----------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_prefill_f32_variants(d, G):
    """Every built (head_dim, group) variant with float32 inputs; chunks that straddle the
    sink and the window, 64-row query tiles and 32-key tiles."""
    w = W.Workload("prefill-f32-variant", 1, 2, 2 * G, 2, d, "f32", 4, 32, 0, 0, 1,
                   fixed_mask=((1,),), seed=61 + G)
    run_prefill(w, [300, 300], 70, max_abs=1e-4)


@pytest.mark.parametrize("chunk", [1, 64, 1024])
def test_prefill_f32_tiny_gqa_1024(chunk):
    """The tiny GQA layer (8 q / 2 kv heads, d 64, float32, KV head 0 retrieval, sink 4 +
    recent 32): a 1,024-token prompt in chunks of 1, 64 and 1,024, every row checked, at the
    float32 bar of 1e-4."""
    w = W.workload("c1")
    run_prefill(w, [1024], chunk, max_abs=1e-4)


@pytest.mark.parametrize("S,R", [(0, 1), (16, 64), (70, 5)])
def test_prefill_f32_sink_recent_ragged(S, R):
    """float32 inputs: S/R around the 32-key tile, ragged prompts in per-sequence calls."""
    w = W.Workload("prefill-f32-sr", 1, 3, 8, 4, 128, "f32", S, R, 0, 0, 2,
                   fixed_mask=((0, 3),), seed=63)
    run_prefill(w, [260, 37, 129], 50, seqwise=True, max_abs=1e-4)


def test_prefill_f32_chunk_mode():
    """float32 inputs with chunk-granular streaming heads."""
    w = W.Workload("prefill-f32-chunk", 1, 2, 8, 2, 64, "f32", 4, 28, 0, 0, 1,
                   fixed_mask=((0,),), seed=65)
    run_prefill(w, [300, 300], 70, mode="chunk", max_abs=1e-4)


def test_prefill_large_values_within_fp16_bound():
    """Values up to about 45,000 in magnitude (bf16, inside the fp16 range the PV product takes
    them in): every output stays within 2^-10 max |v| of the oracle (twice the bound that fp16
    weights allow, 2^-11 sum_t w_t |v_t|), and the log-sum-exp, which the values do not enter,
    within the ordinary tolerance. Both head classes; chunks that start the sequence (few
    visible keys) and later ones."""
    w = W.Workload("large-v", 1, 1, 4, 4, 128, "bf16", 4, 32, 0, 0, 2, fixed_mask=((0, 2),),
                   seed=601)
    mask = W.retrieval_mask(w)[0]
    cache = make_cache(w, capacity=401)
    n, chunk = 400, 200
    q = W.tokens(w, "q", 0, 0, 0, n)
    k = W.tokens(w, "k", 0, 0, 0, n)
    v = torch.from_numpy(W.tokens(w, "v", 0, 0, 0, n) * 10000.0).to(torch.bfloat16)
    vmax = float(v.float().abs().max())
    assert 20000.0 < vmax < 65504.0, vmax
    v = v.double().numpy()
    for c0 in range(0, n, chunk):
        c1 = c0 + chunk
        dq, dk = to_dev(q[c0:c1], torch.bfloat16), to_dev(k[c0:c1], torch.bfloat16)
        dv = to_dev(v[c0:c1], torch.bfloat16)
        lse = torch.empty((c1 - c0, w.hq), dtype=torch.float32, device="cuda")
        out = cache.attn_prefill(0, dq, dk, dv, seq=0, lse=lse)
        cache.kv_append(0, dk, dv, seq=0)
        torch.cuda.synchronize()
        ref, ref_lse = O.prefill_chunk(q[c0:c1], k[:c1], v[:c1], c0, mask, w.sink, w.recent)
        got = out.float().cpu().numpy()
        assert np.all(np.isfinite(got))
        err = np.abs(got - ref).max()
        assert err <= 2.0 ** -10 * vmax, (c0, err, 2.0 ** -10 * vmax)
        assert_close(lse.cpu().numpy(), ref_lse, f"chunk [{c0},{c1}) lse")
