"""duo_attn_gate_mixed (identification-phase attention) on the GPU against the CPU oracle.

Every KV head j blends its causal-mask output and its sink + recent output by alpha[j]
(explainer, "Gate Parameterization"). Layers keep a full cache for every KV head.
|gpu - ref| <= 2e-3 + 1e-2 |ref| elementwise.
"""
import concurrent.futures as cf
import sys

import numpy as np
import pytest
import torch

import head_split_kv_amd as hsk
import workloads as W
from oracle import duo_oracle as O

from gpu_util import assert_close, make_cache, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def all_retrieval(name, batch, hq, hkv, d, S, R, seed, dtype="bf16", **kw):
    return W.Workload(name, 1, batch, hq, hkv, d, dtype, S, R, 0, 0, hkv,
                      fixed_mask=(tuple(range(hkv)),), seed=seed, **kw)


def run_mixed(w, lens, chunk, alpha, check_rows=None, out_dtype=torch.float32, seqwise=False,
              rng_seed=0):
    """Gate-mixed attention of prompts in chunks (appending each chunk after its call).
    ``check_rows``: None = every row, int = that many random rows per chunk. The oracle runs
    over blocks of the sorted rows with the keys up to each block's last position (later keys
    are masked for every one of them)."""
    cache = make_cache(w, out_dtype=out_dtype, capacity=max(lens) + 1)
    dt = torch_dtype(w.dtype)
    rng = np.random.default_rng(rng_seed)
    outs = [np.zeros((n, w.hq, w.d)) for n in lens]
    if seqwise:
        plan = [(b, c0, min(n, c0 + chunk)) for b, n in enumerate(lens) for c0 in range(0, n, chunk)]
    else:
        plan = [(-1, c0, min(lens[0], c0 + chunk)) for c0 in range(0, lens[0], chunk)]
    for b, c0, c1 in plan:
        seqs = range(w.batch) if b < 0 else [b]
        q, k, v = (np.stack([W.tokens(w, t, 0, s, c0, c1) for s in seqs]) for t in "qkv")
        dq, dk, dv = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
        if b >= 0:
            dq, dk, dv = dq[0], dk[0], dv[0]
        out = cache.attn_gate_mixed(0, dq, dk, dv, alpha, seq=b)
        cache.kv_append(0, dk, dv, seq=b)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        if b >= 0:
            got = got[None]
        for si, s in enumerate(seqs):
            outs[s][c0:c1] = got[si]
            kh, vh = W.tokens(w, "k", 0, s, 0, c1), W.tokens(w, "v", 0, s, 0, c1)
            if check_rows is None:
                rows = np.arange(c0, c1)
            else:
                rows = np.unique(rng.integers(c0, c1, size=min(check_rows, c1 - c0)))
            qall = W.tokens(w, "q", 0, s, 0, c1)
            for i in range(0, len(rows), 256):
                blk = rows[i:i + 256]
                t1 = int(blk[-1]) + 1
                ref = O.gate_mixed_attention(qall[blk], kh[:t1], vh[:t1], blk, np.arange(t1),
                                             alpha, w.sink, w.recent)
                assert_close(got[si][blk - c0], ref, f"chunk [{c0},{c1}) seq {s} rows {blk[0]}..")
    return outs, cache


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gate_mixed_variants(d, G):
    """Whole sequences as one chunk (the identification setting), every built variant."""
    w = all_retrieval("mixed-variant", 2, 2 * G, 2, d, 4, 32, seed=81 + G)
    run_mixed(w, [300, 300], 300, np.array([0.25, 0.8], dtype=np.float32))


@pytest.mark.parametrize("S,R", [(0, 1), (4, 32), (16, 64), (70, 5), (64, 256)])
def test_gate_mixed_chunked_sink_recent(S, R):
    """Chunks over a growing full cache, S/R below and above the 64-key tile, gates spread
    over [0, 1] including both ends."""
    w = all_retrieval("mixed-sr", 1, 8, 4, 128, S, R, seed=83)
    run_mixed(w, [400], 96, np.array([0.0, 0.35, 0.7, 1.0], dtype=np.float32))


def test_gate_mixed_ragged_seqwise_bf16_out():
    w = all_retrieval("mixed-ragged", 3, 16, 4, 128, 16, 64, seed=85)
    run_mixed(w, [400, 37, 129], 100, np.array([0.9, 0.1, 0.5, 0.0], dtype=np.float32),
              seqwise=True, out_dtype=torch.bfloat16)


def test_gate_one_is_the_full_prefill():
    """Gate 1 returns exactly the causal prefill of the same all-retrieval cache (f32 out: the
    blend keeps the first pass's value)."""
    w = all_retrieval("mixed-vs-prefill", 1, 8, 2, 128, 4, 32, seed=87)
    dt = torch_dtype(w.dtype)
    cache = make_cache(w, capacity=600)
    for c0 in range(0, 500, 250):
        q, k, v = (to_dev(W.tokens(w, t, 0, 0, c0, c0 + 250)[None], dt) for t in "qkv")
        a = cache.attn_gate_mixed(0, q, k, v, [1.0, 1.0]).cpu().numpy()
        b = cache.attn_prefill(0, q, k, v).cpu().numpy()
        assert np.array_equal(a, b)
        cache.kv_append(0, k, v)


def test_gate_mixed_rejects_streaming_layers_and_bad_gates():
    w = W.Workload("mixed-reject", 1, 1, 8, 2, 128, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((0,),), seed=89)
    cache = make_cache(w, capacity=64)
    dt = torch_dtype(w.dtype)
    q, k, v = (to_dev(W.tokens(w, t, 0, 0, 0, 16)[None], dt) for t in "qkv")
    with pytest.raises(hsk.DuoError) as e:
        cache.attn_gate_mixed(0, q, k, v, [0.5, 0.5])
    assert e.value.status == hsk.DUO_ERR_INVALID
    w2 = all_retrieval("mixed-reject2", 1, 8, 2, 128, 4, 32, seed=89)
    cache2 = make_cache(w2, capacity=64)
    for bad in ([1.5, 0.5], [-0.1, 0.5], [float("nan"), 0.5]):
        with pytest.raises(hsk.DuoError) as e:
            cache2.attn_gate_mixed(0, q, k, v, bad)
        assert e.value.status == hsk.DUO_ERR_INVALID


@pytest.mark.timeout(900)
def test_gate_mixed_mha_32k_whole_sequence():
    """Identification-phase shape: a Llama-2-7B-shaped MHA layer (32 heads, d 128, sink 16 +
    recent 512) over one 32,768-token sequence processed whole, gates drawn in [0, 1] (the
    launch configuration the benchmark times): every output row of all 32 heads. The oracle
    runs per KV head and block of 1,024 rows (keys up to the block's last position; later
    ones are masked for all of its rows) in a thread pool, its large-array numpy work
    releasing the GIL."""
    base = W.workload("c2")
    w = all_retrieval("mixed-c2", 1, 32, 32, 128, 16, 512, seed=base.seed)
    alpha = np.random.default_rng(91).random(32).astype(np.float32)
    P, G = 32768, w.group
    cache = make_cache(w, out_dtype=torch.float32, capacity=P + 1)
    dt = torch_dtype(w.dtype)
    q, k, v = (W.tokens(w, x, 0, 0, 0, P) for x in "qkv")
    out = cache.attn_gate_mixed(0, to_dev(q[None], dt), to_dev(k[None], dt), to_dev(v[None], dt),
                                alpha)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()[0]
    cache.close()
    print("mixed-c2: the GPU pass done", file=sys.stderr, flush=True)

    def check(r0, j):
        r1 = min(P, r0 + 1024)
        hq = slice(j * G, (j + 1) * G)
        ref = O.gate_mixed_attention(q[r0:r1, hq], k[:r1, j:j + 1], v[:r1, j:j + 1],
                                     np.arange(r0, r1), np.arange(r1), alpha[j:j + 1],
                                     w.sink, w.recent)
        assert_close(got[r0:r1, hq], ref, f"rows [{r0},{r1}) kv {j}")

    with cf.ThreadPoolExecutor(8) as ex:
        for r0 in range(0, P, 8192):
            for f in [ex.submit(check, b, j) for b in range(r0, r0 + 8192, 1024)
                      for j in range(w.hkv)]:
                f.result()
            print(f"mixed-c2: rows below {r0 + 8192} checked", file=sys.stderr, flush=True)


@pytest.mark.parametrize("d", [64, 128])
def test_gate_mixed_f32(d):
    """float32 inputs: chunks over a growing full cache, gates across [0, 1]."""
    w = all_retrieval("mixed-f32", 2, 8, 2, d, 4, 32, seed=93, dtype="f32")
    run_mixed(w, [300, 300], 90, np.array([0.3, 1.0], dtype=np.float32))
