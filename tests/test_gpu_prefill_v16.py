"""duo_attn_prefill_staged on a bf16 cache: the values of the chunk, of the retrieval
prefixes and of the streaming caches are converted to fp16 once into caller staging, and the
prefill kernel reads them without converting each V tile in LDS.

The conversion is the one the kernel applies in LDS, so the staged call must return exactly
what duo_attn_prefill returns (outputs and log-sum-exps compared bit for bit, on the same
inputs, in lock-step over two caches), and both must match the CPU float64 oracle within
2e-3 + 1e-2 |ref| (the shared checks of test_gpu_prefill)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W

from gpu_util import make_cache, to_dev, torch_dtype
from test_gpu_prefill import run_prefill

import head_split_kv_amd as hsk
from head_split_kv_amd import _native as N

pytestmark = pytest.mark.gpu


def lockstep(w, lens, chunk, mode="window", seqwise=False, out_dtype=torch.float32):
    """Prefill the prompts of ``w`` through duo_attn_prefill on one cache and through
    duo_attn_prefill_staged on another, appending each chunk to both; every chunk's outputs
    and log-sum-exps must be identical. One staging buffer, grown to what each call needs,
    serves every call."""
    caps = max(lens) + 1
    plain = make_cache(w, out_dtype=out_dtype, capacity=caps, streaming_prefill=mode)
    staged = make_cache(w, out_dtype=out_dtype, capacity=caps, streaming_prefill=mode)
    dt = torch_dtype(w.dtype)
    if seqwise:
        plan = [(b, c0, min(n, c0 + chunk)) for b, n in enumerate(lens)
                for c0 in range(0, n, chunk)]
    else:
        assert len(set(lens)) == 1
        plan = [(-1, c0, min(lens[0], c0 + chunk)) for c0 in range(0, lens[0], chunk)]
    stg = None
    for b, c0, c1 in plan:
        seqs = range(w.batch) if b < 0 else [b]
        q = np.stack([W.tokens(w, "q", 0, s, c0, c1) for s in seqs])
        k = np.stack([W.tokens(w, "k", 0, s, c0, c1) for s in seqs])
        v = np.stack([W.tokens(w, "v", 0, s, c0, c1) for s in seqs])
        dq, dk, dv = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
        if b >= 0:
            dq, dk, dv = dq[0], dk[0], dv[0]
        shape = (dq.shape[0], c1 - c0, w.hq) if b < 0 else (c1 - c0, w.hq)
        la = torch.empty(shape, dtype=torch.float32, device="cuda")
        lb = torch.empty(shape, dtype=torch.float32, device="cuda")
        need = hsk.duo_prefill_staging_bytes(staged, 0, b, c1 - c0)
        if stg is None or stg.numel() < need:  # one buffer, grown as the prefixes grow
            stg = torch.empty(need, dtype=torch.uint8, device="cuda")
        oa = plain.attn_prefill(0, dq, dk, dv, seq=b, lse=la)
        ob = staged.attn_prefill_staged(0, dq, dk, dv, seq=b, lse=lb, staging=stg)
        plain.kv_append(0, dk, dv, seq=b)
        staged.kv_append(0, dk, dv, seq=b)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"chunk [{c0},{c1}) seq {b}: outputs differ"
        assert torch.equal(la, lb), f"chunk [{c0},{c1}) seq {b}: lse differ"
    plain.close()
    staged.close()


def test_staging_bytes_of_a_bf16_cache():
    """The staging size: the retrieval prefixes at the longest current length, the chunk's
    values and every streaming cache, each region 256-byte aligned except the last."""
    w = W.Workload("v16-bytes", 1, 3, 8, 4, 128, "bf16", 4, 28, 0, 0, 2, fixed_mask=((0, 3),),
                   seed=71)
    cache = make_cache(w, capacity=200)
    up = lambda x: (x + 255) // 256 * 256
    row = w.d * 2
    lens = [50, 120, 7]
    for b, n in enumerate(lens):
        k = to_dev(W.tokens(w, "k", 0, b, 0, n), torch.bfloat16)
        v = to_dev(W.tokens(w, "v", 0, b, 0, n), torch.bfloat16)
        cache.kv_append(0, k, v, seq=b)
    torch.cuda.synchronize()
    hr, hs, sr = 2, 2, w.sink + w.recent
    for seq, nb, cmax in ((-1, 3, 120), (0, 1, 50), (2, 1, 7)):
        got = hsk.duo_prefill_staging_bytes(cache, 0, seq, 9)
        assert got == up(nb * hr * cmax * row) + up(nb * 9 * w.hkv * row) + 3 * hs * sr * row
    cache.close()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_v16_variants_match_plain_and_oracle(d, G):
    """Every (head_dim, group) variant: identical to duo_attn_prefill, and within the
    tolerance of the oracle; chunks that straddle the sink and the window."""
    w = W.Workload("v16-variant", 1, 2, 2 * G, 2, d, "bf16", 4, 32, 0, 0, 1,
                   fixed_mask=((1,),), seed=73 + G)
    lockstep(w, [300, 300], 70)
    run_prefill(w, [300, 300], 70, staged=True)


@pytest.mark.parametrize("mode", ["window", "chunk"])
@pytest.mark.parametrize("S,R", [(0, 1), (16, 64), (70, 5)])
def test_v16_ragged_sequences(mode, S, R):
    """Ragged prompts in per-sequence calls (the prefix staging laid out at the longest
    length while one sequence is pre-filled), both streaming modes, bf16 outputs."""
    w = W.Workload("v16-ragged", 1, 3, 16, 4, 128, "bf16", S, R, 0, 0, 2,
                   fixed_mask=((1, 2),), seed=79)
    lockstep(w, [400, 37, 129], 100, mode=mode, seqwise=True, out_dtype=torch.bfloat16)
    run_prefill(w, [400, 37, 129], 100, seqwise=True, mode=mode, staged=True,
                out_dtype=torch.bfloat16)


@pytest.mark.parametrize("chunk", [1, 7, 64, 200])
def test_v16_chunk_sizes(chunk):
    """Chunks from one token up, over sink and window edges."""
    w = W.Workload("v16-chunks", 1, 1, 8, 4, 128, "bf16", 16, 64, 0, 0, 2, fixed_mask=((0, 3),),
                   seed=83)
    lockstep(w, [260], chunk)
    run_prefill(w, [260], chunk, check_rows=None if chunk >= 64 else 40, staged=True)


def test_v16_null_staging_is_plain_prefill():
    """Without staging the staged call on a bf16 cache is duo_attn_prefill."""
    w = W.Workload("v16-null", 1, 1, 8, 2, 128, "bf16", 4, 32, 0, 0, 1, fixed_mask=((0,),),
                   seed=89)
    cache = make_cache(w, capacity=300)
    dt = torch.bfloat16
    q, k, v = (to_dev(W.tokens(w, t, 0, 0, 0, 200), dt) for t in ("q", "k", "v"))
    a = cache.attn_prefill(0, q, k, v, seq=0)
    b = torch.empty_like(a)
    st = N.lib().duo_attn_prefill_staged(cache.handle, 0, 0, ctypes.c_void_p(q.data_ptr()),
                                        ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                        200, ctypes.c_void_p(b.data_ptr()), None, None, 0, None)
    torch.cuda.synchronize()
    assert st == N.DUO_OK
    assert torch.equal(a, b)
    cache.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,mode", [("c2", "window"), ("c2", "chunk"), ("c3", "window")])
def test_v16_full_size_prompt_identical(name, mode):
    """The 32K prompts of the benchmark in 4K chunks (the Llama-2-7B-shaped MHA layer in both
    streaming modes, the Llama-3-8B-shaped GQA layer): the staged call returns exactly what
    duo_attn_prefill returns for every row of every chunk. duo_attn_prefill itself is checked
    against the oracle on every row of the MHA prompt (test_gpu_prefill,
    test_gpu_prefill_chunk)."""
    w = W.workload(name).with_(context=32768)
    lockstep(w, [32768], 4096, mode=mode)


@pytest.mark.parametrize("mode", ["window", "chunk"])
def test_v16_batch_call_over_ragged_prefixes(mode):
    """One chunk call for a whole batch whose sequences hold prefixes of different lengths
    (the prefix staging laid out at the longest one, shorter rows left unwritten): identical
    to duo_attn_prefill, and within the tolerance of the oracle on every row."""
    from gpu_util import assert_close
    from oracle import duo_oracle as O
    w = W.Workload("v16-batch-ragged", 1, 3, 16, 4, 128, "bf16", 16, 64, 0, 0, 2,
                   fixed_mask=((1, 2),), seed=97)
    lens, m = [300, 37, 129], 90
    dt = torch.bfloat16
    caches = [make_cache(w, capacity=max(lens) + m, streaming_prefill=mode) for _ in range(2)]
    for cache in caches:
        for b, n in enumerate(lens):
            cache.kv_append(0, to_dev(W.tokens(w, "k", 0, b, 0, n), dt),
                            to_dev(W.tokens(w, "v", 0, b, 0, n), dt), seq=b)
    q = np.stack([W.tokens(w, "q", 0, b, n, n + m) for b, n in enumerate(lens)])
    k = np.stack([W.tokens(w, "k", 0, b, n, n + m) for b, n in enumerate(lens)])
    v = np.stack([W.tokens(w, "v", 0, b, n, n + m) for b, n in enumerate(lens)])
    dq, dk, dv = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    la = torch.empty((w.batch, m, w.hq), dtype=torch.float32, device="cuda")
    lb = torch.empty_like(la)
    oa = caches[0].attn_prefill(0, dq, dk, dv, seq=-1, lse=la)
    stg = torch.empty(hsk.duo_prefill_staging_bytes(caches[1], 0, -1, m), dtype=torch.uint8,
                      device="cuda")
    ob = caches[1].attn_prefill_staged(0, dq, dk, dv, seq=-1, lse=lb, staging=stg)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    mask = W.retrieval_mask(w)[0]
    got, got_lse = ob.float().cpu().numpy(), lb.cpu().numpy()
    for b, n in enumerate(lens):
        ref, ref_lse = O.attention(W.tokens(w, "q", 0, b, n, n + m),
                                   W.tokens(w, "k", 0, b, 0, n + m),
                                   W.tokens(w, "v", 0, b, 0, n + m), np.arange(n, n + m),
                                   np.arange(n + m), mask, w.sink, w.recent,
                                   chunk_start=n if mode == "chunk" else None)
        assert_close(got[b], ref, f"seq {b} out")
        assert_close(got_lse[b], ref_lse, f"seq {b} lse")
    for cache in caches:
        cache.close()
