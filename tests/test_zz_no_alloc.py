"""duo_attn_decode_noalloc (split-K partials in the library's static device scratch) against
duo_attn_decode (partials in the cache's workspace), through the C ABI: the same outputs and
log-sum-exps within |a - b| <= 2e-3 + 1e-2 |b|, on calls in a row where each later call has a
smaller input than the one before, so that it reads nothing a previous call left behind."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from head_split_kv_amd import _native as N

from gpu_util import assert_close, fill, make_cache, step_inputs

pytestmark = pytest.mark.gpu


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _pair(w, lens, kv_bits=0, splits=0, rope_theta=0.0):
    """A filled cache after one appended step, and the step's query."""
    import head_split_kv_amd as hsk
    mask = W.retrieval_mask(w)
    cache = hsk.DuoCache(num_layers=1, batch=w.batch, num_q_heads=w.hq, num_kv_heads=w.hkv,
                         head_dim=w.d, sink=w.sink, recent=w.recent, capacity=max(lens) + 1,
                         retrieval_mask=mask, dtype=torch.bfloat16, out_dtype=torch.float32,
                         kv_bits=kv_bits, max_splits=0, rope_theta=rope_theta)
    fill(cache, w, 0, lens)
    q, k, v, _ = step_inputs(w, 0, lens)
    cache.kv_append(0, k, v)
    if splits:
        hsk.duo_set_decode_splits(cache, splits)
    return cache, q


def _both(cache, q):
    B, Hq, d = q.shape
    ref = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    ref_lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    L = N.lib()
    st = L.duo_attn_decode(cache.handle, 0, ctypes.c_void_p(q.data_ptr()),
                           ctypes.c_void_p(ref.data_ptr()), ctypes.c_void_p(ref_lse.data_ptr()),
                           _stream())
    assert st == N.DUO_OK, N.status_string(st)
    st = L.duo_attn_decode_noalloc(cache.handle, 0, ctypes.c_void_p(q.data_ptr()),
                                   ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(lse.data_ptr()), _stream())
    assert st == N.DUO_OK, N.status_string(st)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), ref.cpu().numpy(), ref_lse.cpu().numpy()


def test_noalloc_matches_decode_on_calls_in_a_row():
    """Three calls in a row, each smaller than the one before: a 4-sequence GQA batch with
    long ragged contexts (many splits, partials far into the scratch), then one sequence of
    2,000 tokens, then one of 40 tokens with 7 forced splits."""
    w1 = W.Workload("noalloc-a", 1, 4, 32, 8, 128, "bf16", 16, 512, 0, 1, 4, seed=101)
    w2 = W.Workload("noalloc-b", 1, 1, 8, 2, 128, "bf16", 4, 32, 0, 1, 1,
                    fixed_mask=((0,),), seed=103)
    w3 = W.Workload("noalloc-c", 1, 1, 8, 2, 64, "bf16", 4, 8, 0, 1, 1,
                    fixed_mask=((1,),), seed=105)
    for w, lens, splits in ((w1, [70000, 9000, 300, 24000], 0), (w2, [2000], 0),
                            (w3, [40], 7)):
        cache, q = _pair(w, lens, splits=splits)
        out, lse, ref, ref_lse = _both(cache, q)
        assert_close(out, ref, f"{w.name} out")
        assert_close(lse, ref_lse, f"{w.name} lse")
        cache.close()


def test_noalloc_4bit_cache_and_capacity():
    """A 4-bit cache (partials of the splits and of the residual rows), the same with
    pre-RoPE keys, then a smaller bf16 call; and a 4-bit cache too wide for the scratch (512 sequences x 16 query heads x 2
    partials x 130 floats > 8 MiB), which is rejected before anything is launched."""
    w = W.Workload("noalloc-q4", 1, 2, 16, 4, 128, "bf16", 16, 64, 0, 1, 2, seed=107)
    cache, q = _pair(w, [5000, 1300], kv_bits=4)
    out, lse, ref, ref_lse = _both(cache, q)
    assert_close(out, ref, "4-bit out")
    assert_close(lse, ref_lse, "4-bit lse")
    cache.close()
    # the same with pre-RoPE keys (the kernel's rotating form), then smaller again
    cache, q = _pair(w, [3000, 700], kv_bits=4, rope_theta=500000.0)
    out, lse, ref, ref_lse = _both(cache, q)
    assert_close(out, ref, "4-bit pre-RoPE out")
    assert_close(lse, ref_lse, "4-bit pre-RoPE lse")
    cache.close()
    w2 = W.Workload("noalloc-small", 1, 1, 8, 2, 128, "bf16", 4, 32, 0, 1, 1,
                    fixed_mask=((0,),), seed=109)
    cache, q = _pair(w2, [600])
    out, lse, ref, ref_lse = _both(cache, q)
    assert_close(out, ref, "small out")
    cache.close()

    import head_split_kv_amd as hsk
    wide = hsk.DuoCache(num_layers=1, batch=512, num_q_heads=16, num_kv_heads=2, head_dim=128,
                        sink=4, recent=8, capacity=16, retrieval_mask=[[1, 0]],
                        dtype=torch.bfloat16, out_dtype=torch.float32, kv_bits=4)
    k = torch.zeros((512, 1, 2, 128), dtype=torch.bfloat16, device="cuda")
    wide.kv_append(0, k, k)
    q = torch.zeros((512, 16, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((512, 16, 128), dtype=torch.float32, device="cuda")
    st = N.lib().duo_attn_decode_noalloc(wide.handle, 0, ctypes.c_void_p(q.data_ptr()),
                                         ctypes.c_void_p(out.data_ptr()), None, _stream())
    assert st == N.DUO_ERR_CAPACITY, N.status_string(st)
    wide.close()
