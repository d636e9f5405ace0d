"""Kernel timers: one event pair per decode / prefill call while enabled, counts reset on
read, nothing recorded beyond the enabled number of records."""
import pytest
import torch

import workloads as W

from gpu_util import fill, make_cache, step_inputs

pytestmark = pytest.mark.gpu


def test_kernel_timers_count_and_reset():
    import head_split_kv_amd as hsk
    w = W.Workload("timing", 1, 1, 8, 2, 128, "bf16", 4, 32, 0, 4, 1, fixed_mask=((1,),),
                   seed=61, prefill_len=256, prefill_chunk=128)
    cache = make_cache(w, capacity=2048)
    fill(cache, w, 0, [1000])
    hsk.duo_timing_enable(cache, 3)
    lens = [1000]
    for _ in range(4):  # the 4th call is past the 3 records
        q, k, v, _ = step_inputs(w, 0, lens)
        cache.decode_step(0, q, k[:, 0], v[:, 0])
        lens = [n + 1 for n in lens]
    ms, n = hsk.duo_timing_read(cache, "decode")
    assert n == 3 and ms > 0.0
    assert hsk.duo_timing_read(cache, "decode") == (0.0, 0)
    assert hsk.duo_timing_read(cache, "prefill") == (0.0, 0)
    # prefill records only prefill calls
    q = torch.randn(1, 128, 8, 128, device="cuda").to(torch.bfloat16)
    kv = torch.randn(1, 128, 2, 128, device="cuda").to(torch.bfloat16)
    cache.attn_prefill(0, q, kv, kv)
    ms, n = hsk.duo_timing_read(cache, "prefill")
    assert n == 1 and ms > 0.0
    assert hsk.duo_timing_read(cache, "decode") == (0.0, 0)
    hsk.duo_timing_enable(cache, 0)
    q, k, v, _ = step_inputs(w, 0, lens)
    cache.decode_step(0, q, k[:, 0], v[:, 0])
    assert hsk.duo_timing_read(cache, "decode") == (0.0, 0)
    torch.cuda.synchronize()
