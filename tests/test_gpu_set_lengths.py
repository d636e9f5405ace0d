"""duo_cache_init / duo_cache_set_lengths on the GPU: slot tables rebuilt from the lengths
match the oracle's, and a cache whose rows were written outside the library decodes like
the oracle once its lengths are set."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import duo_oracle as O

from gpu_util import assert_close, layer_regions, make_cache, step_inputs, to_dev

pytestmark = pytest.mark.gpu


def test_init_is_empty():
    w = W.Workload("init", 2, 3, 8, 2, 64, "bf16", 4, 16, 0, 1, 1, fixed_mask=((0,), (1,)), seed=71)
    cache = make_cache(w, capacity=64, layers=2)
    assert np.array_equal(cache.lengths(), np.zeros((2, 3), np.int32))
    for layer in range(2):
        assert (cache.slot_positions(layer) == -1).all()


@pytest.mark.parametrize("S,R", [(0, 1), (4, 16), (16, 512)])
def test_set_lengths_rebuilds_slot_tables(S, R):
    w = W.Workload("setlen", 2, 4, 8, 2, 64, "bf16", S, R, 0, 1, 1, fixed_mask=((0,), (1,)), seed=73)
    cache = make_cache(w, capacity=5000, layers=2)
    lens = np.array([[0, 1, S + R - 1, S + R], [S + R + 1, 777, 4096, 5000]], np.int32)
    cache.set_lengths(lens)
    assert np.array_equal(cache.lengths(), lens)
    for layer in range(2):
        got = cache.slot_positions(layer)
        for b in range(4):
            assert np.array_equal(got[b], O.slot_table(int(lens[layer, b]), S, R)), (layer, b)
    # shrinking again is allowed, and so are out-of-range lengths rejected as a whole
    cache.set_lengths(np.zeros((2, 4), np.int32))
    assert (cache.slot_positions(1) == -1).all()
    import head_split_kv_amd as hsk
    with pytest.raises(hsk.DuoError):
        cache.set_lengths(np.full((2, 4), 5001, np.int32))
    assert np.array_equal(cache.lengths(), np.zeros((2, 4), np.int32))


def test_rows_written_outside_then_decode():
    """Write the K/V rows of n tokens straight into the arena (full caches row t, streaming
    caches slot(t) for the held tokens), set the lengths, then run fused decode steps."""
    w = W.Workload("outside", 1, 2, 8, 2, 128, "bf16", 4, 32, 0, 3, 1, fixed_mask=((1,),), seed=79)
    lens0 = [50, 900]
    cache = make_cache(w, capacity=1000)
    reg = layer_regions(cache, 0)
    S, R = w.sink, w.recent
    for b, n in enumerate(lens0):
        kh = W.tokens(w, "k", 0, b, 0, n)
        vh = W.tokens(w, "v", 0, b, 0, n)
        for i, j in enumerate(reg["ret_heads"]):
            reg["full_k"][b, i, :n] = to_dev(kh[:, j], torch.bfloat16)
            reg["full_v"][b, i, :n] = to_dev(vh[:, j], torch.bfloat16)
        table = O.slot_table(n, S, R)
        held = table >= 0
        for i, j in enumerate(reg["str_heads"]):
            reg["str_k"][b, i, np.nonzero(held)[0]] = to_dev(kh[table[held], j], torch.bfloat16)
            reg["str_v"][b, i, np.nonzero(held)[0]] = to_dev(vh[table[held], j], torch.bfloat16)
    cache.set_lengths([lens0])
    mask = W.retrieval_mask(w)[0]
    lens = list(lens0)
    for s in range(3):
        q, k, v, qh = step_inputs(w, 0, lens)
        lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device="cuda")
        out = cache.decode_step(0, q, k[:, 0], v[:, 0], lse=lse)
        lens = [n + 1 for n in lens]
        torch.cuda.synchronize()
        for b, n in enumerate(lens):
            ref, ref_lse = O.decode_step(qh[b], W.tokens(w, "k", 0, b, 0, n),
                                         W.tokens(w, "v", 0, b, 0, n), mask, S, R)
            assert_close(out[b].float().cpu().numpy(), ref, f"step {s} seq {b}")
            assert_close(lse[b].cpu().numpy(), ref_lse, f"step {s} seq {b} lse")
