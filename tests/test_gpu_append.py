"""duo_kv_append on the GPU against the oracle's cache state: slot tables and every stored
row must match bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import duo_oracle as O

from gpu_util import fill, layer_regions, make_cache, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _check_state(cache, w, layer, lens, mask_layer=None):
    """Compare the slot table and all rows of one layer with the oracle, bit-exact."""
    gl = layer if mask_layer is None else mask_layer
    S, R = w.sink, w.recent
    torch.cuda.synchronize()
    slots = cache.slot_positions(layer)
    reg = layer_regions(cache, layer)
    for b, n in enumerate(lens):
        want = O.slot_table(int(n), S, R)
        assert np.array_equal(slots[b], want), (b, n, slots[b], want)
        if n == 0:
            continue
        k = W.tokens(w, "k", gl, b, 0, int(n))
        v = W.tokens(w, "v", gl, b, 0, int(n))
        for r, j in enumerate(reg["ret_heads"]):
            gk = reg["full_k"][b, r, :n].float().cpu().numpy()
            gv = reg["full_v"][b, r, :n].float().cpu().numpy()
            assert np.array_equal(gk, k[:, j]) and np.array_equal(gv, v[:, j]), (b, j)
        for s, j in enumerate(reg["str_heads"]):
            rows_k, table = O.streaming_cache_rows(k[:, j], int(n), S, R)
            rows_v, _ = O.streaming_cache_rows(v[:, j], int(n), S, R)
            ok = table >= 0
            gk = reg["str_k"][b, s].float().cpu().numpy()
            gv = reg["str_v"][b, s].float().cpu().numpy()
            assert np.array_equal(gk[ok], rows_k[ok]), (b, j)
            assert np.array_equal(gv[ok], rows_v[ok]), (b, j)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S,R", [(0, 1), (3, 5), (4, 32), (16, 7)])
def test_append_patterns(dtype, S, R):
    """Append counts 1, < R, = R, > R, > S+R, and appends that straddle the sink boundary,
    on three sequences of different lengths."""
    w = W.Workload("append-tiny", 1, 3, 4, 2, 64, dtype, S, R, 0, 0, 1, fixed_mask=((0,),),
                   seed=11)
    cache = make_cache(w, capacity=400)
    lens = [0, 0, 0]
    plan = [(0, 1), (1, S + 1 if S else 2), (2, R), (0, R + 3), (1, S + R + 5), (2, 1),
            (0, max(1, R - 1)), (1, 2 * (S + R) + 1), (2, 3 * R)]
    dt = torch_dtype(dtype)
    for b, m in plan:
        k = to_dev(W.tokens(w, "k", 0, b, lens[b], lens[b] + m), dt)
        v = to_dev(W.tokens(w, "v", 0, b, lens[b], lens[b] + m), dt)
        cache.kv_append(0, k, v, seq=b)
        lens[b] += m
        _check_state(cache, w, 0, lens)
    assert np.array_equal(cache.lengths()[0], lens)
    # a batched append of 2 tokens to every sequence
    k = np.stack([W.tokens(w, "k", 0, b, lens[b], lens[b] + 2) for b in range(3)])
    v = np.stack([W.tokens(w, "v", 0, b, lens[b], lens[b] + 2) for b in range(3)])
    cache.kv_append(0, to_dev(k, dt), to_dev(v, dt), seq=-1)
    lens = [n + 2 for n in lens]
    _check_state(cache, w, 0, lens)


def test_append_c1_fill_and_steps():
    """Tiny GQA workload: fill 1,024 tokens, then 16 one-token appends."""
    w = W.workload("c1")
    cache = make_cache(w)
    fill(cache, w, 0, [w.context])
    _check_state(cache, w, 0, [w.context])
    dt = torch_dtype(w.dtype)
    for i in range(w.decode_steps):
        p = w.context + i
        cache.kv_append(0, to_dev(W.tokens(w, "k", 0, 0, p, p + 1)[None], dt),
                        to_dev(W.tokens(w, "v", 0, 0, p, p + 1)[None], dt))
        _check_state(cache, w, 0, [p + 1])


def test_append_chunking_invariance():
    """One bulk append and many small ones leave identical caches."""
    w = W.workload("c3").with_(context=3000, decode_steps=0)
    a = make_cache(w, capacity=3000)
    b = make_cache(w, capacity=3000)
    fill(a, w, 0, [3000], chunk=3000)
    fill(b, w, 0, [3000], chunk=97)
    torch.cuda.synchronize()
    ra, rb = layer_regions(a, 0), layer_regions(b, 0)
    for key in ("full_k", "full_v", "str_k", "str_v"):
        assert torch.equal(ra[key], rb[key]), key
    assert np.array_equal(a.slot_positions(0), b.slot_positions(0))
    _check_state(a, w, 0, [3000])


def test_reset_empties_the_cache():
    w = W.workload("c1")
    cache = make_cache(w)
    fill(cache, w, 0, [100])
    cache_lens = cache.lengths()
    assert cache_lens[0, 0] == 100
    import head_split_kv_amd as hsk
    hsk.duo_cache_reset(cache)
    assert cache.lengths()[0, 0] == 0
    assert np.all(cache.slot_positions(0) == -1)
    fill(cache, w, 0, [50])
    _check_state(cache, w, 0, [50])
