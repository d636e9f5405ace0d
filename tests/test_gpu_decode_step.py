"""duo_decode_step (append fused into decode) on the GPU: outputs against the oracle and the
cache state against the separate append + decode path, bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import duo_oracle as O

from gpu_util import assert_close, fill, layer_regions, make_cache, step_inputs

pytestmark = pytest.mark.gpu


def _same_state(a, b, layer):
    ra, rb = layer_regions(a, layer), layer_regions(b, layer)
    assert np.array_equal(a.slot_positions(layer), b.slot_positions(layer))
    assert np.array_equal(a.lengths(), b.lengths())
    lens = a.lengths()[layer]
    S, R = a.sink, a.recent
    for bi, n in enumerate(lens):
        assert torch.equal(ra["full_k"][bi, :, :n], rb["full_k"][bi, :, :n])
        assert torch.equal(ra["full_v"][bi, :, :n], rb["full_v"][bi, :, :n])
        used = min(int(n), S + R)
        assert torch.equal(ra["str_k"][bi, :, :used], rb["str_k"][bi, :, :used])
        assert torch.equal(ra["str_v"][bi, :, :used], rb["str_v"][bi, :, :used])


def run_steps(w, lens0, steps, splits=None, check_every=1):
    import head_split_kv_amd as hsk
    ref_cache = make_cache(w, capacity=max(lens0) + steps)
    cache = make_cache(w, capacity=max(lens0) + steps)
    fill(ref_cache, w, 0, lens0)
    fill(cache, w, 0, lens0)
    if splits is not None:
        hsk.duo_set_decode_splits(cache, splits)
        hsk.duo_set_decode_splits(ref_cache, splits)
    mask = W.retrieval_mask(w)[0]
    lens = list(lens0)
    for s in range(steps):
        q, k, v, qh = step_inputs(w, 0, lens)
        ref_cache.kv_append(0, k, v)
        ref_out = ref_cache.attn_decode(0, q)
        lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device="cuda")
        out = cache.decode_step(0, q, k[:, 0], v[:, 0], lse=lse)
        lens = [n + 1 for n in lens]
        if s % check_every:
            continue
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        got_lse = lse.cpu().numpy()
        assert np.max(np.abs(got - ref_out.float().cpu().numpy())) < 4e-3
        for b, n in enumerate(lens):
            kh = W.tokens(w, "k", 0, b, 0, n)
            vh = W.tokens(w, "v", 0, b, 0, n)
            ref, ref_lse = O.decode_step(qh[b], kh, vh, mask, w.sink, w.recent)
            assert_close(got[b], ref, f"step {s} seq {b} out")
            assert_close(got_lse[b], ref_lse, f"step {s} seq {b} lse")
    _same_state(cache, ref_cache, 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_decode_step_from_empty(dtype, G):
    """Steps from an empty cache: the new slot is first unused, then the ring wraps."""
    w = W.Workload("step-empty", 1, 2, 2 * G, 2, 128, dtype, 3, 5, 0, 14, 1,
                   fixed_mask=((1,),), seed=41 + G)
    run_steps(w, [0, 0], 14)


@pytest.mark.parametrize("S,R", [(0, 1), (0, 7), (4, 32), (16, 512)])
def test_decode_step_sink_recent(S, R):
    w = W.Workload("step-sr", 1, 3, 8, 4, 128, "bf16", S, R, 0, 3, 2, fixed_mask=((0, 3),),
                   seed=43)
    run_steps(w, [max(1, S + R - 2), S + R, 1700], 3)


@pytest.mark.parametrize("splits", [1, 3, 64])
def test_decode_step_split_counts(splits):
    """Including split counts where the new token is the only one in its split."""
    w = W.Workload("step-splits", 1, 2, 8, 2, 64, "bf16", 4, 16, 0, 3, 1,
                   fixed_mask=((0,),), seed=47)
    run_steps(w, [5, 130], 3, splits=splits)


def test_decode_step_gqa_128k():
    """The 128K GQA layer: fused steps against the oracle (every 4th step checked)."""
    w = W.workload("c3").with_(decode_steps=9)
    run_steps(w, [w.context], 9, check_every=4)
