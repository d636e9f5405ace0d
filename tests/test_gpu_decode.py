"""duo_attn_decode on the GPU against the CPU float64 oracle.

Every case fills a context by bulk append, then runs steps of (append one token, decode at
that position) and compares out and lse elementwise with |gpu - ref| <= 2e-3 + 1e-2 |ref|.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import duo_oracle as O

from gpu_util import assert_close, fill, make_cache, step_inputs, to_dev

pytestmark = pytest.mark.gpu


def run_decode(w, lens0, steps, check_steps=None, splits=None, out_dtype=torch.float32,
               layer=0, mask_layer=None, heads=None, cache=None):
    """Fill, then decode ``steps`` steps; check the steps in ``check_steps`` (default all)."""
    import head_split_kv_amd as hsk
    gl = layer if mask_layer is None else mask_layer
    if cache is None:
        cache = make_cache(w, out_dtype=out_dtype, capacity=max(lens0) + steps)
        fill(cache, w, layer, lens0, mask_layer=gl)
    if splits is not None:
        hsk.duo_set_decode_splits(cache, splits)
    mask = W.retrieval_mask(w)[gl]
    lens = list(lens0)
    worst = 0.0
    for s in range(steps):
        q, k, v, qh = step_inputs(w, gl, lens)
        cache.kv_append(layer, k, v)
        lens = [n + 1 for n in lens]
        lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device="cuda")
        out = cache.attn_decode(layer, q, lse=lse)
        if check_steps is not None and s not in check_steps:
            continue
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        got_lse = lse.cpu().numpy()
        for b, n in enumerate(lens):
            kh = W.tokens(w, "k", gl, b, 0, n)
            vh = W.tokens(w, "v", gl, b, 0, n)
            if heads is None:
                ref, ref_lse = O.decode_step(qh[b], kh, vh, mask, w.sink, w.recent)
                worst = max(worst, assert_close(got[b], ref, f"step {s} seq {b} out"))
                assert_close(got_lse[b], ref_lse, f"step {s} seq {b} lse")
            else:  # a subset of KV heads (their query groups), for very long contexts
                G = w.group
                for j in heads:
                    hq = slice(j * G, (j + 1) * G)
                    ref, ref_lse = O.decode_step(qh[b][hq], kh[:, j:j + 1], vh[:, j:j + 1],
                                                 mask[j:j + 1], w.sink, w.recent)
                    worst = max(worst, assert_close(got[b][hq], ref, f"step {s} seq {b} kv {j}"))
                    assert_close(got_lse[b][hq], ref_lse, f"step {s} seq {b} kv {j} lse")
    return cache, worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_variants(dtype, d, G):
    """Every built (dtype, head_dim, group) variant; ragged batch around S+R."""
    w = W.Workload("decode-variant", 1, 3, 2 * G, 2, d, dtype, 4, 32, 0, 3, 1,
                   fixed_mask=((1,),), seed=3 + G)
    run_decode(w, [1, 37, 1500], 3)


@pytest.mark.parametrize("S", [0, 4, 16])
@pytest.mark.parametrize("R", [1, 32, 512])
def test_decode_sink_recent(S, R):
    """Sink/recent sizes, lengths just below, at and above S+R, and long."""
    w = W.Workload("decode-sr", 1, 4, 8, 4, 128, "bf16", S, R, 0, 2, 2, fixed_mask=((0, 3),),
                   seed=5)
    run_decode(w, [max(1, S + R - 2), S + R - 1 if S + R > 1 else 1, S + R + 3, 2100], 2)


@pytest.mark.parametrize("splits", [1, 7, 64, 0])
def test_decode_split_count_invariance(splits):
    """The result does not depend on the number of context splits (log-sum-exp merge)."""
    w = W.Workload("decode-splits", 1, 2, 8, 2, 128, "bf16", 16, 64, 0, 2, 1,
                   fixed_mask=((0,),), seed=7)
    run_decode(w, [5000, 333], 2, splits=splits)


def test_decode_bf16_output():
    w = W.Workload("decode-bf16-out", 1, 2, 8, 2, 128, "bf16", 4, 32, 0, 2, 1,
                   fixed_mask=((1,),), seed=9)
    run_decode(w, [2000, 40], 2, out_dtype=torch.bfloat16)


def test_decode_all_retrieval_and_all_streaming():
    for mask in (((0, 1),), ((),)):
        w = W.Workload("decode-pure", 1, 2, 8, 2, 128, "bf16", 4, 32, 0, 2, 1,
                       fixed_mask=mask, seed=13)
        run_decode(w, [1000, 5], 2)


def test_decode_c1_tiny_gqa_fp32():
    """Tiny GQA decode: 1,024-token context, 16 steps, every output checked."""
    w = W.workload("c1")
    _, worst = run_decode(w, [w.context], w.decode_steps)
    assert worst < 1e-4  # fp32 inputs: only accumulation-order differences remain


def test_decode_c2_mha_32k():
    """Llama-2-7B-shaped MHA layer at 32K context, 64 steps, every step checked."""
    w = W.workload("c2")
    run_decode(w, [w.context], w.decode_steps)


@pytest.mark.timeout(600)
def test_decode_c3_gqa_128k():
    """Llama-3-8B-shaped GQA layer at 128K context, 128 steps, every step checked."""
    w = W.workload("c3")
    run_decode(w, [w.context], w.decode_steps)


def _progress(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.timeout(900)
def test_decode_c4_full_depth_ragged_batch():
    """32 layers, batch 8, ragged 16K..32K, per-layer retrieval masks at 50 %, every layer
    with its own seeded K/V/q streams (so a layer that read or wrote another layer's region
    would see other data). Every layer runs every step (even layers through the fused
    duo_decode_step, odd ones through duo_kv_append + duo_attn_decode); the oracle checks the
    first and last step on every layer and sequence, each layer's history regenerated from
    its streams after the run."""
    w = W.workload("c4")
    lens0 = [int(x) for x in W.initial_lengths(w)]
    steps = w.decode_steps
    cache = make_cache(w, capacity=max(lens0) + steps, layers=w.layers)
    dt = torch.bfloat16
    for layer in range(w.layers):
        for b, n in enumerate(lens0):
            k = to_dev(W.tokens(w, "k", layer, b, 0, n), dt)
            v = to_dev(W.tokens(w, "v", layer, b, 0, n), dt)
            cache.kv_append(layer, k, v, seq=b)
            del k, v
        if layer % 8 == 7:
            _progress(f"c4: filled layers 0..{layer}")
    masks = W.retrieval_mask(w)
    # the step tokens of every layer: [steps, B, heads, d] on the device
    step_tok = []
    for layer in range(w.layers):
        step_tok.append(tuple(
            to_dev(np.stack([W.tokens(w, kind, layer, b, n0, n0 + steps)
                             for b, n0 in enumerate(lens0)], axis=1), dt) for kind in "qkv"))
    _progress("c4: step tokens generated")
    lens = list(lens0)
    check = (0, steps - 1)
    outs = {}  # (step, layer) -> out [B, Hq, d] on the host
    for s in range(steps):
        for layer in range(w.layers):
            qs, ks, vs = step_tok[layer]
            q, k, v = qs[s], ks[s][:, None], vs[s][:, None]
            if layer % 2:  # odd layers: append then decode; even layers: the fused step
                cache.kv_append(layer, k, v)
                out = cache.attn_decode(layer, q)
            else:
                out = cache.decode_step(layer, q, k[:, 0], v[:, 0])
            if s in check:
                outs[(s, layer)] = out.float().cpu().numpy()
        lens = [n + 1 for n in lens]
    _progress(f"c4: {steps} steps run on all {w.layers} layers")
    for layer in range(w.layers):
        for b, n0 in enumerate(lens0):
            kh = W.tokens(w, "k", layer, b, 0, n0 + steps)
            vh = W.tokens(w, "v", layer, b, 0, n0 + steps)
            qh = W.tokens(w, "q", layer, b, n0, n0 + steps)
            for s in check:
                n = n0 + s + 1
                ref, _ = O.decode_step(qh[s], kh[:n], vh[:n], masks[layer], w.sink, w.recent)
                assert_close(outs[(s, layer)][b], ref, f"c4 step {s} layer {layer} seq {b}")
        _progress(f"c4: layer {layer} checked (steps {check}, all sequences)")


@pytest.fixture(scope="module")
def history_1m():
    """K, V of the first 1,048,576 + 4 positions of the 1M-context stream (shared by the
    50 % and 25 % retrieval variants, whose streams are identical)."""
    w = W.workload("c5")
    n = w.context + 4
    k = W.tokens(w, "k", 0, 0, 0, n)
    v = W.tokens(w, "v", 0, 0, 0, n)
    q = W.tokens(w, "q", 0, 0, w.context, n)
    _progress("c5: history generated")
    return k, v, q


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["c5", "c5q"])
def test_decode_c5_1m_context(key, history_1m):
    """1,048,576-token context, 50 % and 25 % retrieval KV heads; all 4 steps are checked on
    all 8 KV heads (their 32 query heads)."""
    w = W.workload(key)
    kh, vh, qh = history_1m
    mask = W.retrieval_mask(w)[0]
    heads = list(range(w.hkv))
    n0 = w.context
    cache = make_cache(w, capacity=n0 + 4)
    dt = torch.bfloat16
    for t0 in range(0, n0, 1 << 17):
        t1 = min(n0, t0 + (1 << 17))
        cache.kv_append(0, to_dev(kh[t0:t1], dt), to_dev(vh[t0:t1], dt), seq=0)
    _progress(f"{key}: filled")
    G = w.group
    for s in range(4):
        p = n0 + s
        cache.kv_append(0, to_dev(kh[p:p + 1][None], dt), to_dev(vh[p:p + 1][None], dt))
        lse = torch.empty((1, w.hq), dtype=torch.float32, device="cuda")
        out = cache.attn_decode(0, to_dev(qh[s:s + 1], dt), lse=lse)
        got = out.float().cpu().numpy()[0]
        got_lse = lse.cpu().numpy()[0]
        for j in heads:
            hq = slice(j * G, (j + 1) * G)
            ref, ref_lse = O.decode_step(qh[s][hq], kh[:p + 1, j:j + 1], vh[:p + 1, j:j + 1],
                                         mask[j:j + 1], w.sink, w.recent)
            assert_close(got[hq], ref, f"{key} step {s} kv {j}")
            assert_close(got_lse[hq], ref_lse, f"{key} step {s} kv {j} lse")
        _progress(f"{key}: step {s} checked")


@pytest.mark.timeout(900)
def test_decode_c5_1m_context_kv4(history_1m):
    """The 1,048,576-token layer at 50 % retrieval with 4-bit full caches: 2 steps, checked on
    two retrieval KV heads and one streaming head against decode_step_kv4."""
    import head_split_kv_amd as hsk
    w = W.workload("c5")
    kh, vh, qh = history_1m
    mask = W.retrieval_mask(w)[0]
    ret = [int(j) for j in np.nonzero(mask)[0]]
    heads = [ret[0], ret[-1], int(np.nonzero(mask == 0)[0][0])]
    n0 = w.context
    cache = hsk.DuoCache(num_layers=1, batch=1, num_q_heads=w.hq, num_kv_heads=w.hkv,
                         head_dim=w.d, sink=w.sink, recent=w.recent, capacity=n0 + 2,
                         retrieval_mask=[mask], dtype=torch.bfloat16, out_dtype=torch.float32,
                         kv_bits=4)
    dt = torch.bfloat16
    for t0 in range(0, n0, 1 << 17):
        t1 = min(n0, t0 + (1 << 17))
        cache.kv_append(0, to_dev(kh[t0:t1], dt), to_dev(vh[t0:t1], dt), seq=0)
    _progress("c5 4-bit: filled")
    G = w.group
    for s in range(2):
        p = n0 + s
        cache.kv_append(0, to_dev(kh[p:p + 1][None], dt), to_dev(vh[p:p + 1][None], dt))
        lse = torch.empty((1, w.hq), dtype=torch.float32, device="cuda")
        out = cache.attn_decode(0, to_dev(qh[s:s + 1], dt), lse=lse)
        got = out.float().cpu().numpy()[0]
        got_lse = lse.cpu().numpy()[0]
        for j in heads:
            hq = slice(j * G, (j + 1) * G)
            ref, ref_lse = O.decode_step_kv4(qh[s][hq], kh[:p + 1, j:j + 1], vh[:p + 1, j:j + 1],
                                             mask[j:j + 1], w.sink, w.recent)
            assert_close(got[hq], ref, f"c5 4-bit step {s} kv {j}")
            assert_close(got_lse[hq], ref_lse, f"c5 4-bit step {s} kv {j} lse")
        _progress(f"c5 4-bit: step {s} checked")
    cache.close()


def test_decode_split_merge_reads_only_its_own_call():
    """Back-to-back calls that share the cache's split-K workspace, at automatic, 48 and 3
    splits: every call's outputs match the oracle, so no merge reads a partial left by the
    call before. The queries alternate between unrelated draws (one scaled by -3) and two
    layers of different lengths, so stale partials would be far off."""
    import head_split_kv_amd as hsk
    w = W.Workload("decode-fused-merge", 2, 2, 32, 8, 128, "bf16", 16, 64, 0, 1, 4, seed=111)
    lens_by_layer = [[20000, 3000], [9000, 15000]]
    cache = make_cache(w, capacity=20001, layers=2)
    for layer in range(2):
        fill(cache, w, layer, lens_by_layer[layer])
    masks = W.retrieval_mask(w)
    hist = {}
    for layer in range(2):
        q, k, v, _ = step_inputs(w, layer, lens_by_layer[layer])
        cache.kv_append(layer, k, v)
        hist[layer] = [(W.tokens(w, "k", layer, b, 0, n + 1), W.tokens(w, "v", layer, b, 0, n + 1))
                       for b, n in enumerate(lens_by_layer[layer])]
    rng = np.random.default_rng(5)
    for splits in (0, 48, 3):
        hsk.duo_set_decode_splits(cache, splits)
        for rep in range(4):
            layer = rep % 2
            qh = rng.standard_normal((w.batch, w.hq, w.d)).astype(np.float32)
            qh = W.bf16_round(qh * (1.0 if rep < 2 else -3.0))
            out = cache.attn_decode(layer, to_dev(qh, torch.bfloat16))
            got = out.float().cpu().numpy()
            for b in range(w.batch):
                kh, vh = hist[layer][b]
                ref, _ = O.decode_step(qh[b], kh, vh, masks[layer], w.sink, w.recent)
                assert_close(got[b], ref, f"splits {splits} call {rep} layer {layer} seq {b}")


def test_decode_wide_grid():
    """A batch whose blocks cannot all be resident at once (16 sequences x 4 retrieval heads x
    64 forced splits): the splits run in several rounds and their merge still matches the
    oracle."""
    w = W.Workload("decode-wide", 1, 16, 32, 8, 128, "bf16", 16, 64, 0, 2, 4, seed=113)
    run_decode(w, [3000 + 97 * b for b in range(16)], 2, splits=64)
