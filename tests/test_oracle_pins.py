"""Pins of the CPU oracle against things other than itself (CPU only).

Each ``pin_*`` function checks one oracle function against an independent formulation:
a literal simulation of the cache policy, a scalar-loop softmax over the simulated cache,
torch's float64 ``scaled_dot_product_attention``, attention over a sliced window, the
worked example of the chunked pre-filling figure and the memory numbers the pages print.
``test_planted_mistakes_are_caught`` plants plausible mistakes in the oracle (on the CPU)
and requires that some pin fails for each.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import duo_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------------------------
# Independent formulations used by the pins
# --------------------------------------------------------------------------------------------

def sim_decode_cache(n, S, R):
    """Streaming cache as a Python list, per the decoding procedure: append each token, and
    when the cache holds more than S+R tokens drop the oldest token that is not a sink."""
    cache = []
    for t in range(n):
        cache.append(t)
        if len(cache) > S + R:
            victim = min(x for x in cache if x >= S)
            cache.remove(victim)
    return cache


def sim_chunked_cache(n, S, R, chunk):
    """Chunked pre-filling: append a whole chunk, then prune to sinks + last R non-sinks."""
    cache = []
    for c0 in range(0, n, chunk):
        cache.extend(range(c0, min(n, c0 + chunk)))
        sinks = [x for x in cache if x < S]
        rest = [x for x in cache if x >= S]
        cache = sinks + rest[len(rest) - min(R, len(rest)):]
    return cache


def sim_ring_pointer(n, S, R):
    """Physical slots filled with a write pointer: sinks fill 0..S-1, then the pointer runs
    over S..S+R-1 and wraps back to S."""
    slots = [-1] * (S + R)
    ptr = 0
    for t in range(n):
        if t < S:
            slots[t] = t
            ptr = S
            continue
        slots[ptr] = t
        ptr = ptr + 1 if ptr + 1 < S + R else S
    return slots


def scalar_head_attention(q, keys, vals, scale):
    """Softmax over the given keys with Python floats: returns (out list, lse)."""
    z = [scale * math.fsum(qi * ki for qi, ki in zip(q, k)) for k in keys]
    m = max(z)
    w = [math.exp(x - m) for x in z]
    den = math.fsum(w)
    d = len(vals[0])
    out = [math.fsum(w[i] * vals[i][c] for i in range(len(keys))) / den for c in range(d)]
    return out, m + math.log(den)


def rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------------------------

def pin_cache_policy():
    for S in range(0, 5):
        for R in range(1, 7):
            for n in range(0, 25):
                want = sorted(sim_decode_cache(n, S, R))
                assert sorted(O.streaming_valid_tokens(n, S, R).tolist()) == want, (S, R, n)
                table = O.slot_table(n, S, R)
                assert sorted(int(x) for x in table if x >= 0) == want, (S, R, n)
                assert list(table) == sim_ring_pointer(n, S, R), (S, R, n)
                for chunk in range(1, n + 1):
                    if n % chunk == 0:
                        assert sorted(sim_chunked_cache(n, S, R, chunk)) == want, (S, R, n, chunk)


def pin_streaming_rows():
    rng = np.random.default_rng(1)
    S, R, n = 3, 5, 17
    x = rand(rng, n, 4)
    rows, table = O.streaming_cache_rows(x, n, S, R)
    slots = sim_ring_pointer(n, S, R)
    for s, t in enumerate(slots):
        if t < 0:
            assert np.all(np.isnan(rows[s]))
        else:
            assert np.array_equal(rows[s], x[t])


def pin_decode_scalar_bruteforce():
    """Decode output from the list-simulated cache with a scalar-loop softmax."""
    rng = np.random.default_rng(2)
    for (S, R, Hkv, G, d) in [(2, 3, 2, 2, 4), (0, 2, 1, 3, 3), (1, 1, 2, 1, 5), (4, 6, 1, 2, 2)]:
        retrieval = np.array([1, 0][:Hkv] if Hkv > 1 else [0])
        n = 13
        k = rand(rng, n, Hkv, d)
        v = rand(rng, n, Hkv, d)
        q = rand(rng, Hkv * G, d)
        out, lse = O.decode_step(q, k, v, retrieval, S, R)
        for h in range(Hkv * G):
            j = h // G
            pos = list(range(n)) if retrieval[j] else sim_decode_cache(n, S, R)
            o_ref, l_ref = scalar_head_attention(q[h].tolist(), [k[t, j].tolist() for t in pos],
                                                 [v[t, j].tolist() for t in pos], 1 / math.sqrt(d))
            assert np.allclose(out[h], o_ref, rtol=0, atol=1e-12), (S, R, h)
            assert abs(lse[h] - l_ref) < 1e-12, (S, R, h)


def _sdpa_causal(q, k, v):
    """torch float64 causal attention, ``[T, H, d]`` inputs, all queries 0..T-1."""
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    return o[0].permute(1, 0, 2).numpy()


def pin_all_retrieval_is_causal_attention():
    rng = np.random.default_rng(3)
    for (Hkv, G, d, T, start) in [(2, 4, 8, 40, 17), (4, 1, 16, 33, 0), (1, 8, 4, 20, 19)]:
        q = rand(rng, T, Hkv * G, d)
        k = rand(rng, T, Hkv, d)
        v = rand(rng, T, Hkv, d)
        ref = _sdpa_causal(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1))
        out, _ = O.prefill_chunk(q[start:], k, v, start, np.ones(Hkv), 2, 3)
        assert np.allclose(out, ref[start:], rtol=0, atol=1e-12)
        o1, _ = O.decode_step(q[T - 1], k, v, np.ones(Hkv), 2, 3)
        assert np.allclose(o1, ref[T - 1], rtol=0, atol=1e-12)


def pin_short_streaming_is_full():
    """A streaming head whose context holds at most S+R tokens sees everything."""
    rng = np.random.default_rng(4)
    S, R, d = 3, 6, 8
    for n in range(1, S + R + 1):
        k = rand(rng, n, 1, d)
        v = rand(rng, n, 1, d)
        q = rand(rng, 2, d)
        a, la = O.decode_step(q, k, v, [0], S, R)
        b, lb = O.decode_step(q, k, v, [1], S, R)
        assert np.array_equal(a, b) and np.array_equal(la, lb)
    n = S + R + 4  # beyond S+R the two must differ
    k, v, q = rand(rng, n, 1, d), rand(rng, n, 1, d), rand(rng, 2, d)
    a, _ = O.decode_step(q, k, v, [0], S, R)
    b, _ = O.decode_step(q, k, v, [1], S, R)
    assert not np.allclose(a, b)


def pin_no_sink_is_sliding_window():
    """S = 0: attention over the slice [p-R+1, p]; R >= n: full causal attention."""
    rng = np.random.default_rng(5)
    T, Hkv, G, d = 30, 2, 2, 8
    q = rand(rng, T, Hkv * G, d)
    k = rand(rng, T, Hkv, d)
    v = rand(rng, T, Hkv, d)
    for R in (1, 4, 9):
        out, _ = O.prefill_chunk(q, k, v, 0, np.zeros(Hkv), 0, R)
        for p in range(T):
            lo = max(0, p - R + 1)
            kk = np.repeat(k[lo:p + 1], G, axis=1)
            vv = np.repeat(v[lo:p + 1], G, axis=1)
            z = np.einsum("hd,thd->ht", q[p], kk) / math.sqrt(d)
            w = np.exp(z - z.max(axis=1, keepdims=True))
            ref = np.einsum("ht,thd->hd", w / w.sum(axis=1, keepdims=True), vv)
            assert np.allclose(out[p], ref, rtol=0, atol=1e-12), (R, p)
    full = _sdpa_causal(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1))
    out, _ = O.prefill_chunk(q, k, v, 0, np.zeros(Hkv), 0, T)
    assert np.allclose(out, full, rtol=0, atol=1e-12)


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, *kv = line.split()
            d = dict(x.split("=", 1) for x in kv)
            rows.append((kind, d))
    return rows


def pin_fig5_worked_example():
    rows = _read_golden("chunked_prefill_fig5.txt")
    head = rows[0][1] if rows[0][0].startswith("sink") else None
    S, R, chunk = 1, 2, 4
    assert rows[0][0] == "sink=1"
    assert head["recent"] == "2" and head["chunk"] == "4"
    for kind, d in rows[1:]:
        if not kind.startswith("after="):
            continue
        n = int(kind.split("=")[1])
        want = sorted(int(x) for x in d["cache"].split(","))
        assert sorted(O.streaming_valid_tokens(n, S, R).tolist()) == want
        assert sorted(sim_chunked_cache(n, S, R, chunk)) == want
        table = O.slot_table(n, S, R)
        assert sorted(int(x) for x in table if x >= 0) == want
    # the ring convention places them as [0, 3, 2] and [0, 7, 6]
    assert list(O.slot_table(4, S, R)) == [0, 3, 2]
    assert list(O.slot_table(8, S, R)) == [0, 7, 6]


def pin_chunk_granular_fig5():
    """Chunk-granular reading: the second chunk of Figure 5 sees the pruned cache {0, 2, 3}
    plus its own tokens up to the query."""
    rows = _read_golden("chunked_prefill_fig5.txt")
    att = [d for kind, d in rows if kind == "attend"]
    assert len(att) == 1
    start = int(att[0]["start"])
    held = [int(x) for x in att[0]["held"].split(",")]
    S, R, chunk = 1, 2, 4
    assert sorted(sim_chunked_cache(start, S, R, chunk)) == held
    q_pos = np.arange(start, start + chunk)
    m = O.chunk_visible_mask(q_pos, np.arange(start + chunk), start, False, S, R)
    for i, p in enumerate(q_pos):
        assert sorted(np.nonzero(m[i])[0].tolist()) == held + list(range(start, p + 1))
    assert np.array_equal(O.chunk_visible_mask(q_pos, np.arange(8), start, True, S, R),
                          O.visible_mask(q_pos, np.arange(8), True, S, R))


def pin_chunk_granular_gather():
    """Chunk-granular prefill equals plain attention over the gathered keys [pruned cache ;
    chunk] with a causal mask on the chunk part, the pruned cache taken from the chunked
    cache simulation (chunks of the same size before this one)."""
    rng = np.random.default_rng(11)
    for (S, R, chunk, n_chunks, G) in [(2, 5, 4, 4, 1), (1, 2, 4, 2, 2), (0, 3, 7, 3, 1), (3, 9, 5, 4, 4)]:
        T = chunk * n_chunks
        d = 8
        q = rand(rng, T, G, d)
        k = rand(rng, T, 1, d)
        v = rand(rng, T, 1, d)
        for c in range(n_chunks):
            start = c * chunk
            held = sorted(sim_chunked_cache(start, S, R, chunk))
            out, lse = O.prefill_chunk(q[start:start + chunk], k, v, start, [0], S, R,
                                       chunk_granular=True)
            for i in range(chunk):
                keys = held + list(range(start, start + i + 1))
                for h in range(G):
                    z = (k[keys, 0] @ q[start + i, h]) / math.sqrt(d)
                    w = np.exp(z - z.max())
                    ref = (w @ v[keys, 0]) / w.sum()
                    assert np.allclose(out[i, h], ref, rtol=0, atol=1e-12), (S, R, chunk, c, i)
                    assert abs(lse[i, h] - (z.max() + math.log(w.sum()))) < 1e-12


def pin_chunk_granular_short_is_full():
    """While the chunk starts within the first S+R tokens the pruned cache is the whole
    prefix, so the chunk-granular streaming head is causal attention."""
    rng = np.random.default_rng(12)
    S, R, d = 2, 6, 8
    T = 20
    q = rand(rng, T, 1, d)
    k = rand(rng, T, 1, d)
    v = rand(rng, T, 1, d)
    ref = _sdpa_causal(q, k, v)
    for start in (0, 3, S + R):
        out, _ = O.prefill_chunk(q[start:], k, v, start, [0], S, R, chunk_granular=True)
        assert np.allclose(out, ref[start:], rtol=0, atol=1e-12), start
    out, _ = O.prefill_chunk(q[S + R + 1:], k, v, S + R + 1, [0], S, R, chunk_granular=True)
    assert not np.allclose(out, ref[S + R + 1:])


def pin_memory_numbers():
    rows = _read_golden("kv_memory.txt")
    for kind, d in rows:
        if kind == "full_fp16_bytes":
            b = 2 * O.full_kv_elements(int(d["layers"]), int(d["kv_heads"]), int(d["tokens"]),
                                       int(d["d"]))
            assert b == 137_438_953_472
            assert 137e9 <= b < 138e9
        elif kind == "budget_ratio":
            got = O.budget_ratio(float(d["r"]), int(d["length"]), int(d["sink"]), int(d["recent"]))
            assert abs(got - float(d["value"])) < 1e-12
        elif kind == "budget_ratio_page_discrepancy":
            r, L = float(d["r"]), int(d["length"])
            SR = int(d["sink"]) + int(d["recent"])
            got = O.budget_ratio(r, L, int(d["sink"]), int(d["recent"]))
            assert abs(got - float(d["formula"])) < 1e-12
            # the printed value equals the streaming term weighted by r instead of 1 - r
            assert abs((r * L + r * SR) / L - float(d["page"])) < 1e-12
    # limits: 25 % retrieval (MHA) -> 4x less KV, 50 % (GQA) -> 2x, as L grows
    assert abs(1 / O.budget_ratio(0.25, 10**9, 64, 256) - 4) < 1e-5
    assert abs(1 / O.budget_ratio(0.5, 10**9, 64, 256) - 2) < 1e-5


def pin_memory_formula_by_count():
    """Per-layer element count equals the tokens stored by the simulated caches times d."""
    for (Hr, Hs, S, R, d) in [(1, 3, 2, 5, 4), (8, 24, 16, 512, 128), (0, 2, 0, 3, 2)]:
        for L in (0, 1, 3, S + R - 1, S + R, S + R + 1, 4 * (S + R) + 3):
            counted = (Hr * L + Hs * len(sim_decode_cache(L, S, R))) * d
            assert O.duo_kv_elements_layer(Hr, Hs, L, S, R, d) == counted, (L, S, R)
            full = O.full_kv_elements(1, Hr + Hs, L, d)
            assert full == 2 * (Hr + Hs) * L * d


def pin_chunk_invariance_and_decode_equivalence():
    rng = np.random.default_rng(6)
    T, Hkv, G, d, S, R = 23, 3, 2, 6, 2, 4
    retrieval = np.array([0, 1, 0])
    q = rand(rng, T, Hkv * G, d)
    k = rand(rng, T, Hkv, d)
    v = rand(rng, T, Hkv, d)
    one, lone = O.prefill_chunk(q, k, v, 0, retrieval, S, R)
    for chunk in (1, 3, 7, T):
        parts = [O.prefill_chunk(q[c:c + chunk], k, v, c, retrieval, S, R)
                 for c in range(0, T, chunk)]
        got = np.concatenate([p[0] for p in parts])
        assert np.allclose(got, one, rtol=0, atol=1e-13)
    for p in range(T):
        o, l = O.decode_step(q[p], k[:p + 1], v[:p + 1], retrieval, S, R)
        assert np.allclose(o, one[p], rtol=0, atol=1e-13)
        assert np.allclose(l, lone[p], rtol=0, atol=1e-13)


def pin_head_permutation():
    """Permuting KV heads (with their flags and query groups) permutes the outputs."""
    rng = np.random.default_rng(7)
    T, Hkv, G, d, S, R = 19, 4, 2, 5, 1, 3
    retrieval = np.array([1, 0, 0, 1])
    q = rand(rng, T, Hkv * G, d)
    k = rand(rng, T, Hkv, d)
    v = rand(rng, T, Hkv, d)
    perm = np.array([2, 0, 3, 1])
    qperm = np.concatenate([np.arange(j * G, (j + 1) * G) for j in perm])
    a, _ = O.prefill_chunk(q, k, v, 0, retrieval, S, R)
    b, _ = O.prefill_chunk(q[:, qperm], k[:, perm], v[:, perm], 0, retrieval[perm], S, R)
    assert np.allclose(a[:, qperm], b, rtol=0, atol=1e-13)


def pin_gqa_equals_repeated_mha():
    rng = np.random.default_rng(8)
    T, Hkv, G, d, S, R = 17, 2, 4, 8, 2, 5
    retrieval = np.array([0, 1])
    q = rand(rng, T, Hkv * G, d)
    k = rand(rng, T, Hkv, d)
    v = rand(rng, T, Hkv, d)
    a, la = O.prefill_chunk(q, k, v, 0, retrieval, S, R)
    b, lb = O.prefill_chunk(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0,
                            np.repeat(retrieval, G), S, R)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def pin_lambda_mask_literal():
    """S=2, R=3 over 7 positions, written out by hand from the mask's description."""
    want = np.array([
        [1, 0, 0, 0, 0, 0, 0],
        [1, 1, 0, 0, 0, 0, 0],
        [1, 1, 1, 0, 0, 0, 0],
        [1, 1, 1, 1, 0, 0, 0],
        [1, 1, 1, 1, 1, 0, 0],
        [1, 1, 0, 1, 1, 1, 0],
        [1, 1, 0, 0, 1, 1, 1],
    ], dtype=bool)
    got = O.visible_mask(np.arange(7), np.arange(7), False, 2, 3)
    assert np.array_equal(got, want)
    assert np.array_equal(O.visible_mask(np.arange(7), np.arange(7), True, 2, 3),
                          np.tril(np.ones((7, 7), dtype=bool)))


def pin_retrieval_count_nearest():
    """The retrieval count is the integer nearest ratio * N (the product rounded to double,
    halves up), by search over every count; the pages' two budgets give 256 of the 1,024 Llama-2-7B heads and 128 of the
    32 x 8 Llama-3-8B KV heads."""
    from fractions import Fraction
    for n in range(0, 13):
        for ratio in (0.0, 0.1, 0.25, 1 / 3, 0.5, 0.7, 0.75, 0.9, 1.0):
            target = Fraction(ratio * n)  # the product as rounded to double
            best = min(range(n + 1), key=lambda c: (abs(Fraction(c) - target), -c))
            assert O.retrieval_count(n, ratio) == best, (n, ratio)
    assert O.retrieval_count(32 * 32, 0.25) == 256
    assert O.retrieval_count(32 * 8, 0.5) == 128


def _gates(rng, L, H, levels):
    return rng.integers(0, levels, size=(L, H)) / float(levels)  # exact, with ties


def pin_binarize_bruteforce():
    """Among all head subsets of the retrieval count, the chosen set has the largest gate sum
    and, among those, the lexicographically first (layer, head) list: the stated tie-break."""
    import itertools
    rng = np.random.default_rng(31)
    for (L, H) in [(1, 4), (2, 3), (3, 2), (2, 4)]:
        for levels in (3, 8, 1000):
            a = _gates(rng, L, H, levels)
            for ratio in (0.25, 0.5, 0.7, 1 / 3):
                mask, tau = O.binarize_gates(a, ratio)
                n = L * H
                k = O.retrieval_count(n, ratio)
                flat = a.reshape(-1)
                best = None
                for sub in itertools.combinations(range(n), k):
                    key = (-sum(flat[list(sub)]), sub)
                    if best is None or key < best:
                        best = key
                want = np.zeros(n, dtype=np.uint8)
                want[list(best[1])] = 1
                assert np.array_equal(mask.reshape(-1), want), (L, H, levels, ratio)


def pin_binarize_equation4():
    """With distinct gates the assignment is Equation 4 itself: retrieval iff alpha > tau,
    exactly the target count of heads. The result depends on the gates' order only, and a
    larger ratio keeps every head a smaller one kept."""
    rng = np.random.default_rng(32)
    for (L, H) in [(32, 32), (32, 8), (5, 7)]:
        a = rng.random((L, H))
        prev = None
        for ratio in (0.0, 0.1, 0.25, 0.5, 0.75, 1.0):
            mask, tau = O.binarize_gates(a, ratio)
            assert np.array_equal(mask, (a > tau).astype(np.uint8)), (L, H, ratio)
            assert int(mask.sum()) == O.retrieval_count(L * H, ratio)
            m2, _ = O.binarize_gates(3.0 * a ** 3 - 1.0, ratio)
            assert np.array_equal(m2, mask)
            if prev is not None:
                assert np.all(mask >= prev)
            prev = mask
    m, _ = O.binarize_gates(rng.random((32, 32)), 0.25)
    assert m.sum() == 256
    m, _ = O.binarize_gates(rng.random((32, 8)), 0.5)
    assert m.sum() == 128


def pin_head_reordering_preserves_layer():
    """Reordering Q/K/V output rows and the output projection's input columns by the head
    order leaves an attention layer's output unchanged, and puts the H_r retrieval heads
    first: projection, per-head attention with the reordered mask, output projection."""
    rng = np.random.default_rng(33)
    for (Hkv, G, mask_row) in [(4, 2, [0, 1, 0, 1]), (3, 1, [1, 0, 1]), (4, 4, [0, 0, 1, 0])]:
        d, hidden, T, S, R = 8, 24, 14, 2, 4
        Hq = Hkv * G
        x = rng.standard_normal((T, hidden))
        wq = rng.standard_normal((Hq * d, hidden))
        wk = rng.standard_normal((Hkv * d, hidden))
        wv = rng.standard_normal((Hkv * d, hidden))
        wo = rng.standard_normal((hidden, Hq * d))
        mask = np.array(mask_row, dtype=np.uint8)

        def layer(wq, wk, wv, wo, mask):
            q = (x @ wq.T).reshape(T, Hq, d)
            k = (x @ wk.T).reshape(T, Hkv, d)
            v = (x @ wv.T).reshape(T, Hkv, d)
            heads, _ = O.attention(q, k, v, np.arange(T), np.arange(T), mask, S, R)
            return heads.reshape(T, Hq * d) @ wo.T, q

        ref, q_ref = layer(wq, wk, wv, wo, mask)
        kv_order = O.head_order(mask)
        q_order = O.query_head_order(kv_order, G)
        assert sorted(kv_order.tolist()) == list(range(Hkv))
        assert sorted(q_order.tolist()) == list(range(Hq))
        mask2 = mask[kv_order]
        hr = int(mask.sum())
        assert mask2.tolist() == [1] * hr + [0] * (Hkv - hr)
        got, q_got = layer(O.reorder_output_rows(wq, q_order, d),
                           O.reorder_output_rows(wk, kv_order, d),
                           O.reorder_output_rows(wv, kv_order, d),
                           O.reorder_input_cols(wo, q_order, d), mask2)
        assert np.allclose(got, ref, rtol=0, atol=1e-9)
        assert np.array_equal(q_got, q_ref[:, q_order])
        # stable inside each class
        assert list(kv_order[:hr]) == sorted(kv_order[:hr])
        assert list(kv_order[hr:]) == sorted(kv_order[hr:])


def pin_gate_mixed_bruteforce():
    """Scalar loops over tiny inputs: per query head, two separately normalized softmax
    averages (causal keys; sink + recent keys) blended by the KV head's gate. Gate 1 is
    causal attention, gate 0 is the Lambda-masked attention of a streaming head, and while
    every query is within S + R tokens the gate does not matter."""
    rng = np.random.default_rng(41)
    T, Hkv, G, d, S, R = 11, 2, 2, 4, 2, 3
    q, k, v = rand(rng, T, Hkv * G, d), rand(rng, T, Hkv, d), rand(rng, T, Hkv, d)
    alpha = np.array([0.3, 0.85])
    pos = np.arange(T)
    out = O.gate_mixed_attention(q, k, v, pos, pos, alpha, S, R)
    for p in range(T):
        for h in range(Hkv * G):
            j = h // G
            parts = []
            for keys in (list(range(p + 1)),
                         [t for t in range(p + 1) if t < S or t >= p - R + 1]):
                z = [sum(q[p, h, c] * k[t, j, c] for c in range(d)) / math.sqrt(d) for t in keys]
                mz = max(z)
                w = [math.exp(x - mz) for x in z]
                parts.append([sum(w[i] * v[t, j, c] for i, t in enumerate(keys)) / sum(w)
                              for c in range(d)])
            want = [alpha[j] * parts[0][c] + (1 - alpha[j]) * parts[1][c] for c in range(d)]
            assert np.allclose(out[p, h], want, rtol=0, atol=1e-12), (p, h)
    full, _ = O.attention(q, k, v, pos, pos, [1, 1], S, R)
    stream, _ = O.attention(q, k, v, pos, pos, [0, 0], S, R)
    assert np.allclose(O.gate_mixed_attention(q, k, v, pos, pos, [1, 1], S, R), full, atol=1e-14)
    assert np.allclose(O.gate_mixed_attention(q, k, v, pos, pos, [0, 0], S, R), stream, atol=1e-14)
    short = np.arange(S + R)
    a = O.gate_mixed_attention(q[:S + R], k[:S + R], v[:S + R], short, short, [0.1, 0.9], S, R)
    assert np.allclose(a, _sdpa_causal(q[:S + R], np.repeat(k[:S + R], G, axis=1),
                                       np.repeat(v[:S + R], G, axis=1)), atol=1e-12)


def _bf16_grid(rng, *shape):
    """float32 values that bf16 represents exactly."""
    x = rng.standard_normal(shape).astype(np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def pin_kv4_nearest_level():
    """For 4 and 8 bits (L = 15, 255): every code is the nearest of the L + 1 stored levels
    zero + c * scale (up to float32 rounding of the quotient), found by search over all
    levels in float64; the error is at most half a step inside the levels' span, and beyond
    it no more than the bfloat16 rounding of the minimum and of the step moved the span; the
    stored scale and zero are the bfloat16 roundings of (max - min) / L and of the minimum."""
    rng = np.random.default_rng(51)
    for bits, shape, axis in ((4, (64, 16), 0), (4, (8, 128), 1), (4, (64, 3), 0),
                              (8, (128, 16), 0), (8, (8, 128), 1), (8, (300, 3), 0)):
        L = (1 << bits) - 1
        x = _bf16_grid(rng, *shape)
        codes, scale, zero = O.kv4_codes(x, axis, bits=bits)
        assert codes.max() <= L
        s = np.expand_dims(scale.astype(np.float64), axis)
        z = np.expand_dims(zero.astype(np.float64), axis)
        levels = z[..., None] + s[..., None] * np.arange(L + 1)
        dist = np.abs(x.astype(np.float64)[..., None] - levels)
        best = dist.min(axis=-1)
        got = np.take_along_axis(dist, codes[..., None].astype(np.int64), -1)[..., 0]
        assert np.all(got <= best + 1e-6 * s), shape
        mn = x.min(axis=axis, keepdims=True).astype(np.float64)
        mx = x.max(axis=axis, keepdims=True).astype(np.float64)
        slack = np.maximum(np.maximum(z - mn, 0), np.maximum(mx - (z + L * s), 0))
        assert np.all(got <= 0.5 * s * (1 + 1e-6) + slack), shape
        assert np.all(np.abs(z - mn) <= np.abs(mn) * 2.0 ** -8), shape
        assert np.all(np.abs(s - (mx - mn) / L) <= (mx - mn) / L * 2.0 ** -8 + 1e-30), shape
        # bfloat16 values: the low 16 bits of the float32 are zero
        assert not np.any(scale.view(np.uint32) & 0xFFFF) and not np.any(zero.view(np.uint32) & 0xFFFF)


def pin_kv4_axes_and_exact_grids():
    """Keys are quantized per channel (over tokens), values per token (over channels): a key
    block whose every channel is constant, or a value block whose every token is constant,
    reads back exactly; so does a block whose values lie on L + 1 evenly spaced dyadic levels
    from min to max along the quantization axis (both ends present), for 4 and 8 bits."""
    rng = np.random.default_rng(52)
    G, d = O.KV4_GROUP, 16
    for bits in (4, 8):
        L = (1 << bits) - 1
        kc = np.tile(_bf16_grid(rng, 1, d), (G, 1))          # channel-constant keys
        vc = np.tile(_bf16_grid(rng, G, 1), (1, d))          # token-constant values
        assert np.array_equal(O.kv4_history(kc, G, True, bits), kc.astype(np.float64))
        assert np.array_equal(O.kv4_history(vc, G, False, bits), vc.astype(np.float64))

        def grid_idx(m):  # m level indices in 0..L with both ends present
            return rng.permutation(np.concatenate([[0, L], rng.integers(0, L + 1, m - 2)]))
        step = 2.0 ** rng.integers(-6, 0, size=d)
        base = np.round(rng.standard_normal(d) * 8) / 8
        kidx = np.stack([grid_idx(G) for _ in range(d)], axis=1)
        kg = (base[None, :] + kidx * step[None, :]).astype(np.float32)
        assert np.array_equal(O.kv4_history(kg, G, True, bits), kg.astype(np.float64))
        vidx = np.stack([grid_idx(d) for _ in range(G)], axis=0)
        vg = (np.float32(-1.5) + vidx * 2.0 ** -6).astype(np.float32)
        assert np.array_equal(O.kv4_history(vg, G, False, bits), vg.astype(np.float64))


def pin_kv4_groups_and_residual():
    """Groups are the aligned positions g*128 .. g*128+127: a group reads back the same whatever
    the other groups hold; tokens after the last complete group (and every token of a
    sequence shorter than one group) read back exactly."""
    rng = np.random.default_rng(53)
    G = O.KV4_GROUP
    for bits in (4, 8):
        for is_key in (True, False):
            x = _bf16_grid(rng, 3 * G + 17, 8)
            h = O.kv4_history(x, x.shape[0], is_key, bits)
            assert np.array_equal(h[3 * G:], x[3 * G:].astype(np.float64))
            assert not np.array_equal(h[:3 * G], x[:3 * G].astype(np.float64))
            y = x.copy()
            y[G:2 * G] = _bf16_grid(rng, G, 8)
            hy = O.kv4_history(y, y.shape[0], is_key, bits)
            assert np.array_equal(hy[:G], h[:G]) and np.array_equal(hy[2 * G:], h[2 * G:])
            for n in (1, G - 1):
                assert np.array_equal(O.kv4_history(x, n, is_key, bits), x[:n].astype(np.float64))
            assert np.array_equal(O.kv4_history(x, 2 * G, is_key, bits)[:G], h[:G])
        # 8 bits read back closer than 4 on general data
        x = _bf16_grid(rng, 2 * G, 8)
        e4 = np.abs(O.kv4_history(x, 2 * G, True, 4) - x).max()
        e8 = np.abs(O.kv4_history(x, 2 * G, True, 8) - x).max()
        assert e8 < e4 / 8


def pin_kv4_decode():
    """Quantization touches retrieval heads only, and a history on the exact grids decodes
    exactly as the unquantized one; on general data the output moves by no more than the
    quantization error allows."""
    rng = np.random.default_rng(54)
    G = O.KV4_GROUP
    n, Hkv, Gq, d, S, R = 2 * G + 5, 2, 2, 16, 2, 8
    q = _bf16_grid(rng, Hkv * Gq, d)
    k = _bf16_grid(rng, n, Hkv, d)
    v = _bf16_grid(rng, n, Hkv, d)
    for bits, bound in ((4, 0.5), (8, 0.05)):
        a, _ = O.decode_step(q, k, v, [0, 0], S, R)
        b, _ = O.decode_step_kv4(q, k, v, [0, 0], S, R, bits=bits)
        assert np.array_equal(a, b)
        a, _ = O.decode_step(q, k, v, [1, 0], S, R)
        b, _ = O.decode_step_kv4(q, k, v, [1, 0], S, R, bits=bits)
        assert np.array_equal(a[Gq:], b[Gq:]) and 0 < np.abs(a[:Gq] - b[:Gq]).max() < bound
        # channel-constant keys and token-constant values are exact
        k2 = np.repeat(_bf16_grid(rng, 1, Hkv, d), n, axis=0)
        v2 = np.repeat(_bf16_grid(rng, n, Hkv, 1), d, axis=2)
        a, _ = O.decode_step(q, k2, v2, [1, 1], S, R)
        b, _ = O.decode_step_kv4(q, k2, v2, [1, 1], S, R, bits=bits)
        assert np.allclose(a, b, rtol=0, atol=1e-12)


def pin_kv4_prefill():
    """Prefill over a quantized cache: with no earlier tokens it is plain prefill; the bf16
    read-back of the groups is the bf16 rounding of the exact dequantized values (within half
    a bf16 step) and exact on the dyadic grids; a chunk that starts on a group boundary and
    completes no group ends near the decode step of its last token (whose cache holds the same
    groups, read back exactly); quantization touches retrieval heads only; a brute-force first
    row; nothing is quantized when no group is complete before the chunk."""
    rng = np.random.default_rng(55)
    G = O.KV4_GROUP
    Hkv, Gq, d, S, R = 2, 2, 16, 2, 8
    for bits in (4, 8):
        m = 40
        k = _bf16_grid(rng, 2 * G + m, Hkv, d)
        v = _bf16_grid(rng, 2 * G + m, Hkv, d)
        q = _bf16_grid(rng, m, Hkv * Gq, d)
        a, la = O.prefill_chunk(q, k, v, 0, [1, 0], S, R)
        b, lb = O.prefill_chunk_kv4(q, k, v, 0, [1, 0], S, R, bits=bits)
        assert np.array_equal(a, b) and np.array_equal(la, lb)
        start = 2 * G
        for is_key in (True, False):
            xx = (k if is_key else v)[:, 1]
            ex = O.kv4_history(xx, start, is_key, bits)
            hb = O.kv4_history_bf16(xx, start, is_key, bits)
            assert np.all(np.abs(hb - ex) <= 2.0 ** -8 * np.abs(ex) * (1 + 2.0 ** -20) + 1e-30)
            assert not np.any(hb.astype(np.float32).view(np.uint32) & 0xFFFF)
        kg = np.tile((np.float32(-1.5) + rng.integers(0, 16, (1, 1, d)) * 2.0 ** -4)
                     .astype(np.float32), (start, 1, 1))
        assert np.array_equal(O.kv4_history_bf16(kg[:, 0], start, True, bits),
                              kg[:, 0].astype(np.float64))
        c, lc = O.prefill_chunk_kv4(q, k, v, start, [1, 0], S, R, bits=bits)
        e, le = O.decode_step_kv4(q[-1], k, v, [1, 0], S, R, bits=bits)
        assert np.allclose(c[-1], e, rtol=0, atol=2e-2) and np.allclose(lc[-1], le, atol=2e-2)
        f, lf = O.prefill_chunk(q, k, v, start, [1, 0], S, R)
        assert np.array_equal(c[:, Gq:], f[:, Gq:])       # the streaming head: exact
        assert np.abs(c[:, :Gq] - f[:, :Gq]).max() > 0     # the retrieval head: quantized
        # the first query sees the quantized groups and itself only: brute force
        cs = [O.kv4_codes(k[g0:g0 + G, 0], 0, bits) for g0 in (0, G)]
        kd = np.concatenate([O.to_bf16(c_.astype(np.float32) * s_ + z_) for c_, s_, z_ in cs])
        cs = [O.kv4_codes(v[g0:g0 + G, 0], 1, bits) for g0 in (0, G)]
        vd = np.concatenate([O.to_bf16(c_.astype(np.float32) * s_[:, None] + z_[:, None])
                             for c_, s_, z_ in cs])
        kq = np.concatenate([kd.astype(np.float64), k[start:start + 1, 0]])
        vq = np.concatenate([vd.astype(np.float64), v[start:start + 1, 0]])
        z = kq @ q[0, 0].astype(np.float64) / math.sqrt(d)
        p_ = np.exp(z - z.max())
        assert np.allclose(c[0, 0], p_ @ vq / p_.sum(), rtol=0, atol=1e-12)
        # a chunk at 100 that completes group 0: the cache before it holds no complete group,
        # so nothing is quantized (the chunk's tokens are exact even where they complete it)
        g, lg = O.prefill_chunk_kv4(q, k, v, 100, [1, 0], S, R, bits=bits)
        h, lh = O.prefill_chunk(q, k, v, 100, [1, 0], S, R)
        assert np.array_equal(g, h) and np.array_equal(lg, lh)


def pin_kv4_prefill_rope():
    """Prefill over a pre-RoPE quantized cache (keys appended before RoPE, queries after it):
    every chunk query ends within the bound that the bf16 reading of its keys and values allows
    of the decode step at its position, which turns every key exactly and reads the dequantized
    keys and values unrounded. The chunk starts after the last complete group and completes
    none, so both read the same groups. Per key element the two differ by at most half a bf16
    step (2^-8 relative) plus a float32 rounding; a logit then moves by at most
    delta = sigma (2^-8 + 2^-22) sum_i |q_i| |k_i|, the weights by a factor within
    exp(+-2 delta), the output by (exp(2 delta) - 1) max_t |v_t - o| plus the values' own
    2^-8 max |v|, and the log-sum-exp by delta. Each query is the turned key of one visible
    token (a dequantized earlier token, a chunk token, a sink or a window slot), so its weight
    dominates only where that key is turned at its own position: without RoPE, or with the
    earlier tokens unturned, the outputs leave the bound."""
    rng = np.random.default_rng(57)
    G = O.KV4_GROUP
    Hkv, Gq, d, S, R, theta, amp = 2, 2, 16, 2, 8, 10000.0, 2.0
    sigma = 1.0 / math.sqrt(d)
    for bits in (4, 8):
        start, m = 2 * G + 8, 24
        k = _bf16_grid(rng, start + m, Hkv, d)
        v = _bf16_grid(rng, start + m, Hkv, d)
        ret = [1, 0]
        # the keys as the decode step reads them, turned
        kk = np.asarray(k, dtype=np.float64).copy()
        vv = np.asarray(v, dtype=np.float64).copy()
        kk[:, 0] = O.kv4_history(k[:, 0], start + m, True, bits)
        vv[:, 0] = O.kv4_history(v[:, 0], start + m, False, bits)
        kk = O.rope(kk, np.arange(start + m), theta)
        q = np.zeros((m, Hkv * Gq, d))
        for i in range(m):
            p = start + i
            for h in range(Hkv * Gq):
                j = h // Gq
                if ret[j]:  # an earlier (quantized or residual) token, or one of the chunk
                    t = int(rng.integers(0, start)) if h % 2 == 0 else int(rng.integers(start, p + 1))
                else:       # a sink, or a slot of the window
                    t = int(rng.integers(0, S)) if h % 2 == 0 else int(rng.integers(p - R + 1, p + 1))
                q[i, h] = O.to_bf16(amp * kk[t, j])
        c, lc = O.prefill_chunk_kv4(q, k, v, start, ret, S, R, bits=bits, rope_theta=theta)
        plain, _ = O.prefill_chunk_kv4(q, k, v, start, ret, S, R, bits=bits)
        outside = 0
        for i in range(m):
            p = start + i
            e, le = O.decode_step_kv4(q[i], k[:p + 1], v[:p + 1], ret, S, R, bits=bits,
                                      rope_theta=theta)
            for h in range(Hkv * Gq):
                j = h // Gq
                vis = O.visible_mask([p], np.arange(p + 1), bool(ret[j]), S, R)[0]
                kv, vv_ = kk[:p + 1][vis, j], vv[:p + 1][vis, j]
                delta = sigma * (2.0 ** -8 + 2.0 ** -22) * (np.abs(kv) @ np.abs(q[i, h])).max()
                spread = np.abs(vv_ - e[h][None, :]).max(axis=0)
                bound = (math.expm1(2 * delta) * spread + 2.0 ** -8 * np.abs(vv_).max(axis=0)
                         + 1e-12)
                assert np.all(np.abs(c[i, h] - e[h]) <= bound), (bits, i, h)
                assert abs(lc[i, h] - le[h]) <= delta + 1e-12
                outside += int(np.any(np.abs(plain[i, h] - e[h]) > bound))
        assert outside > m  # without RoPE most rows leave the bound


def pin_rope_complex_form():
    """RoPE equals multiplying the complex channels z_i = x_i + i x_{i+d/2} by
    exp(i t theta^(-2i/d)), written here with complex arithmetic and the exponent as
    exp(-(2i/d) ln theta); it keeps norms and is the identity at position 0."""
    rng = np.random.default_rng(61)
    for d, theta in ((8, 10000.0), (16, 500000.0), (128, 500000.0)):
        n = 9
        x = rng.standard_normal((n, 3, d))
        pos = np.array([0, 1, 2, 7, 100, 4097, 131071, 1 << 20, 3 * (1 << 19) + 5])
        h = d // 2
        w = np.exp(-(2.0 * np.arange(h) / d) * math.log(theta))
        z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * pos[:, None, None] * w[None, None, :])
        want = np.concatenate([z.real, z.imag], axis=-1)
        got = O.rope(x, pos, theta)
        assert np.allclose(got, want, rtol=0, atol=1e-9)
        assert np.allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-9)
        assert np.array_equal(O.rope(x[:1], [0], theta), x[:1])


def pin_rope_relative_positions():
    """A rotated query and key score depends on the positions only through their difference."""
    rng = np.random.default_rng(62)
    d, theta = 32, 10000.0
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((1, d))
    for s_, t, u in ((3, 11, 5), (0, 0, 12345), (700, 20, 1 << 16)):
        a = O.rope(q, [s_], theta) @ O.rope(k, [t], theta).T
        b = O.rope(q, [s_ + u], theta) @ O.rope(k, [t + u], theta).T
        assert abs(a[0, 0] - b[0, 0]) < 1e-9
    assert not np.allclose(O.rope(k, [5], theta), k)


def pin_kv4_rope_decode():
    """With pre-RoPE keys, keys that are exact in 4 bits (constant over each group's tokens,
    per channel) decode as plain attention over keys rotated at their positions by the
    complex form, the quantized and the residual tokens alike; streaming heads rotate their
    exact keys the same way, and the rotation changes the result."""
    rng = np.random.default_rng(63)
    G = O.KV4_GROUP
    n, Hkv, Gq, d, S, R, theta = 2 * G + 7, 2, 2, 16, 2, 8, 10000.0
    q = _bf16_grid(rng, Hkv * Gq, d)
    base = _bf16_grid(rng, 3, Hkv, d)
    k = np.concatenate([np.repeat(base[0:1], G, 0), np.repeat(base[1:2], G, 0),
                        np.repeat(base[2:3], n - 2 * G, 0)]) + 0.0
    k[2 * G:] = _bf16_grid(rng, n - 2 * G, Hkv, d)  # the residual tokens need not be constant
    v = np.repeat(_bf16_grid(rng, n, Hkv, 1), d, axis=2)
    h = d // 2
    w = np.exp(-(2.0 * np.arange(h) / d) * math.log(theta))
    z = (k[..., :h] + 1j * k[..., h:]) * np.exp(1j * np.arange(n)[:, None, None] * w)
    krot = np.concatenate([z.real, z.imag], axis=-1)
    for mask in ([1, 0], [1, 1], [0, 1]):
        a, _ = O.decode_step(q, krot, v, mask, S, R)
        b, _ = O.decode_step_kv4(q, k, v, mask, S, R, rope_theta=theta)
        assert np.allclose(a, b, rtol=0, atol=1e-9), mask
        c, _ = O.decode_step_kv4(q, k, v, mask, S, R)
        assert np.abs(b - c).max() > 1e-3


PINS = [pin_cache_policy, pin_streaming_rows, pin_decode_scalar_bruteforce,
        pin_all_retrieval_is_causal_attention, pin_short_streaming_is_full,
        pin_no_sink_is_sliding_window, pin_fig5_worked_example, pin_memory_numbers,
        pin_memory_formula_by_count, pin_chunk_invariance_and_decode_equivalence,
        pin_head_permutation, pin_gqa_equals_repeated_mha, pin_lambda_mask_literal,
        pin_chunk_granular_fig5, pin_chunk_granular_gather, pin_chunk_granular_short_is_full,
        pin_retrieval_count_nearest, pin_binarize_bruteforce, pin_binarize_equation4,
        pin_head_reordering_preserves_layer, pin_gate_mixed_bruteforce, pin_kv4_nearest_level,
        pin_kv4_axes_and_exact_grids, pin_kv4_groups_and_residual, pin_kv4_decode,
        pin_kv4_prefill, pin_kv4_prefill_rope,
        pin_rope_complex_form, pin_rope_relative_positions, pin_kv4_rope_decode]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# --------------------------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail
# --------------------------------------------------------------------------------------------

def _window_too_wide(q_pos, k_pos, retrieval, sink, recent):
    p = np.asarray(q_pos)[:, None]
    t = np.asarray(k_pos)[None, :]
    c = t <= p
    return c if retrieval else c & ((t < sink) | (t >= p - recent))


def _window_excludes_self_slot(q_pos, k_pos, retrieval, sink, recent):
    p = np.asarray(q_pos)[:, None]
    t = np.asarray(k_pos)[None, :]
    c = t <= p
    return c if retrieval else c & ((t < sink) | (t >= p - recent + 2))


def _sink_off_by_one(q_pos, k_pos, retrieval, sink, recent):
    p = np.asarray(q_pos)[:, None]
    t = np.asarray(k_pos)[None, :]
    c = t <= p
    return c if retrieval else c & ((t <= sink) | (t >= p - recent + 1))


def _streaming_not_causal(q_pos, k_pos, retrieval, sink, recent):
    p = np.asarray(q_pos)[:, None]
    t = np.asarray(k_pos)[None, :]
    return (t <= p) if retrieval else ((t < sink) | (t >= p - recent + 1))


def _lse_log2(q, k, v, mask, scale):
    out, lse = _ORIG_MSA(q, k, v, mask, scale)
    return out, lse / math.log(2)


def _softmax_unmasked_den(q, k, v, mask, scale):
    z = scale * (np.asarray(q) @ np.asarray(k).T)
    zm = np.where(mask, z, -np.inf)
    m = zm.max(axis=1, keepdims=True)
    w = np.exp(zm - m)
    den = np.exp(z - m).sum(axis=1, keepdims=True)  # denominator over all keys
    return (w @ np.asarray(v)) / den, (m + np.log(den))[:, 0]


def _chunk_held_one_short(q_pos, k_pos, start, retrieval, sink, recent):
    p = np.asarray(q_pos)[:, None]
    t = np.asarray(k_pos)[None, :]
    if retrieval:
        return (t <= p) & (t >= 0)
    held = (t >= 0) & (t < start) & ((t < sink) | (t >= start - recent + 1))
    return held | ((t >= start) & (t <= p))


def _binarize_ties_high_first(alpha, ratio):
    a = np.asarray(alpha, dtype=np.float64)
    L, H = a.shape
    k = O.retrieval_count(L * H, ratio)
    ranking = sorted(((i, j) for i in range(L) for j in range(H)), key=lambda lh: (-a[lh], -lh[0], -lh[1]))
    mask = np.zeros((L, H), dtype=np.uint8)
    for lh in ranking[:k]:
        mask[lh] = 1
    return mask, float(a[ranking[k]]) if k < L * H else -math.inf


def _binarize_tau_last_kept(alpha, ratio):
    mask, _ = _ORIG_BIN(alpha, ratio)
    a = np.asarray(alpha, dtype=np.float64)
    return mask, float(a[mask == 1].min()) if mask.any() else float(a.max())


def _binarize_per_layer(alpha, ratio):
    a = np.asarray(alpha, dtype=np.float64)
    rows = [_ORIG_BIN(a[i:i + 1], ratio) for i in range(a.shape[0])]
    return np.concatenate([r[0] for r in rows]), min(r[1] for r in rows)


def _mixed_unnormalized(q, k, v, q_pos, k_pos, alpha, sink, recent, scale=None):
    """Blends the unnormalized sums and normalizes once (a plausible fused-kernel mistake)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    P, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = 1 / math.sqrt(d) if scale is None else scale
    out = np.empty((P, Hq, d))
    for h in range(Hq):
        j = h // G
        z = sc * (q[:, h] @ k[:, j].T)
        num, den = 0, 0
        for r, wgt in ((True, alpha[j]), (False, 1 - alpha[j])):
            m = O.visible_mask(q_pos, k_pos, r, sink, recent)
            e = np.where(m, np.exp(z - z.max(axis=1, keepdims=True)), 0)
            num = num + wgt * (e @ v[:, j])
            den = den + wgt * e.sum(axis=1, keepdims=True)
        out[:, h] = num / den
    return out


def _kv4_codes_variant(floor=False, extra_level=False, ignore_bits=False):
    def f(x, axis, bits=4):
        L = 15 if ignore_bits else (1 << bits) - 1
        x = np.asarray(x, dtype=np.float32)
        mn = x.min(axis=axis, keepdims=True)
        mx = x.max(axis=axis, keepdims=True)
        scale = (mx - mn) / np.float32(L + 1 if extra_level else L)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = (x - mn) / scale
            c = np.floor(r) if floor else np.rint(r)
        c = np.where(scale == 0, np.float32(0.0), c)
        return np.clip(c, 0, L).astype(np.uint8), np.squeeze(scale, axis), np.squeeze(mn, axis)
    return f


def _kv4_history_variant(swap_axes=False, quantize_tail=False, misaligned=False):
    def f(x_hist, n, is_key, bits=4):
        x = np.asarray(x_hist, dtype=np.float32)[:n]
        out = x.astype(np.float64).copy()
        G = O.KV4_GROUP
        starts = list(range(0, (n // G) * G, G))
        if misaligned:
            starts = list(range(n % G, n - G + 1, G))
        if quantize_tail and n % G:
            starts.append((n // G) * G)
        for g0 in starts:
            blk = x[g0:g0 + G]
            per_channel = is_key != swap_axes
            codes, scale, zero = O.kv4_codes(blk, axis=0 if per_channel else 1, bits=bits)
            if per_channel:
                out[g0:g0 + len(blk)] = codes * scale.astype(np.float64)[None] + zero[None]
            else:
                out[g0:g0 + len(blk)] = codes * scale.astype(np.float64)[:, None] + zero[:, None]
        return out
    return f


def _rope_variant(interleaved=False, sign=1.0, exponent=2.0, offset=0):
    def f(x, pos, theta):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        h = d // 2
        inv = np.power(float(theta), -exponent * np.arange(h) / d)
        a = sign * (np.asarray(pos, dtype=np.float64) + offset)[:, None] * inv[None, :]
        shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (h,)
        c, s_ = np.cos(a).reshape(shape), np.sin(a).reshape(shape)
        if interleaved:
            x1, x2 = x[..., 0::2], x[..., 1::2]
            out = np.empty_like(x)
            out[..., 0::2] = x1 * c - x2 * s_
            out[..., 1::2] = x1 * s_ + x2 * c
            return out
        x1, x2 = x[..., :h], x[..., h:]
        return np.concatenate([x1 * c - x2 * s_, x1 * s_ + x2 * c], axis=-1)
    return f


def _kv4_rope_before_quant(q, k_hist, v_hist, retrieval, sink, recent, scale=None,
                           rope_theta=None, bits=4):
    k = np.asarray(k_hist, dtype=np.float64)
    if rope_theta:
        k = O.rope(k, np.arange(k.shape[0]), rope_theta).astype(np.float32)
    return _ORIG_KV4(q, k, v_hist, retrieval, sink, recent, scale, bits=bits)


def _kv4_prefill_quantizes_chunk(q, k_hist, v_hist, start, retrieval, sink, recent, scale=None,
                                 chunk_granular=False, bits=4, rope_theta=None):
    if rope_theta:
        return _ORIG_PF4(q, k_hist, v_hist, start, retrieval, sink, recent, scale,
                         chunk_granular, bits, rope_theta)
    m = np.asarray(q).shape[0]
    k = np.asarray(k_hist, dtype=np.float64).copy()
    v = np.asarray(v_hist, dtype=np.float64).copy()
    for j in range(k.shape[1]):
        if retrieval[j]:
            k[:start + m, j] = O.kv4_history_bf16(k_hist[:, j], start + m, True, bits)
            v[:start + m, j] = O.kv4_history_bf16(v_hist[:, j], start + m, False, bits)
    return O.prefill_chunk(q, k, v, start, retrieval, sink, recent, scale, chunk_granular)



def _kv4_prefill_rope_variant(prefix_unturned=False, chunk_from_zero=False):
    """prefill_chunk_kv4 with pre-RoPE keys, planted mistakes: the dequantized prefix keys left
    unturned, or the chunk's own keys turned at their offsets in the chunk."""
    def f(q, k_hist, v_hist, start, retrieval, sink, recent, scale=None, chunk_granular=False,
          bits=4, rope_theta=None):
        if not rope_theta:
            return _ORIG_PF4(q, k_hist, v_hist, start, retrieval, sink, recent, scale,
                             chunk_granular, bits)
        k = np.asarray(k_hist, dtype=np.float64).copy()
        v = np.asarray(v_hist, dtype=np.float64).copy()
        pos = np.arange(k.shape[0])
        if chunk_from_zero:
            pos = np.where(pos >= start, pos - start, pos)
        k = O.to_bf16(O.rope(k, pos, rope_theta)).astype(np.float64)
        for j in range(k.shape[1]):
            if retrieval[j] and start > 0:
                kd = O.kv4_history_f32(k_hist[:, j], start, True, bits)
                k[:start, j] = (O.to_bf16(kd) if prefix_unturned else
                                O.to_bf16(O.rope(kd, np.arange(start), rope_theta)))
                v[:start, j] = O.kv4_history_bf16(v_hist[:, j], start, False, bits)
        return O.prefill_chunk(q, k, v, start, retrieval, sink, recent, scale, chunk_granular)
    return f


_ORIG_KV4 = O.decode_step_kv4
_ORIG_PF4 = O.prefill_chunk_kv4
_ORIG_MSA = O.masked_softmax_attention
_ORIG_BIN = O.binarize_gates
_ORIG_MIX = O.gate_mixed_attention

MUTANTS = {
    "window_too_wide": ("visible_mask", _window_too_wide),
    "window_too_narrow": ("visible_mask", _window_excludes_self_slot),
    "sink_off_by_one": ("visible_mask", _sink_off_by_one),
    "streaming_not_causal": ("visible_mask", _streaming_not_causal),
    "interleaved_groups": ("kv_head_of", lambda h, G: h % G),
    "no_scale": ("default_scale", lambda d: 1.0),
    "lse_base2": ("masked_softmax_attention", _lse_log2),
    "den_over_unmasked": ("masked_softmax_attention", _softmax_unmasked_den),
    "ring_from_zero": ("slot_of", lambda t, S, R: t if t < S else (t - S) % R),
    "ring_wrong_modulus": ("slot_of", lambda t, S, R: t if t < S else S + (t - S) % max(1, R - 1)),
    "recent_one_short": ("streaming_valid_tokens",
                         lambda n, S, R: np.concatenate([np.arange(min(S, n)),
                                                         np.arange(max(S, n - R + 1), n)])),
    "memory_no_min": ("duo_kv_elements_layer",
                      lambda Hr, Hs, L, S, R, d: (Hr * L + Hs * (S + R)) * d),
    "budget_weights_r": ("budget_ratio", lambda r, L, S, R: (r * L + r * min(L, S + R)) / L),
    "full_kv_no_factor2": ("full_kv_elements", lambda D, H, L, d: D * H * L * d),
    "chunk_held_one_short": ("chunk_visible_mask", _chunk_held_one_short),
    "chunk_window_per_query": ("chunk_visible_mask",
                               lambda q, k, st, r, S, R: O.visible_mask(q, k, r, S, R)),
    "count_floor": ("retrieval_count", lambda n, r: int(math.floor(r * n))),
    "binarize_ties_high_first": ("binarize_gates", _binarize_ties_high_first),
    "binarize_tau_last_kept": ("binarize_gates", _binarize_tau_last_kept),
    "binarize_per_layer": ("binarize_gates", _binarize_per_layer),
    "head_order_streaming_first": ("head_order",
                                   lambda m: np.argsort(np.asarray(m) != 0, kind="stable")),
    "kv4_floor": ("kv4_codes", _kv4_codes_variant(floor=True)),
    "kv4_sixteen_steps": ("kv4_codes", _kv4_codes_variant(extra_level=True)),
    "kv8_levels_of_4_bits": ("kv4_codes", _kv4_codes_variant(ignore_bits=True)),
    "kv4_axes_swapped": ("kv4_history", _kv4_history_variant(swap_axes=True)),
    "kv4_tail_quantized": ("kv4_history", _kv4_history_variant(quantize_tail=True)),
    "kv4_groups_misaligned": ("kv4_history", _kv4_history_variant(misaligned=True)),
    "mixed_alpha_swapped": ("gate_mixed_attention",
                            lambda q, k, v, qp, kp, a, S, R, scale=None: _ORIG_MIX(
                                q, k, v, qp, kp, 1 - np.asarray(a), S, R, scale)),
    "mixed_unnormalized_blend": ("gate_mixed_attention", _mixed_unnormalized),
    "rope_interleaved_pairs": ("rope", _rope_variant(interleaved=True)),
    "rope_negative_angle": ("rope", _rope_variant(sign=-1.0)),
    "rope_exponent_halved": ("rope", _rope_variant(exponent=1.0)),
    "rope_position_plus_one": ("rope", _rope_variant(offset=1)),
    "kv4_rope_before_quantization": ("decode_step_kv4", _kv4_rope_before_quant),
    "kv4_prefill_quantizes_the_chunk": ("prefill_chunk_kv4", _kv4_prefill_quantizes_chunk),
    "kv4_prefill_rope_prefix_unturned": ("prefill_chunk_kv4",
                                         _kv4_prefill_rope_variant(prefix_unturned=True)),
    "kv4_prefill_rope_chunk_from_zero": ("prefill_chunk_kv4",
                                         _kv4_prefill_rope_variant(chunk_from_zero=True)),
    "query_order_interleaved": ("query_head_order",
                                lambda o, G: np.array([g * len(o) + j for j in o for g in range(G)])),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    np.seterr(all="ignore")
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
