"""The C ABI on the host (CPU only): exports, configuration checks, arena layout, the KV
byte model against the oracle, and the error paths that return before any launch.

These tests never make a call that passes validation with device work to do: every call
that could launch is given an argument that must be rejected first, so they are safe with
or without a GPU.
"""
import ctypes
import os
import re

import numpy as np
import torch
import pytest

from oracle import duo_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

hsk = pytest.importorskip("head_split_kv_amd")
from head_split_kv_amd import _native as N  # noqa: E402

if not os.path.exists(N.LIB_PATH):
    pytest.skip("libduo.so not built", allow_module_level=True)


def declared_symbols():
    with open(os.path.join(ROOT, "include", "duo.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^(?:duo_status|const char\*)\s+(duo_\w+)\(", text, re.M)))


def cfg_of(**kw):
    base = dict(num_layers=2, batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, sink=4,
                recent=16, capacity=1000, retrieval_mask=[[1, 0], [0, 1]])
    base.update(kw)
    return hsk.make_config(**base)


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 12
    assert sorted(N.EXPORTS) == names
    L = N.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(5):
        assert N.status_string(s).startswith(("DUO_OK", "DUO_ERR_"))


@pytest.mark.parametrize("bad,status", [
    (dict(recent=0), N.DUO_ERR_INVALID),
    (dict(sink=-1), N.DUO_ERR_INVALID),
    (dict(batch=0), N.DUO_ERR_INVALID),
    (dict(batch=513), N.DUO_ERR_INVALID),
    (dict(num_q_heads=6, num_kv_heads=4, retrieval_mask=[[1, 0, 0, 0], [0, 1, 0, 0]]),
     N.DUO_ERR_INVALID),
    (dict(capacity=0), N.DUO_ERR_INVALID),
    (dict(head_dim=96), N.DUO_ERR_UNSUPPORTED),
    (dict(num_q_heads=6, num_kv_heads=2), N.DUO_ERR_UNSUPPORTED),
    (dict(num_q_heads=32, num_kv_heads=2), N.DUO_ERR_UNSUPPORTED),
])
def test_config_checks(bad, status):
    import torch
    kw = dict(bad)
    cfg, _ = cfg_of(**kw)
    lay = N.DuoLayout()
    assert N.lib().duo_layout_query(ctypes.byref(cfg), ctypes.byref(lay)) == status
    # out dtype must be fp32 or the input dtype
    cfg2, _ = cfg_of(dtype=torch.float32, out_dtype=torch.bfloat16)
    assert N.lib().duo_layout_query(ctypes.byref(cfg2), ctypes.byref(lay)) == N.DUO_ERR_UNSUPPORTED


def test_kv_bits_checked_and_kv4_layout():
    import torch
    lay = N.DuoLayout()
    for bits, status in ((0, N.DUO_OK), (16, N.DUO_OK), (4, N.DUO_OK), (8, N.DUO_OK),
                         (2, N.DUO_ERR_INVALID), (-4, N.DUO_ERR_INVALID)):
        cfg, _keep = cfg_of()
        cfg.kv_bits = bits
        assert N.lib().duo_layout_query(ctypes.byref(cfg), ctypes.byref(lay)) == status, bits
    for bits in (4, 8):
        cfg, _keep = cfg_of(dtype=torch.float32, kv_bits=bits)
        assert N.lib().duo_layout_query(ctypes.byref(cfg), ctypes.byref(lay)) == N.DUO_ERR_UNSUPPORTED
    # a 4-bit retrieval head needs a partial for its residual rows besides its context splits
    for ms, status in ((1, N.DUO_ERR_INVALID), (2, N.DUO_OK), (0, N.DUO_OK)):
        cfg, _keep = cfg_of(kv_bits=4, max_splits=ms)
        assert N.lib().duo_layout_query(ctypes.byref(cfg), ctypes.byref(lay)) == status, ms
    # the 4-bit full caches are sized by the documented per-head geometry
    cfg4, _k4 = cfg_of(kv_bits=4)
    cfg16, _k16 = cfg_of()
    l4, l16 = N.DuoLayout(), N.DuoLayout()
    assert N.lib().duo_layout_query(ctypes.byref(cfg4), ctypes.byref(l4)) == N.DUO_OK
    assert N.lib().duo_layout_query(ctypes.byref(cfg16), ctypes.byref(l16)) == N.DUO_OK
    cap, D, G = 1000, 128, N.KV4_GROUP
    groups = -(-cap // G)
    stride = groups * G * D // 2 + max(groups * 2 * D * 2, groups * G * 4) + G * D * 2
    per_layer = [3 * 1 * stride, 3 * 1 * stride]  # batch 3, one retrieval head per layer
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert l4.full_v_off - l4.full_k_off == al(sum(al(x) for x in per_layer))
    assert l4.arena_bytes < l16.arena_bytes
    # 8 bits: twice the code bytes, the same parameter block and residual
    cfg8, _k8 = cfg_of(kv_bits=8)
    l8 = N.DuoLayout()
    assert N.lib().duo_layout_query(ctypes.byref(cfg8), ctypes.byref(l8)) == N.DUO_OK
    stride8 = groups * G * D + max(groups * 2 * D * 2, groups * G * 4) + G * D * 2
    assert l8.full_v_off - l8.full_k_off == al(2 * al(3 * stride8))
    assert l4.arena_bytes < l8.arena_bytes < l16.arena_bytes


def test_rope_theta_checked_and_rope_layout():
    """Pre-RoPE keys are built for 4-bit caches only; their cos/sin tables follow the
    workspace: tau16 [128][d/2 + 4] words and the base rows [cap / 128 + 1] of (cos, sin)
    float pairs per channel pair, each 256-byte aligned."""
    lay = N.DuoLayout()
    for bits, theta, status in ((4, 10000.0, N.DUO_OK), (4, 0.0, N.DUO_OK), (4, -1.0, N.DUO_OK),
                                (8, 10000.0, N.DUO_OK),
                                (0, 10000.0, N.DUO_ERR_UNSUPPORTED),
                                (16, 500000.0, N.DUO_ERR_UNSUPPORTED),
                                (4, float("nan"), N.DUO_ERR_INVALID),
                                (4, float("inf"), N.DUO_ERR_INVALID)):
        cfg, _keep = cfg_of(kv_bits=bits)
        cfg.rope_theta = theta
        assert N.lib().duo_layout_query(ctypes.byref(cfg), ctypes.byref(lay)) == status, (bits, theta)
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for D, cap in ((128, 1000), (64, 1024), (128, 131072 + 5)):
        cfg, _keep = cfg_of(kv_bits=4, head_dim=D, capacity=cap, rope_theta=500000.0)
        plain, _k2 = cfg_of(kv_bits=4, head_dim=D, capacity=cap)
        lr, lp = N.DuoLayout(), N.DuoLayout()
        assert N.lib().duo_layout_query(ctypes.byref(cfg), ctypes.byref(lr)) == N.DUO_OK
        assert N.lib().duo_layout_query(ctypes.byref(plain), ctypes.byref(lp)) == N.DUO_OK
        assert lp.rope_bytes == 0 and lp.rope_off == 0
        want = al(128 * (D // 2 + 4) * 4) + al((cap // 128 + 1) * D * 4)
        assert lr.rope_bytes == want, D
        assert lr.rope_off == al(lr.workspace_off + lr.workspace_bytes)
        assert lr.arena_bytes == al(lr.rope_off + lr.rope_bytes)
        assert lr.arena_bytes == lp.arena_bytes + al(want)


@pytest.mark.parametrize("bits", [4, 8])
def test_kv4_bytes_model(bits):
    """Per retrieval head: d bits / 4 bytes of K and V codes per grouped token, 4 d bytes of
    key parameters per group, 4 bytes of value parameters per grouped token, residual tokens
    at 4 d bytes (bf16 K and V); streaming heads unchanged."""
    cfg, _keep = cfg_of(kv_bits=bits)
    full, duo = ctypes.c_uint64(), ctypes.c_uint64()
    D, G, S, R = 128, N.KV4_GROUP, 4, 16
    for lens in ([0, 1, 127], [128, 129, 999], [256, 500, 1000]):
        ln = np.array(lens, dtype=np.int32)
        assert N.lib().duo_kv_bytes(ctypes.byref(cfg), ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                    0, ctypes.byref(full), ctypes.byref(duo)) == N.DUO_OK
        want = 0
        for n in lens:
            g, t = n // G, (n // G) * G
            want += t * D * bits // 4 + g * 4 * D + t * 4 + (n - t) * 4 * D  # a retrieval head
            want += 2 * min(n, S + R) * D * 2                               # a streaming head
        assert duo.value == want, lens
        assert full.value == sum(2 * 2 * n * D * 2 for n in lens)


def test_streaming_prefill_mode_checked():
    lay = N.DuoLayout()
    for mode, status in ((N.PREFILL_WINDOW, N.DUO_OK), (N.PREFILL_CHUNK, N.DUO_OK),
                         (2, N.DUO_ERR_INVALID), (-1, N.DUO_ERR_INVALID)):
        cfg, _keep = cfg_of()
        cfg.streaming_prefill = mode
        assert N.lib().duo_layout_query(ctypes.byref(cfg), ctypes.byref(lay)) == status, mode
    with pytest.raises(ValueError):
        cfg_of(streaming_prefill="sliding")


def test_layout_covers_the_split_caches():
    cfg, mask = cfg_of()
    lay = hsk.duo_layout_query(cfg)
    offs = [lay.full_k_off, lay.full_v_off, lay.str_k_off, lay.str_v_off, lay.slot_pos_off,
            lay.seq_len_off, lay.workspace_off]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    es, B, D, cap, SR = 2, 3, 128, 1000, 20
    n_ret = int(mask.sum())
    n_str = mask.size - n_ret
    assert lay.full_v_off - lay.full_k_off >= B * n_ret * cap * D * es
    assert lay.str_v_off - lay.str_k_off >= B * n_str * SR * D * es
    assert lay.seq_len_off - lay.slot_pos_off >= 2 * B * SR * 4
    assert lay.arena_bytes >= lay.workspace_off + lay.workspace_bytes


@pytest.mark.parametrize("layer", [0, 1])
def test_kv_bytes_match_oracle_memory_model(layer):
    import torch
    for dtype, es in ((torch.bfloat16, 2), (torch.float32, 4)):
        cfg, mask = cfg_of(dtype=dtype, out_dtype=torch.float32)
        lens = [0, 7, 3000]
        full, duo = hsk.duo_kv_bytes(cfg, lens, layer)
        hr = int(mask[layer].sum())
        hs = 2 - hr
        want_duo = sum(2 * O.duo_kv_elements_layer(hr, hs, n, 4, 16, 128) * es for n in lens)
        want_full = sum(O.full_kv_elements(1, 2, n, 128) * es for n in lens)
        assert (full, duo) == (want_full, want_duo)


def test_kv_bytes_at_workload_shapes():
    """Full/split KV ratios of the Llama-shaped layers (128K GQA 50 %, 32K MHA 25 %)."""
    import workloads as W
    for key, ratio in (("c3", 1_048_576 / 526_400), ("c2", 1_048_576 / 274_816)):
        w = W.workload(key)
        cfg, _ = hsk.make_config(num_layers=1, batch=1, num_q_heads=w.hq, num_kv_heads=w.hkv,
                                 head_dim=w.d, sink=w.sink, recent=w.recent, capacity=w.capacity,
                                 retrieval_mask=W.retrieval_mask(w))
        full, duo = hsk.duo_kv_bytes(cfg, [w.context], 0)
        assert abs(full / duo - ratio) < 1e-9


class FakeCache:
    """A host object over a fake (never dereferenced) arena address: only calls that the
    host rejects before launching are made on it."""

    def __init__(self, **kw):
        self.cfg, self.mask = cfg_of(**kw)
        lay = hsk.duo_layout_query(self.cfg)
        self.h = ctypes.c_void_p()
        st = N.lib().duo_cache_create(ctypes.byref(self.cfg), ctypes.c_void_p(1 << 40),
                                      lay.arena_bytes, ctypes.byref(self.h))
        assert st == N.DUO_OK
        self.lay = lay

    def lengths(self):
        out = np.empty((self.cfg.num_layers, self.cfg.batch), dtype=np.int32)
        assert N.lib().duo_cache_lengths(self.h, out.ctypes.data_as(
            ctypes.POINTER(ctypes.c_int32))) == 0
        return out

    def close(self):
        N.lib().duo_cache_destroy(self.h)


def test_create_rejects_small_or_misaligned_arena():
    cfg, _ = cfg_of()
    lay = hsk.duo_layout_query(cfg)
    h = ctypes.c_void_p()
    L = N.lib()
    assert L.duo_cache_create(ctypes.byref(cfg), ctypes.c_void_p(1 << 40),
                              lay.arena_bytes - 1, ctypes.byref(h)) == N.DUO_ERR_INVALID
    assert L.duo_cache_create(ctypes.byref(cfg), ctypes.c_void_p((1 << 40) + 16),
                              lay.arena_bytes, ctypes.byref(h)) == N.DUO_ERR_INVALID
    assert L.duo_cache_create(ctypes.byref(cfg), None, lay.arena_bytes,
                              ctypes.byref(h)) == N.DUO_ERR_INVALID


def test_error_paths_leave_state_unchanged():
    fc = FakeCache()
    L = N.lib()
    p = ctypes.c_void_p(1 << 41)  # aligned, never dereferenced
    mis = ctypes.c_void_p((1 << 41) + 8)
    before = fc.lengths().copy()
    # bad layer / sequence / count
    assert L.duo_kv_append(fc.h, 2, -1, p, p, 1, None) == N.DUO_ERR_INVALID
    assert L.duo_kv_append(fc.h, -1, -1, p, p, 1, None) == N.DUO_ERR_INVALID
    assert L.duo_kv_append(fc.h, 0, 3, p, p, 1, None) == N.DUO_ERR_INVALID
    assert L.duo_kv_append(fc.h, 0, -2, p, p, 1, None) == N.DUO_ERR_INVALID
    assert L.duo_kv_append(fc.h, 0, -1, p, p, -1, None) == N.DUO_ERR_INVALID
    assert L.duo_kv_append(fc.h, 0, -1, None, p, 1, None) == N.DUO_ERR_INVALID
    assert L.duo_kv_append(fc.h, 0, -1, mis, p, 1, None) == N.DUO_ERR_INVALID
    # zero tokens is a no-op that launches nothing
    assert L.duo_kv_append(fc.h, 0, -1, p, p, 0, None) == N.DUO_OK
    # capacity: 1001 tokens into a 1000-token cache
    assert L.duo_kv_append(fc.h, 0, -1, p, p, 1001, None) == N.DUO_ERR_CAPACITY
    assert L.duo_kv_append(fc.h, 1, 1, p, p, 1001, None) == N.DUO_ERR_CAPACITY
    assert L.duo_attn_prefill(fc.h, 0, -1, p, p, p, 1001, p, None, None) == N.DUO_ERR_CAPACITY
    # decode of empty sequences is rejected
    assert L.duo_attn_decode(fc.h, 0, p, p, None, None) == N.DUO_ERR_INVALID
    assert L.duo_attn_decode(fc.h, 0, mis, p, None, None) == N.DUO_ERR_INVALID
    assert L.duo_decode_step(fc.h, 0, p, None, p, p, None, None) == N.DUO_ERR_INVALID
    assert L.duo_decode_step(fc.h, 0, p, mis, p, p, None, None) == N.DUO_ERR_INVALID
    assert L.duo_decode_step(fc.h, 5, p, p, p, p, None, None) == N.DUO_ERR_INVALID
    assert L.duo_attn_prefill(fc.h, 0, -1, p, p, p, 0, p, None, None) == N.DUO_OK
    assert L.duo_attn_prefill(fc.h, 0, 5, p, p, p, 4, p, None, None) == N.DUO_ERR_INVALID
    assert L.duo_attn_prefill(fc.h, 0, 0, p, mis, p, 4, p, None, None) == N.DUO_ERR_INVALID
    assert L.duo_slot_positions(fc.h, 9, None, None) == N.DUO_ERR_INVALID
    assert L.duo_set_decode_splits(fc.h, -1) == N.DUO_ERR_INVALID
    assert L.duo_set_decode_splits(fc.h, 257) == N.DUO_ERR_INVALID
    assert L.duo_set_decode_splits(fc.h, 7) == N.DUO_OK
    # lengths: out of range or missing -> INVALID, nothing launched
    bad = (ctypes.c_int32 * 6)(0, 1001, 0, 0, 0, 0)  # [L=2][B=3], capacity 1000
    assert L.duo_cache_set_lengths(fc.h, bad, None) == N.DUO_ERR_INVALID
    neg = (ctypes.c_int32 * 6)(0, 0, -1, 0, 0, 0)
    assert L.duo_cache_set_lengths(fc.h, neg, None) == N.DUO_ERR_INVALID
    assert L.duo_cache_set_lengths(fc.h, None, None) == N.DUO_ERR_INVALID
    assert L.duo_cache_init(None, p, 0, None, None) == N.DUO_ERR_INVALID
    # kernel timers: argument checks only (creating events needs a device)
    ms, cnt = ctypes.c_double(1.0), ctypes.c_int32(5)
    assert L.duo_timing_enable(fc.h, -1) == N.DUO_ERR_INVALID
    assert L.duo_timing_enable(fc.h, (1 << 16) + 1) == N.DUO_ERR_INVALID
    assert L.duo_timing_enable(None, 4) == N.DUO_ERR_INVALID
    assert L.duo_timing_enable(fc.h, 0) == N.DUO_OK  # off: nothing to create
    assert L.duo_timing_read(fc.h, 2, ctypes.byref(ms), ctypes.byref(cnt)) == N.DUO_ERR_INVALID
    assert L.duo_timing_read(fc.h, 0, None, ctypes.byref(cnt)) == N.DUO_ERR_INVALID
    assert L.duo_timing_read(fc.h, 1, ctypes.byref(ms), ctypes.byref(cnt)) == N.DUO_OK
    assert (ms.value, cnt.value) == (0.0, 0)
    assert np.array_equal(fc.lengths(), before)
    assert L.duo_cache_destroy(None) == N.DUO_OK
    fc.close()


def test_prefill_staged_checks_before_launch():
    """duo_prefill_staging_bytes: 0 on an fp32 cache; on bf16, 4- and 8-bit caches the fp16
    copies of the chunk's and the streaming caches' values (empty caches here, so no prefix),
    after the chunk and streaming keys with pre-RoPE keys; argument checks.
    duo_attn_prefill_staged rejects bad arguments and short staging before launching;
    duo_attn_prefill refuses every layer of a pre-RoPE cache, streaming-only layers
    included."""
    L = N.lib()
    n = ctypes.c_uint64(7)
    p = ctypes.c_void_p(1 << 40)
    row = 128 * 2
    up = lambda x: (x + 255) // 256 * 256
    fc = FakeCache(dtype=torch.float32)
    assert L.duo_prefill_staging_bytes(fc.h, 0, -1, 5, ctypes.byref(n)) == N.DUO_OK
    assert n.value == 0
    fc.close()
    for bits in (0, 4, 8):
        fc = FakeCache(kv_bits=bits)
        assert L.duo_prefill_staging_bytes(fc.h, 0, -1, 5, ctypes.byref(n)) == N.DUO_OK
        # B 3, Hkv 2 (layer 0: one streaming head), d 128, S + R = 20, empty caches: the fp16
        # values of the chunk and of the streaming caches
        assert n.value == up(3 * 5 * 2 * row) + 3 * 1 * 20 * row
        if bits == 0:
            assert L.duo_attn_prefill_staged(fc.h, 0, -1, p, p, p, 5, p, None, p,
                                             n.value - 16, None) == N.DUO_ERR_INVALID
            assert L.duo_attn_prefill_staged(fc.h, 0, -1, p, p, p, 5, p, None,
                                             ctypes.c_void_p((1 << 40) + 8), n.value,
                                             None) == N.DUO_ERR_INVALID
        assert L.duo_prefill_staging_bytes(fc.h, 2, -1, 5, ctypes.byref(n)) == N.DUO_ERR_INVALID
        assert L.duo_prefill_staging_bytes(fc.h, 0, 3, 5, ctypes.byref(n)) == N.DUO_ERR_INVALID
        assert L.duo_prefill_staging_bytes(fc.h, 0, -1, -1, ctypes.byref(n)) == N.DUO_ERR_INVALID
        assert L.duo_prefill_staging_bytes(fc.h, 0, -1, 5, None) == N.DUO_ERR_INVALID
        assert L.duo_attn_prefill_staged(fc.h, 0, -2, p, p, p, 4, p, None, p, 0,
                                         None) == N.DUO_ERR_INVALID
        assert L.duo_attn_prefill_staged(fc.h, 0, -1, p, p, p, -1, p, None, p, 0,
                                         None) == N.DUO_ERR_INVALID
        fc.close()
    # pre-RoPE keys: B 3, Hkv 2 (layer 0: one retrieval, one streaming head; layer 1: two
    # streaming heads), d 128, S + R = 20, empty caches: the chunk's keys, then the streaming
    # keys of every sequence
    for bits in (4, 8):
        fc = FakeCache(kv_bits=bits, rope_theta=10000.0, retrieval_mask=[[1, 0], [0, 0]])
        for layer, hs in ((0, 1), (1, 2)):
            for seq, nb in ((-1, 3), (1, 1)):
                assert L.duo_prefill_staging_bytes(fc.h, layer, seq, 5, ctypes.byref(n)) == 0
                keys = up(nb * 5 * 2 * row) + 3 * hs * 20 * row  # chunk, streaming keys
                assert n.value == up(keys) + up(nb * 5 * 2 * row) + 3 * hs * 20 * row
            keys = up(3 * 5 * 2 * row) + 3 * hs * 20 * row
            need = up(keys) + up(3 * 5 * 2 * row) + 3 * hs * 20 * row
            assert L.duo_attn_prefill_staged(fc.h, layer, -1, p, p, p, 5, p, None, p, need - 16,
                                             None) == N.DUO_ERR_INVALID
            assert L.duo_attn_prefill_staged(fc.h, layer, -1, p, p, p, 5, p, None, None, need,
                                             None) == N.DUO_ERR_INVALID
            assert L.duo_attn_prefill(fc.h, layer, -1, p, p, p, 5, p, None,
                                      None) == N.DUO_ERR_UNSUPPORTED
        fc.close()



def test_read_probe_rejects_bad_arguments():
    """The streaming-read probe checks its arguments before launching anything."""
    L = N.lib()
    vp = ctypes.c_void_p
    big = vp(1 << 40)
    flag = vp((1 << 40) + 4096)
    assert L.duo_read_probe(None, 1024, flag, 0, None) == N.DUO_ERR_INVALID
    assert L.duo_read_probe(big, 1024, None, 0, None) == N.DUO_ERR_INVALID
    assert L.duo_read_probe(vp((1 << 40) + 8), 1024, flag, 0, None) == N.DUO_ERR_INVALID
    assert L.duo_read_probe(big, 1000, flag, 0, None) == N.DUO_ERR_INVALID
    assert L.duo_read_probe(big, 0, flag, 0, None) == N.DUO_ERR_INVALID
    assert L.duo_read_probe(big, 1024, flag, -1, None) == N.DUO_ERR_INVALID
    assert L.duo_read_probe(big, 1024, vp((1 << 40) + 4098), 0, None) == N.DUO_ERR_INVALID
