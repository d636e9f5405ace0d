"""Gate binarization and head order in the C library against the CPU oracle (host-only
calls, so they run without a GPU), and the argument checks of the weight reordering that
return before any launch.

Parity bar: bit-exact (integer masks and orders; tau is one of the input gates).
"""
import ctypes
import math
import os

import numpy as np
import pytest

from oracle import duo_oracle as O

hsk = pytest.importorskip("head_split_kv_amd")
from head_split_kv_amd import _native as N  # noqa: E402

if not os.path.exists(N.LIB_PATH):
    pytest.skip("libduo.so not built", allow_module_level=True)


def _gate_cases():
    rng = np.random.default_rng(61)
    cases = []
    for (L, H) in [(1, 1), (1, 5), (3, 4), (32, 32), (32, 8), (7, 3)]:
        cases.append(rng.random((L, H)).astype(np.float32))                 # distinct
        cases.append((rng.integers(0, 4, (L, H)) / 4.0).astype(np.float32))  # many ties
        cases.append(np.full((L, H), 0.5, dtype=np.float32))                 # all equal
    # a trained-looking mix: most gates near 0, a few near 1, exact 0/1 clamps
    a = np.clip(rng.normal(0.05, 0.1, (32, 8)), 0, 1)
    a[rng.integers(0, 32, 40), rng.integers(0, 8, 40)] = 1.0
    cases.append(a.astype(np.float32))
    return cases


@pytest.mark.parametrize("ratio", [0.0, 0.1, 0.25, 1 / 3, 0.5, 0.7, 0.75, 1.0])
def test_binarize_matches_oracle(ratio):
    for a in _gate_cases():
        mask, tau, n = hsk.duo_binarize_gates(a, ratio)
        want, want_tau = O.binarize_gates(a.astype(np.float64), ratio)
        assert np.array_equal(mask, want), (a.shape, ratio)
        assert n == O.retrieval_count(a.size, ratio) == int(want.sum())
        assert tau == want_tau or (math.isinf(tau) and math.isinf(want_tau))


def test_binarize_page_budgets():
    """25 % of the 1,024 Llama-2-7B gates and 50 % of the 256 Llama-3-8B KV-head gates."""
    rng = np.random.default_rng(62)
    m, _, n = hsk.duo_binarize_gates(rng.random((32, 32)), 0.25)
    assert n == 256 and m.sum() == 256
    m, _, n = hsk.duo_binarize_gates(rng.random((32, 8)), 0.5)
    assert n == 128 and m.sum() == 128


def test_binarize_rejects_bad_input():
    L = N.lib()
    a = np.zeros((2, 2), dtype=np.float32)
    m = np.zeros((2, 2), dtype=np.uint8)
    pa = a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    pm = m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    assert L.duo_binarize_gates(pa, 2, 2, 1.5, pm, None, None) == N.DUO_ERR_INVALID
    assert L.duo_binarize_gates(pa, 2, 2, -0.1, pm, None, None) == N.DUO_ERR_INVALID
    assert L.duo_binarize_gates(pa, 2, 2, float("nan"), pm, None, None) == N.DUO_ERR_INVALID
    assert L.duo_binarize_gates(pa, 0, 2, 0.5, pm, None, None) == N.DUO_ERR_INVALID
    assert L.duo_binarize_gates(None, 2, 2, 0.5, pm, None, None) == N.DUO_ERR_INVALID
    assert L.duo_binarize_gates(pa, 2, 2, 0.5, None, None, None) == N.DUO_ERR_INVALID
    a[1, 1] = np.nan
    assert L.duo_binarize_gates(pa, 2, 2, 0.5, pm, None, None) == N.DUO_ERR_INVALID
    a[1, 1] = np.inf
    assert L.duo_binarize_gates(pa, 2, 2, 0.5, pm, None, None) == N.DUO_ERR_INVALID
    a[1, 1] = 0.0
    assert L.duo_binarize_gates(pa, 2, 2, 0.5, pm, None, None) == N.DUO_OK


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_head_order_matches_oracle(G):
    rng = np.random.default_rng(63 + G)
    for H in (1, 2, 5, 8, 32, 64):
        for _ in range(6):
            m = (rng.random(H) < rng.random()).astype(np.uint8)
            kv, q = hsk.duo_head_order(m, G)
            want = O.head_order(m)
            assert np.array_equal(kv, want)
            assert np.array_equal(q, O.query_head_order(want, G))


def test_head_order_rejects_bad_input():
    L = N.lib()
    m = np.ones(4, dtype=np.uint8)
    o = np.zeros(8, dtype=np.int32)
    pm = m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    po = o.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert L.duo_head_order(pm, 0, 1, po, None) == N.DUO_ERR_INVALID
    assert L.duo_head_order(pm, 4, 0, po, None) == N.DUO_ERR_INVALID
    assert L.duo_head_order(None, 4, 1, po, None) == N.DUO_ERR_INVALID
    assert L.duo_head_order(pm, 4, 1, None, None) == N.DUO_ERR_INVALID
    assert L.duo_head_order(pm, 4, 1, po, None) == N.DUO_OK


def test_permute_blocks_rejects_before_launch():
    """Every call here fails a host check, so nothing is launched (safe without a GPU)."""
    L = N.lib()
    order = np.array([1, 0, 2], dtype=np.int32)
    po = order.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    src, dst = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 24)
    bad = np.array([0, 0, 2], dtype=np.int32)
    oob = np.array([0, 1, 3], dtype=np.int32)
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))  # noqa: E731
    assert L.duo_permute_blocks(src, dst, 4, 3, 64, P(bad), None) == N.DUO_ERR_INVALID
    assert L.duo_permute_blocks(src, dst, 4, 3, 64, P(oob), None) == N.DUO_ERR_INVALID
    assert L.duo_permute_blocks(src, dst, 4, 3, 24, po, None) == N.DUO_ERR_INVALID
    assert L.duo_permute_blocks(src, dst, 4, 3, 0, po, None) == N.DUO_ERR_INVALID
    assert L.duo_permute_blocks(src, dst, -1, 3, 64, po, None) == N.DUO_ERR_INVALID
    assert L.duo_permute_blocks(src, dst, 4, 0, 64, po, None) == N.DUO_ERR_INVALID
    assert L.duo_permute_blocks(src, dst, 4, 1025, 64, po, None) == N.DUO_ERR_INVALID
    assert L.duo_permute_blocks(ctypes.c_void_p((1 << 20) + 8), dst, 4, 3, 64, po,
                                None) == N.DUO_ERR_INVALID
    assert L.duo_permute_blocks(None, dst, 4, 3, 64, po, None) == N.DUO_ERR_INVALID
    assert L.duo_permute_blocks(src, dst, 4, 3, 64, None, None) == N.DUO_ERR_INVALID
    # overlapping source and destination
    assert L.duo_permute_blocks(src, ctypes.c_void_p((1 << 20) + 64), 4, 3, 64, po,
                                None) == N.DUO_ERR_INVALID
    # 2^23 * 3 * 256 = 6.4e9 chunks and 2^22 * 3 * 256 = 3.2e9 chunks, beyond 2^31
    for outer in (1 << 23, 1 << 22):
        assert outer * 3 * ((1 << 12) // 16) > (1 << 31)
        assert L.duo_permute_blocks(src, ctypes.c_void_p(1 << 44), outer, 3, 1 << 12, po,
                                    None) == N.DUO_ERR_INVALID
    # one block of 2^31 chunks
    one = np.array([0], dtype=np.int32)
    assert L.duo_permute_blocks(src, ctypes.c_void_p(1 << 44), 1, 1, 1 << 35, P(one),
                                None) == N.DUO_ERR_INVALID
    # outer = 0 is a valid no-op (nothing to launch)
    assert L.duo_permute_blocks(src, dst, 0, 3, 64, po, None) == N.DUO_OK
