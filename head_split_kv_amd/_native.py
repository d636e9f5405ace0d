"""ctypes view of ``libduo.so`` (the C ABI declared in ``include/duo.h``).

Loading fails loudly when the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libduo.so")

DUO_OK, DUO_ERR_INVALID, DUO_ERR_CAPACITY, DUO_ERR_UNSUPPORTED, DUO_ERR_HIP = range(5)
DUO_F32, DUO_BF16 = 0, 1

# Every symbol include/duo.h declares.
EXPORTS = (
    "duo_layout_query", "duo_cache_create", "duo_cache_init", "duo_cache_reset",
    "duo_cache_set_lengths", "duo_cache_destroy",
    "duo_kv_append", "duo_attn_decode", "duo_attn_decode_noalloc", "duo_decode_step", "duo_attn_prefill",
    "duo_attn_prefill_staged", "duo_prefill_staging_bytes", "duo_attn_gate_mixed",
    "duo_slot_positions",
    "duo_cache_lengths", "duo_kv_bytes", "duo_set_decode_splits", "duo_timing_enable",
    "duo_timing_read", "duo_read_probe", "duo_binarize_gates", "duo_head_order", "duo_permute_blocks",
    "duo_status_string",
)
TIMING_DECODE, TIMING_PREFILL = 0, 1
PREFILL_WINDOW, PREFILL_CHUNK = 0, 1
KV4_GROUP = 128


class DuoConfig(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("sink", ctypes.c_int32),
        ("recent", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("max_splits", ctypes.c_int32),
        ("prefill_tiles", ctypes.c_int32),
        ("retrieval_mask", ctypes.POINTER(ctypes.c_uint8)),
        ("streaming_prefill", ctypes.c_int32),
        ("kv_bits", ctypes.c_int32),
        ("rope_theta", ctypes.c_float),
    ]


class DuoLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "arena_bytes", "full_k_off", "full_v_off", "str_k_off", "str_v_off", "slot_pos_off",
        "seq_len_off", "workspace_off", "workspace_bytes", "rope_off", "rope_bytes")]


class DuoError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libduo.so not found at {LIB_PATH}; build it with `python -m head_split_kv_amd.build`"
        )
    L = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    vp = ctypes.c_void_p
    i32 = ctypes.c_int32
    P = ctypes.POINTER
    u64 = ctypes.c_uint64
    sig = {
        "duo_layout_query": (st, [P(DuoConfig), P(DuoLayout)]),
        "duo_cache_create": (st, [P(DuoConfig), vp, ctypes.c_uint64, P(vp)]),
        "duo_cache_init": (st, [P(DuoConfig), vp, ctypes.c_uint64, vp, P(vp)]),
        "duo_cache_reset": (st, [vp, vp]),
        "duo_cache_set_lengths": (st, [vp, P(i32), vp]),
        "duo_cache_destroy": (st, [vp]),
        "duo_kv_append": (st, [vp, i32, i32, vp, vp, i32, vp]),
        "duo_attn_decode": (st, [vp, i32, vp, vp, vp, vp]),
        "duo_attn_decode_noalloc": (st, [vp, i32, vp, vp, vp, vp]),
        "duo_decode_step": (st, [vp, i32, vp, vp, vp, vp, vp, vp]),
        "duo_attn_prefill": (st, [vp, i32, i32, vp, vp, vp, i32, vp, vp, vp]),
        "duo_attn_prefill_staged": (st, [vp, i32, i32, vp, vp, vp, i32, vp, vp, vp, u64, vp]),
        "duo_prefill_staging_bytes": (st, [vp, i32, i32, i32, P(ctypes.c_uint64)]),
        "duo_attn_gate_mixed": (st, [vp, i32, i32, vp, vp, vp, i32, P(ctypes.c_float), vp, vp]),
        "duo_slot_positions": (st, [vp, i32, P(i32), vp]),
        "duo_cache_lengths": (st, [vp, P(i32)]),
        "duo_kv_bytes": (st, [P(DuoConfig), P(i32), i32, P(ctypes.c_uint64),
                              P(ctypes.c_uint64)]),
        "duo_set_decode_splits": (st, [vp, i32]),
        "duo_timing_enable": (st, [vp, i32]),
        "duo_timing_read": (st, [vp, i32, P(ctypes.c_double), P(i32)]),
        "duo_read_probe": (st, [vp, ctypes.c_uint64, vp, i32, vp]),
        "duo_binarize_gates": (st, [P(ctypes.c_float), i32, i32, ctypes.c_double,
                                    P(ctypes.c_uint8), P(ctypes.c_float), P(i32)]),
        "duo_head_order": (st, [P(ctypes.c_uint8), i32, i32, P(i32), P(i32)]),
        "duo_permute_blocks": (st, [vp, vp, ctypes.c_int64, i32, ctypes.c_int64, P(i32), vp]),
        "duo_status_string": (ctypes.c_char_p, [st]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().duo_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status != DUO_OK:
        raise DuoError(status, where)
