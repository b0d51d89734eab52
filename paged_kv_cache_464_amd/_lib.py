"""ctypes declarations of libpa.so (the C ABI in include/pa.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any operation.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_OK = 0
PA_ERR_INVALID = -1
PA_ERR_NO_BLOCKS = -2
PA_ERR_BAD_SEQ = -3
PA_ERR_HIP = -4
PA_ERR_UNBOUND = -5

PA_DTYPE_FP16 = 0
PA_DTYPE_FP8_E4M3 = 1
PA_DTYPE_INT8 = 2

PA_DEV_BAD_SLOT = 1
PA_DEV_BAD_BLOCK = 2
PA_DEV_BAD_LEN = 4
PA_DEV_BAD_ORDER = 8

PA_LOADS_AUTO = 0
PA_LOADS_STREAMING = 1
PA_LOADS_CACHED = 2

PA_NOALLOC_SCRATCH_BYTES = 33554432

PA_SHARED_REREAD = 1


class pa_pool_info(C.Structure):
    _fields_ = [("layers", C.c_int32), ("kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("block_size", C.c_int32), ("dtype", C.c_int32), ("num_blocks", C.c_int32),
                ("elem_bytes", C.c_int32), ("bound", C.c_int32),
                ("tile_bytes", C.c_uint64), ("kv_bytes", C.c_uint64), ("total_bytes", C.c_uint64),
                ("softmax_scale", C.c_float), ("reserved", C.c_int32)]


class pa_stats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("num_blocks", "free_blocks", "used_blocks",
                                          "shared_blocks", "num_seqs", "cow_copies",
                                          "alloc_failures", "cache_hits", "cache_misses",
                                          "cache_evictions", "cached_blocks")]


class pa_profile(C.Structure):
    _fields_ = [("decode_launches", C.c_int32), ("reduce_launches", C.c_int32),
                ("decode_ms", C.c_double), ("reduce_ms", C.c_double)]


class pa_shared_plan(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("num_seqs", C.c_int32), ("num_q_heads", C.c_int32),
                ("max_blocks", C.c_int32), ("num_items", C.c_int32), ("num_slots", C.c_int32),
                ("chunk_tokens", C.c_int32), ("num_private", C.c_int32), ("flags", C.c_int32),
                ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_uint64)]


_P = C.c_void_p
_I32 = C.c_int32
_PI32 = C.POINTER(C.c_int32)

# name -> (restype, argtypes); every symbol declared in include/pa.h
SIGNATURES = {
    "pa_pool_create": (C.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, C.POINTER(_P)]),
    "pa_pool_destroy": (C.c_int, [_P]),
    "pa_pool_info_get": (C.c_int, [_P, C.POINTER(pa_pool_info)]),
    "pa_pool_set_free_order": (C.c_int, [_P, _PI32, _I32]),
    "pa_pool_set_load_policy": (C.c_int, [_P, _I32]),
    "pa_pool_load_policy": (C.c_int, [_P, _PI32, _PI32]),
    "pa_pool_bind": (C.c_int, [_P, _P, C.POINTER(C.c_float), C.POINTER(C.c_float)]),
    "pa_pool_bind_int8": (C.c_int, [_P, _P, C.POINTER(C.c_float), C.POINTER(C.c_float), _PI32, _PI32]),
    "pa_multi_token_workspace_bytes": (C.c_int, [_P, _PI32, _I32, _I32, C.POINTER(C.c_uint64)]),
    "pa_multi_token_attention": (C.c_int, [_P, _I32, _P, _I32, _PI32, _P, _I32, _P, _I32, C.c_float, _P, _P,
                                           C.c_uint64, _P]),
    "pa_seq_create": (C.c_int, [_P, _PI32]),
    "pa_seq_create_cached": (C.c_int, [_P, _PI32, _I32, _PI32, _PI32, _PI32]),
    "pa_alloc": (C.c_int, [_P, _I32, _I32, _PI32, _PI32, _P]),
    "pa_alloc_tokens": (C.c_int, [_P, _I32, _I32, _PI32, _PI32, _PI32, _P]),
    "pa_alloc_batch": (C.c_int, [_P, _PI32, _PI32, _I32, _PI32, _PI32, _PI32, _PI32, _P]),
    "pa_fork": (C.c_int, [_P, _I32, _PI32]),
    "pa_free": (C.c_int, [_P, _I32]),
    "pa_seq_len": (C.c_int, [_P, _I32, _PI32, _PI32]),
    "pa_block_tables": (C.c_int, [_P, _PI32, _I32, _I32, _PI32, _PI32]),
    "pa_pool_stats": (C.c_int, [_P, C.POINTER(pa_stats)]),
    "pa_refcounts": (C.c_int, [_P, _PI32]),
    "pa_free_queue": (C.c_int, [_P, _PI32, _PI32]),
    "pa_write_kv": (C.c_int, [_P, _I32, _P, _P, _P, _I32, _P]),
    "pa_gather_kv": (C.c_int, [_P, _I32, _P, _I32, _P, _P, _P]),
    "pa_copy_blocks": (C.c_int, [_P, _PI32, _PI32, _I32, _P]),
    "pa_decode_workspace_bytes": (C.c_int, [_P, _I32, _I32, _I32, _I32, C.POINTER(C.c_uint64)]),
    "pa_decode": (C.c_int, [_P, _I32, _P, _I32, _P, _I32, _P, _I32, _P, C.c_float, _I32, _P, _P,
                            C.c_uint64, _P]),
    "pa_decode_noalloc": (C.c_int, [_P, _I32, _P, _I32, _P, _I32, _P, _I32, _P, C.c_float, _I32, _P, _P]),
    "pa_order_longest_first": (C.c_int, [_PI32, _I32, _PI32]),
    "pa_shared_prefix_groups": (C.c_int, [_P, _PI32, _PI32, _I32, _I32, _I32, _PI32, _PI32, _PI32, _PI32]),
    "pa_decode_shared_prefix_workspace_bytes": (C.c_int, [_P, _I32, _I32, _PI32, _PI32, _PI32, _I32, _I32, _I32,
                                                          _PI32, C.POINTER(C.c_uint64)]),
    "pa_shared_prefix_plan": (C.c_int, [_P, _I32, _I32, _I32, _PI32, _PI32, _PI32, _I32, _I32, _PI32, _P,
                                        C.c_uint64, _P, C.POINTER(pa_shared_plan)]),
    "pa_decode_shared_prefix": (C.c_int, [_P, _I32, C.POINTER(pa_shared_plan), _P, _P, _P, _P, _P, _P,
                                          C.c_float, _P, _P]),
    "pa_stream_read": (C.c_int, [_P, C.c_uint64, _P, _P]),
    "pa_write_kv_decode": (C.c_int, [_P, _I32, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32, _P,
                                     C.c_float, _I32, _P, _P, C.c_uint64, _P]),
    "pa_decode_partials": (C.c_int, [_P, _I32, _P, _I32, _P, _I32, _P, _I32, _P, C.c_float, _I32,
                                     _P, C.c_uint64, _P]),
    "pa_lse_reduce": (C.c_int, [_P, _P, C.c_uint64, _P, _I32, _I32, _I32, _I32, _P, _P]),
    "pa_device_status": (C.c_int, [_P, C.POINTER(C.c_uint32), _I32, _P]),
    "pa_profile_begin": (C.c_int, [_P, _I32, _I32]),
    "pa_profile_end": (C.c_int, [_P, C.POINTER(pa_profile)]),
    "pa_last_error": (C.c_char_p, []),
}

_lib = None


def load() -> C.CDLL:
    """Load libpa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m paged_kv_cache_464_amd.build)")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
