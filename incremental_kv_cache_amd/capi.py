"""ctypes declarations of the C ABI in include/kvcache.h (argument marshalling only)."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvcache.so")

# status codes (include/kvcache.h)
KVC_OK = 0
KVC_ERR_ZERO_BATCH = 1
KVC_ERR_ZERO_CAPACITY = 2
KVC_ERR_CAPACITY_EXCEEDS_POSITIONS = 3
KVC_ERR_ELEMENT_COUNT_OVERFLOW = 4
KVC_ERR_ALLOCATION_FAILED = 5
KVC_ERR_INPUT_RANK = 10
KVC_ERR_SINGLE_TOKEN_REQUIRED = 11
KVC_ERR_INPUT_BATCH_MISMATCH = 12
KVC_ERR_INPUT_WIDTH_MISMATCH = 13
KVC_ERR_CACHE_MODEL_WIDTH_MISMATCH = 14
KVC_ERR_CACHE_HEAD_COUNT_MISMATCH = 15
KVC_ERR_CACHE_HEAD_WIDTH_MISMATCH = 16
KVC_ERR_CACHE_LAYER_MISMATCH = 17
KVC_ERR_CACHE_LAYER_REVISION_MISMATCH = 18
KVC_ERR_CACHE_ROPE_MISMATCH = 19
KVC_ERR_FULL = 20
KVC_ERR_OUT_OF_BLOCKS = 21
KVC_ERR_CACHE_WINDOW_MISMATCH = 22
KVC_ERR_NONFINITE_KEY = 30
KVC_ERR_NONFINITE_VALUE = 31
KVC_ERR_NONFINITE_QUERY = 32
KVC_ERR_ROTARY_POSITION = 33
KVC_ERR_NONFINITE_OUTPUT = 34
KVC_ERR_TOKEN_RANGE = 35
KVC_ERR_BAD_CUT = 40
KVC_ERR_EMPTY_QUERY = 41
KVC_ERR_CHUNK_ROWS = 42
KVC_ERR_NULL_ARGUMENT = 50
KVC_ERR_DTYPE_UNSUPPORTED = 51
KVC_ERR_SHAPE_UNSUPPORTED = 52
KVC_ERR_BAD_ARGUMENT = 53
KVC_ERR_SCRATCH_EXCEEDED = 54
KVC_ERR_DEVICE = 60
KVC_ERR_DEFERRED = 61
KVC_ERR_INTERNAL = 62

KVC_F64, KVC_F32, KVC_BF16 = 0, 1, 2
KVC_POS_ROPE, KVC_POS_NONE = 0, 1
KVC_SYNC, KVC_ASYNC = 0, 1
KVC_TRUNCATE_KEEP_STALE_POSITION = 1
KVC_STAGE_PROJECT, KVC_STAGE_ATTEND, KVC_STAGE_MERGE, KVC_STAGE_COMMIT, KVC_STAGE_OUTPUT = 0, 1, 2, 3, 4
KVC_STAGES = 5
KVC_PE_NONE, KVC_PE_SINUSOIDAL = 0, 1
KVC_STATIC_SCRATCH_BYTES = 32 << 20


class ErrorDetail(C.Structure):
    _fields_ = [
        ("status", C.c_int32), ("parameter", C.c_int32), ("sequence", C.c_int32), ("layer", C.c_int32),
        ("expected", C.c_int64), ("actual", C.c_int64),
        ("cache_revision", C.c_uint64), ("layer_revision", C.c_uint64),
        ("flat_index", C.c_int64), ("value", C.c_double),
        ("rope_feature_width", C.c_int32 * 2), ("rope_max_positions", C.c_int32 * 2),
        ("rope_base", C.c_double * 2), ("message", C.c_char * 256),
    ]


class Work(C.Structure):
    _fields_ = [
        ("full_prefix_rows_per_projection", C.c_int64),
        ("incremental_rows_per_projection", C.c_int64),
        ("reused_key_value_rows", C.c_int64),
        ("position_min", C.c_int32), ("position_max", C.c_int32),
    ]

    def as_dict(self):
        return {"full_prefix_rows_per_projection": self.full_prefix_rows_per_projection,
                "incremental_rows_per_projection": self.incremental_rows_per_projection,
                "reused_key_value_rows": self.reused_key_value_rows,
                "position_min": self.position_min, "position_max": self.position_max}


class CacheDesc(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("heads", C.c_int32), ("head_width", C.c_int32), ("model_width", C.c_int32),
        ("capacity", C.c_int32), ("max_chunk_rows", C.c_int32), ("kv_dtype", C.c_int32),
        ("pos_mode", C.c_int32), ("rope_max_positions", C.c_int32), ("device", C.c_int32),
        ("rope_base", C.c_double), ("block_rows", C.c_int32), ("pool_blocks", C.c_int32),
        ("kv_heads", C.c_int32), ("window", C.c_int32),
    ]


P = C.c_void_p
PP = C.POINTER(C.c_void_p)
I32 = C.c_int32
I64 = C.c_int64
PI32 = C.POINTER(C.c_int32)
PI64 = C.POINTER(C.c_int64)

PROTOTYPES = {
    "kvc_params_create": (I32, [I32, I32, P, P, P, P, PP]),
    "kvc_params_create_grouped": (I32, [I32, I32, I32, P, P, P, P, PP]),
    "kvc_params_mark_updated": (I32, [P, I32]),
    "kvc_params_destroy": (None, [P]),
    "kvc_layer_create": (I32, [P, I32, I32, C.c_double, I32, PP]),
    "kvc_layer_create_windowed": (I32, [P, I32, I32, C.c_double, I32, I32, PP]),
    "kvc_layer_destroy": (None, [P]),
    "kvc_reuse_cut": (I32, [P, I32, I64, PI64]),
    "kvc_cache_create": (I32, [P, I32, I32, I32, P, PP]),
    "kvc_cache_create_paged": (I32, [P, I32, I32, I32, I32, I32, P, PP]),
    "kvc_cache_destroy": (None, [P]),
    "kvc_fork": (I32, [P, I32, I32, I32]),
    "kvc_pool_usage": (I32, [P, PI32, PI32]),
    "kvc_append_and_attend": (I32, [P, P, P, I32, PI64, P, I32, C.POINTER(Work)]),
    "kvc_append_and_attend_static": (I32, [P, P, P, I32, PI64, P, I32, C.POINTER(Work)]),
    "kvc_continue_chunk": (I32, [P, P, P, I32, PI32, P, I32, C.POINTER(Work)]),
    "kvc_newest_weights": (I32, [P, I32, P, I64, PI32]),
    "kvc_truncate": (I32, [P, PI32, I32]),
    "kvc_reset": (I32, [P]),
    "kvc_snapshot": (I32, [P, I32, P, P, PI32, I64, PI32]),
    "kvc_lengths": (I32, [P, PI32, PI32]),
    "kvc_sync": (I32, [P]),
    "kvc_lcp_cut": (I32, [PI32, I64, PI32, I64, PI64]),
    "kvc_cache_describe": (I32, [P, C.POINTER(CacheDesc)]),
    "kvc_storage_pointers": (I32, [P, PP, PP, PI64]),
    "kvc_copy_storage": (I32, [P, P, P]),
    "kvc_profile_enable": (I32, [P, I32]),
    "kvc_profile_read": (I32, [P, C.POINTER(C.c_float), PI32]),
    "kvc_stream_read": (I32, [P, I64, P, P]),
    "kvc_mfma_rate": (I32, [I64, P, P, C.POINTER(C.c_double)]),
    "kvc_session_create": (I32, [PP, I32, P, I32, I32, I32, I32, I32, P, PP]),
    "kvc_session_destroy": (None, [P]),
    "kvc_session_chunk": (I32, [P, P, I32, PI32, P, I32, C.POINTER(Work)]),
    "kvc_session_decode": (I32, [P, P, P, I32, C.POINTER(Work)]),
    "kvc_session_truncate": (I32, [P, PI32, I32]),
    "kvc_session_reset": (I32, [P]),
    "kvc_session_sync": (I32, [P]),
    "kvc_session_layer_cache": (I32, [P, I32, PP]),
    "kvc_last_error": (C.POINTER(ErrorDetail), []),
    "kvc_status_name": (C.c_char_p, [I32]),
}


def declare(lib: C.CDLL) -> C.CDLL:
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = None


def lib() -> C.CDLL:
    """The in-tree libkvcache.so.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with `python -m incremental_kv_cache_amd.build`")
        _lib = declare(C.CDLL(LIB_PATH))
    return _lib
