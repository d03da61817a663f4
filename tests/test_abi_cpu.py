"""The C ABI library loads and exports every declared symbol; host-only calls work (CPU)."""
import ctypes as C
import os
import re

import pytest

from incremental_kv_cache_amd import capi
from incremental_kv_cache_amd import kvcache as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvcache.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(capi.LIB_PATH):
        pytest.fail(f"{capi.LIB_PATH} not built (run __graft_entry__.build())")
    return capi.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(capi.PROTOTYPES), "binding prototypes and header disagree"


def test_status_names(lib):
    assert K.kvc_status_name(0) == "KVC_OK"
    for name in dir(capi):
        if name.startswith("KVC_ERR_"):
            assert K.kvc_status_name(getattr(capi, name)) == name
    assert K.kvc_status_name(9999) == "KVC_ERR_UNKNOWN"


def test_lcp_cut_through_the_abi(lib):
    """Prefix-reuse note cut rules, computed by the library's host helper."""
    assert K.kvc_lcp_cut([1, 2, 3, 4, 5, 6, 7, 8], [1, 2, 3, 4, 20, 6, 7, 8, 9, 10, 11, 12]) == 4
    assert K.kvc_lcp_cut([1, 2, 3, 4, 5, 6, 7, 8], list(range(1, 13))) == 8
    assert K.kvc_lcp_cut([1, 2, 3, 4, 5, 6, 7, 8], [1, 2, 3, 4]) == 3
    assert K.kvc_lcp_cut([], [7]) == 0
    with pytest.raises(K.KvcError) as e:
        K.kvc_lcp_cut([1], [])
    assert e.value.name == "KVC_ERR_EMPTY_QUERY"


def test_params_and_layer_validation_without_device(lib):
    """Parameter and layer handles need no device; their argument checks run on the host."""
    dummy = C.c_void_p(16)
    out = C.c_void_p()
    assert lib.kvc_params_create(4, capi.KVC_F64, dummy, dummy, dummy, None, None) == capi.KVC_ERR_NULL_ARGUMENT
    assert lib.kvc_params_create(0, capi.KVC_F64, dummy, dummy, dummy, None, C.byref(out)) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_params_create(4, 7, dummy, dummy, dummy, None, C.byref(out)) == capi.KVC_ERR_DTYPE_UNSUPPORTED
    assert lib.kvc_params_create(4, capi.KVC_F64, dummy, dummy, dummy, None, C.byref(out)) == capi.KVC_OK
    params = out
    layer = C.c_void_p()
    assert lib.kvc_layer_create(params, 3, 0, 10000.0, 4, C.byref(layer)) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_layer_create(params, 4, 0, 10000.0, 4, C.byref(layer)) == capi.KVC_ERR_SHAPE_UNSUPPORTED
    assert lib.kvc_layer_create(params, 2, 0, -1.0, 4, C.byref(layer)) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_layer_create(params, 2, 0, 10000.0, 4, C.byref(layer)) == capi.KVC_OK
    # cache-constructor checks that precede any allocation (Chapter 37 order)
    cache = C.c_void_p()
    assert lib.kvc_cache_create(layer, 0, 4, 1, None, C.byref(cache)) == capi.KVC_ERR_ZERO_BATCH
    assert lib.kvc_cache_create(layer, 1, 0, 1, None, C.byref(cache)) == capi.KVC_ERR_ZERO_CAPACITY
    assert lib.kvc_cache_create(layer, 1, 5, 1, None, C.byref(cache)) == capi.KVC_ERR_CAPACITY_EXCEEDS_POSITIONS
    d = lib.kvc_last_error().contents
    assert (d.expected, d.actual) == (4, 5)
    assert b"need more rotary positions than the layer" in d.message
    assert lib.kvc_params_mark_updated(params, 3) == capi.KVC_ERR_BAD_ARGUMENT
    lib.kvc_layer_destroy(layer)
    lib.kvc_params_destroy(params)


def test_binding_rejects_outputs_and_row_counts_the_kernels_would_overrun():
    """The binding checks a caller-supplied output (type, shape, device) and the
    per-sequence row counts before any pointer reaches the library: a wrong one
    would make the kernels write past the buffer or read past the host array."""
    import types

    import torch

    from incremental_kv_cache_amd import kvcache as K

    B, D = 2, 8
    desc = {"kv_dtype": K.KVC_F32, "batch": B, "model_width": D}
    cache = types.SimpleNamespace(_lib=None, ptr=None, desc=desc)
    layer = types.SimpleNamespace(ptr=None)
    x1 = torch.zeros((B, 1, D), dtype=torch.float32)
    for bad, exc in ((torch.zeros((B, 1, D), dtype=torch.float64), TypeError),
                     (torch.zeros((B, 1, D), dtype=torch.bfloat16), TypeError),
                     (torch.zeros((B, 1, D - 1), dtype=torch.float32), ValueError),
                     (torch.zeros((B + 1, 1, D), dtype=torch.float32), ValueError),
                     (torch.zeros((B * D,), dtype=torch.float32), ValueError)):
        with pytest.raises(exc, match="out"):
            K.kvc_append_and_attend(layer, cache, x1, out=bad)
    xn = torch.zeros((B, 4, D), dtype=torch.float32)
    with pytest.raises(ValueError, match="out"):
        K.kvc_continue_chunk(layer, cache, xn, out=torch.zeros((B, 3, D), dtype=torch.float32))
    with pytest.raises(TypeError, match="out"):
        K.kvc_continue_chunk(layer, cache, xn, out=torch.zeros((B, 4, D), dtype=torch.float64))
    for rows in ([4], [4, 4, 4], [[4, 4]]):
        with pytest.raises(ValueError, match="n_rows"):
            K.kvc_continue_chunk(layer, cache, xn, n_rows=rows)
    session = types.SimpleNamespace(_lib=None, ptr=None, desc=desc)
    tok = torch.zeros((B, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="n_rows"):
        K.kvc_session_chunk(session, tok, n_rows=[1])
    with pytest.raises(ValueError, match="tokens"):
        K.kvc_session_chunk(session, torch.zeros((B + 1, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match="out"):
        K.kvc_session_chunk(session, tok, out=torch.zeros((B, 5, D), dtype=torch.float32))
    with pytest.raises(ValueError, match="tokens"):
        K.kvc_session_decode(session, torch.zeros((B, 1), dtype=torch.int32))
    with pytest.raises(TypeError, match="out"):
        K.kvc_session_decode(session, torch.zeros((B,), dtype=torch.int32),
                             out=torch.zeros((B, 1, D), dtype=torch.float64))
