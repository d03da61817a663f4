"""Host side of the entry point that allocates nothing (kvc_append_and_attend_static).

The manager runs against tests/hostcheck_backend.cpp, whose stand-in kernels
tag each candidate row; its "static scratch" is host memory whose reported
size a test hook can shrink.  Checked here: the same request checks and the
same appended rows as kvc_append_and_attend, the cache's own candidate
buffers untouched by the static call, a call needing more than the scratch
refused with its need before any work, and the cache's own scratch back in
use afterwards.
"""
import ctypes as C

import numpy as np
import pytest

from incremental_kv_cache_amd import capi
from tests import hostcheck

DUMMY = C.c_void_p(64)


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    lib = hostcheck.build(tmp_path_factory, "hoststatic")
    lib.kvc_test_fake_kernels.argtypes = [C.c_int]
    lib.kvc_test_static_scratch_bytes.argtypes = [C.c_ulonglong]
    return lib


@pytest.fixture
def fake(lib):
    lib.kvc_test_fake_kernels(1)
    lib.kvc_test_static_scratch_bytes(0)
    yield lib
    lib.kvc_test_fake_kernels(0)
    lib.kvc_test_static_scratch_bytes(0)


def _setup(lib, batch=3, cap=64, heads=2, d=8):
    p = C.c_void_p()
    assert lib.kvc_params_create(d, capi.KVC_F64, DUMMY, DUMMY, DUMMY, None, C.byref(p)) == 0
    lay = C.c_void_p()
    assert lib.kvc_layer_create(p, heads, capi.KVC_POS_ROPE, 10000.0, cap, C.byref(lay)) == 0
    c = C.c_void_p()
    assert lib.kvc_cache_create(lay, batch, cap, 16, None, C.byref(c)) == 0
    return lay, c


def _decode(lib, fn, lay, c, batch, d, flags=0):
    shape = (C.c_int64 * 3)(batch, 1, d)
    w = capi.Work()
    st = getattr(lib, fn)(lay, c, DUMMY, 3, shape, DUMMY, flags, C.byref(w))
    return st, w.as_dict()


def _snap(lib, c, seq, heads=2, dh=4):
    n = C.c_int32()
    assert lib.kvc_snapshot(c, seq, None, None, None, 0, C.byref(n)) == 0
    k = np.zeros((heads, n.value, dh))
    v = np.zeros((heads, n.value, dh))
    pos = np.zeros(n.value, np.int32)
    assert lib.kvc_snapshot(c, seq, k.ctypes.data_as(C.c_void_p), v.ctypes.data_as(C.c_void_p),
                            pos.ctypes.data_as(capi.PI32), n.value, C.byref(n)) == 0
    return k, v, pos


def test_static_entry_point_appends_what_the_regular_one_does(fake):
    lib = fake
    B, d = 3, 8
    rows = np.array([5, 0, 9], np.int32)
    caches = []
    for fn in ("kvc_append_and_attend", "kvc_append_and_attend_static"):
        lib.kvc_test_fake_kernels(1)  # restart the tag counter: both caches get the same tags
        lay, c = _setup(lib)
        w = capi.Work()
        assert lib.kvc_continue_chunk(lay, c, DUMMY, 9, rows.ctypes.data_as(capi.PI32), DUMMY, 0, C.byref(w)) == 0
        works = []
        for _ in range(3):
            st, work = _decode(lib, fn, lay, c, B, d)
            assert st == 0, lib.kvc_last_error().contents.message
            works.append(work)
        caches.append((lay, c, works))
    (_, c0, w0), (_, c1, w1) = caches
    assert w0 == w1
    assert w1[0]["full_prefix_rows_per_projection"] == int(rows.sum()) + B
    for b in range(B):
        for a, e in zip(_snap(lib, c0, b), _snap(lib, c1, b)):
            np.testing.assert_array_equal(a, e)
    # the regular entry point still uses the cache's own scratch after a static call
    st, _ = _decode(lib, "kvc_append_and_attend", caches[1][0], c1, B, d)
    assert st == 0
    for c in (c0, c1):
        lib.kvc_cache_destroy(c)


def test_static_entry_point_checks_and_scratch_size(fake):
    lib = fake
    B, d = 3, 8
    lay, c = _setup(lib)
    # request checks come first, in the chapter's order, as for kvc_append_and_attend
    shape = (C.c_int64 * 3)(B, 2, d)
    assert lib.kvc_append_and_attend_static(lay, c, DUMMY, 3, shape, DUMMY, 0, None) == \
        capi.KVC_ERR_SINGLE_TOKEN_REQUIRED
    shape = (C.c_int64 * 3)(B + 1, 1, d)
    assert lib.kvc_append_and_attend_static(lay, c, DUMMY, 3, shape, DUMMY, 0, None) == \
        capi.KVC_ERR_INPUT_BATCH_MISMATCH
    assert lib.kvc_append_and_attend_static(None, c, DUMMY, 3, shape, DUMMY, 0, None) == capi.KVC_ERR_NULL_ARGUMENT
    # f64, B = 3, H = 2, d_h = 4, C = 64: queries and each candidate buffer 3 * 2 * 4 * 8 = 192
    # bytes, partials (one 512-row tile) 3 * 2 * 1 * 6 * 8 = 288 bytes; each rounded up to 256
    need = 3 * 256 + 512
    lib.kvc_test_static_scratch_bytes(need - 1)
    before = [_snap(lib, c, b) for b in range(B)]
    st, _ = _decode(lib, "kvc_append_and_attend_static", lay, c, B, d)
    assert st == capi.KVC_ERR_SCRATCH_EXCEEDED
    e = lib.kvc_last_error().contents
    assert (e.expected, e.actual) == (need - 1, need)
    after = [_snap(lib, c, b) for b in range(B)]
    for x, y in zip(before, after):
        for a, e2 in zip(x, y):
            np.testing.assert_array_equal(a, e2)
    lib.kvc_test_static_scratch_bytes(need)
    st, work = _decode(lib, "kvc_append_and_attend_static", lay, c, B, d)
    assert st == 0 and work["incremental_rows_per_projection"] == B
    assert lib.kvc_status_name(capi.KVC_ERR_SCRATCH_EXCEEDED) == b"KVC_ERR_SCRATCH_EXCEEDED"
    lib.kvc_cache_destroy(c)
