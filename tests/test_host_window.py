"""Sliding-window caches on the CPU: ring bookkeeping, cut rules, binding.

A window layer's query reads only its last `window` rows (prefix-reuse note,
"Why a sliding-window partial hit must fall back"), so its cache is a ring of
`capacity` rows: lengths keep counting past the capacity and only the last
`capacity` rows are held; a cut that would need a row the ring no longer
holds is refused and kvc_reuse_cut falls back to 0.  The manager runs against
tests/hostcheck_backend.cpp with its stand-in kernels (tagged rows, appended
through the ring), as in tests/test_host_paging.py.
"""
import ctypes as C

import numpy as np
import pytest

from incremental_kv_cache_amd import capi
from tests import hostcheck
from oracle import prefix as P

DUMMY = C.c_void_p(64)


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    lib = hostcheck.build(tmp_path_factory, "hostwindow")
    lib.kvc_test_fake_kernels.argtypes = [C.c_int]
    return lib


@pytest.fixture
def fake(lib):
    lib.kvc_test_fake_kernels(1)
    yield lib
    lib.kvc_test_fake_kernels(0)


def _params(lib):
    p = C.c_void_p()
    assert lib.kvc_params_create(4, capi.KVC_F64, DUMMY, DUMMY, DUMMY, None, C.byref(p)) == 0
    return p


def _layer(lib, p, window, max_pos=1 << 20):
    lay = C.c_void_p()
    st = lib.kvc_layer_create_windowed(p, 2, capi.KVC_POS_ROPE, 10000.0, max_pos, window, C.byref(lay))
    assert st == 0, lib.kvc_last_error().contents.message
    return lay


def _cache(lib, lay, batch, cap, chunk):
    c = C.c_void_p()
    st = lib.kvc_cache_create(lay, batch, cap, chunk, None, C.byref(c))
    assert st == 0, lib.kvc_last_error().contents.message
    return c


def _chunk(lib, lay, c, rows):
    arr = np.ascontiguousarray(np.asarray(rows, np.int32))
    return lib.kvc_continue_chunk(lay, c, DUMMY, max(1, int(arr.max())), arr.ctypes.data_as(capi.PI32), DUMMY, 0,
                                  None)


def _lengths(lib, c, batch):
    ln = np.zeros(batch, np.int32)
    npos = np.zeros(batch, np.int32)
    assert lib.kvc_lengths(c, ln.ctypes.data_as(capi.PI32), npos.ctypes.data_as(capi.PI32)) == 0
    return ln.tolist(), npos.tolist()


def _snap(lib, c, seq):
    n = C.c_int32()
    assert lib.kvc_snapshot(c, seq, None, None, None, 0, C.byref(n)) == 0
    k = np.zeros((2, n.value, 2))
    pos = np.zeros(n.value, np.int32)
    assert lib.kvc_snapshot(c, seq, k.ctypes.data_as(C.c_void_p), None, pos.ctypes.data_as(capi.PI32), n.value,
                            C.byref(n)) == 0
    return k, pos


def test_window_layer_and_cache_checks(lib):
    p = _params(lib)
    bad = C.c_void_p()
    assert lib.kvc_layer_create_windowed(p, 2, capi.KVC_POS_ROPE, 1e4, 4096, -1, C.byref(bad)) == \
        capi.KVC_ERR_BAD_ARGUMENT
    lay = _layer(lib, p, 300)
    c = C.c_void_p()
    for cap, chunk in ((256, 1), (600, 1), (512, 513)):
        # smaller than the window, not a multiple of 256, a chunk larger than the ring
        assert lib.kvc_cache_create(lay, 2, cap, chunk, None, C.byref(c)) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_cache_create_paged(lay, 2, 512, 1, 256, 4, None, C.byref(c)) == capi.KVC_ERR_BAD_ARGUMENT
    c = _cache(lib, lay, 2, 512, 100)
    d = capi.CacheDesc()
    assert lib.kvc_cache_describe(c, C.byref(d)) == 0 and (d.window, d.capacity) == (300, 512)
    # the window is part of the binding, checked after the rotary setup
    other = _layer(lib, p, 0)
    shape = (C.c_int64 * 3)(2, 1, 4)
    assert lib.kvc_append_and_attend(other, c, DUMMY, 3, shape, DUMMY, 0, None) == capi.KVC_ERR_CACHE_WINDOW_MISMATCH
    e = lib.kvc_last_error().contents
    assert (e.expected, e.actual) == (0, 300)
    lib.kvc_cache_destroy(c)


def test_ring_holds_the_last_capacity_rows(fake):
    """Chunks and decodes well past the capacity: no FULL, lengths and positions
    keep counting, the snapshot holds the last 256 rows in order (their tags
    are those of the calls that appended them)."""
    lib = fake
    lay = _layer(lib, _params(lib), 100)
    c = _cache(lib, lay, 2, 256, 200)
    ref = [[], []]  # (call, chunk row) of every appended row
    call = 0
    shape = (C.c_int64 * 3)(2, 1, 4)
    for step in range(9):
        call += 1
        if step % 3 == 2:
            assert lib.kvc_append_and_attend(lay, c, DUMMY, 3, shape, DUMMY, 0, None) == 0
            rows = [1, 1]
        else:
            rows = [200, 150 - 40 * step % 150]
            assert _chunk(lib, lay, c, rows) == 0, lib.kvc_last_error().contents.message
        for b in range(2):
            ref[b] += [(call, i) for i in range(rows[b])]
    ln, npos = _lengths(lib, c, 2)
    assert ln == [len(ref[0]), len(ref[1])] and npos == ln and ln[0] > 256
    for b in range(2):
        k, pos = _snap(lib, c, b)
        held = min(ln[b], 256)
        assert k.shape[1] == held and list(pos) == list(range(ln[b] - held, ln[b]))
        tags = [call * 1e6 + b * 1e4 + i * 1e2 for call, i in ref[b][-held:]]
        np.testing.assert_array_equal(k[0, :, 0], tags)


def test_window_cuts_and_reuse(fake):
    """A cut is allowed when every row the continuation's first row reads is still
    held (cut - window + 1 >= len - capacity) or it is 0; others are refused with
    the smallest allowed cut, leaving the state unchanged; kvc_reuse_cut falls
    back to 0 exactly where oracle.prefix.window_continuable says so."""
    lib = fake
    W, cap = 100, 256
    lay = _layer(lib, _params(lib), W)
    c = _cache(lib, lay, 1, cap, 200)
    for _ in range(3):
        assert _chunk(lib, lay, c, [200]) == 0
    L = 600
    assert _lengths(lib, c, 1)[0] == [L]
    lo = L - cap + W - 1  # 443
    for lcp in (0, 1, lo - 1, lo, 500, L):
        out = C.c_int64()
        assert lib.kvc_reuse_cut(c, 0, lcp, C.byref(out)) == 0
        want = lcp if P.window_continuable(L, lcp, W, cap) else 0
        assert out.value == want, (lcp, out.value)
    before = _lengths(lib, c, 1), _snap(lib, c, 0)
    cut = np.array([lo - 1], np.int32)
    assert lib.kvc_truncate(c, cut.ctypes.data_as(capi.PI32), 0) == capi.KVC_ERR_BAD_CUT
    e = lib.kvc_last_error().contents
    assert (e.expected, e.actual) == (lo, lo - 1)
    after = _lengths(lib, c, 1), _snap(lib, c, 0)
    assert before[0] == after[0] and np.array_equal(before[1][0], after[1][0])
    cut = np.array([lo], np.int32)
    assert lib.kvc_truncate(c, cut.ctypes.data_as(capi.PI32), 0) == 0
    assert _lengths(lib, c, 1) == ([lo], [lo])
    # the ring still holds rows L - cap .. lo - 1: rows below were written over by
    # rows lo .. L - 1 before the cut, so a further cut below lo is refused
    k, pos = _snap(lib, c, 0)
    assert list(pos) == list(range(L - cap, lo))
    cut = np.array([lo - 3], np.int32)
    assert lib.kvc_truncate(c, cut.ctypes.data_as(capi.PI32), 0) == capi.KVC_ERR_BAD_CUT
    # appending again refills the discarded rows' slots: the oldest held row stays
    assert _chunk(lib, lay, c, [100]) == 0
    k, pos = _snap(lib, c, 0)
    assert list(pos) == list(range(L - cap, lo + 100))
    # past the old length the oldest held rows go
    assert _chunk(lib, lay, c, [150]) == 0
    k, pos = _snap(lib, c, 0)
    assert list(pos) == list(range(lo + 250 - cap, lo + 250))
    cut = np.array([0], np.int32)
    assert lib.kvc_truncate(c, cut.ctypes.data_as(capi.PI32), 0) == 0
    assert _chunk(lib, lay, c, [5]) == 0
    k, pos = _snap(lib, c, 0)
    assert list(pos) == list(range(5))


def test_window_fork_copies_the_ring(fake):
    lib = fake
    lay = _layer(lib, _params(lib), 64)
    c = _cache(lib, lay, 2, 256, 200)
    for _ in range(2):
        assert _chunk(lib, lay, c, [200, 0]) == 0
    assert lib.kvc_fork(c, 0, 1, 100) == capi.KVC_ERR_BAD_CUT  # rows 37..99 are gone
    assert lib.kvc_fork(c, 0, 1, 350) == 0
    assert _lengths(lib, c, 2) == ([400, 350], [400, 350])
    k0, p0 = _snap(lib, c, 0)
    k1, p1 = _snap(lib, c, 1)
    assert list(p1) == list(range(144, 350))
    np.testing.assert_array_equal(k1, k0[:, :350 - 144])


def _reuse(lib, c, lcp):
    out = C.c_int64()
    assert lib.kvc_reuse_cut(c, 0, lcp, C.byref(out)) == 0, lib.kvc_last_error().contents.message
    return out.value


def test_session_reset_and_truncate_keep_the_held_rows_in_step(fake):
    """A session's window layer wraps its ring, then is reset (or cut to 0) and
    refilled: the oldest held row starts again from 0 on the host as on the
    device, so a cut whose window the refilled ring holds is accepted
    (prefix-reuse note, "Why a sliding-window partial hit must fall back": a cut
    is refused only when the rows its continuation reads are gone)."""
    lib = fake
    W, cap = 100, 256
    lay = _layer(lib, _params(lib), W)
    layers = (C.c_void_p * 1)(lay)
    for rewind in ("reset", "cut0"):
        s = C.c_void_p()
        st = lib.kvc_session_create(layers, 1, DUMMY, 32, capi.KVC_PE_NONE, 1, cap, 200, None, C.byref(s))
        assert st == 0, lib.kvc_last_error().contents.message
        c = C.c_void_p()
        assert lib.kvc_session_layer_cache(s, 0, C.byref(c)) == 0
        rows = np.array([200], np.int32)
        for _ in range(2):  # 400 rows: slots 0 .. 143 written twice, rows 0 .. 143 gone
            assert lib.kvc_session_chunk(s, DUMMY, 200, rows.ctypes.data_as(capi.PI32), DUMMY, 0, None) == 0
        assert _reuse(lib, c, 150) == 0  # row 51 .. 149 of the continuation are gone
        if rewind == "reset":
            assert lib.kvc_session_reset(s) == 0
        else:
            zero = np.array([0], np.int32)
            assert lib.kvc_session_truncate(s, zero.ctypes.data_as(capi.PI32), 0) == 0
        assert lib.kvc_session_chunk(s, DUMMY, 200, rows.ctypes.data_as(capi.PI32), DUMMY, 0, None) == 0
        host_view = [_reuse(lib, c, lcp) for lcp in (0, 50, 150, 200)]
        assert host_view == [0, 50, 150, 200], rewind
        cut = np.array([150], np.int32)
        assert lib.kvc_session_truncate(s, cut.ctypes.data_as(capi.PI32), 0) == 0, \
            lib.kvc_last_error().contents.message
        assert _lengths(lib, c, 1) == ([150], [150])
        # the device's bookkeeping agrees: resyncing the host copy changes nothing
        assert lib.kvc_session_sync(s) == 0
        assert [_reuse(lib, c, lcp) for lcp in (0, 50, 150)] == [0, 50, 150]
        _, pos = _snap(lib, c, 0)
        assert list(pos) == list(range(150))
        lib.kvc_session_destroy(s)


def test_reset_after_a_failed_async_call_is_suppressed_then_repeated(fake):
    """KVC_ASYNC: a reset enqueued behind a call that failed on the device is
    suppressed like the commits (it returns OK without waiting); the next
    synchronous call reports DEFERRED and restores the host's lengths and held
    rows from the device, and the repeated reset then takes effect."""
    lib = fake
    lib.kvc_test_fail_next.argtypes = [C.c_longlong]
    W, cap = 100, 256
    lay = _layer(lib, _params(lib), W)
    c = _cache(lib, lay, 1, cap, 200)
    for _ in range(2):
        assert _chunk(lib, lay, c, [200]) == 0  # 400 rows: the ring has wrapped
    before = _lengths(lib, c, 1), _snap(lib, c, 0)[1].tolist()
    lib.kvc_test_fail_next(0)
    rows = np.array([10], np.int32)
    assert lib.kvc_continue_chunk(lay, c, DUMMY, 10, rows.ctypes.data_as(capi.PI32), DUMMY, capi.KVC_ASYNC,
                                  None) == 0
    assert lib.kvc_reset(c) == 0  # suppressed on the device
    assert lib.kvc_sync(c) == capi.KVC_ERR_DEFERRED
    assert (_lengths(lib, c, 1), _snap(lib, c, 0)[1].tolist()) == before
    assert _reuse(lib, c, 150) == 0  # the held rows are the device's again
    assert lib.kvc_reset(c) == 0
    assert _lengths(lib, c, 1) == ([0], [0])
    assert _chunk(lib, lay, c, [5]) == 0
    assert _snap(lib, c, 0)[1].tolist() == list(range(5))
