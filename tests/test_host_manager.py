"""Host cache manager on the CPU: validation order, binding, truncate/reset bookkeeping.

The manager (incremental_kv_cache_amd/csrc/kvc_host.cpp) is linked here against
tests/hostcheck_backend.cpp, a stand-in backend whose "device" memory is host
memory and which cannot run kernels.  Every request that passes validation
therefore stops with KVC_ERR_DEVICE at the launch point, which is how these
tests see that validation let it through.  The checks follow Chapter 37's
order ("Bind the state, calculate completely, then commit") and its
error-evidence cases.
"""
import ctypes as C

import numpy as np
import pytest

from incremental_kv_cache_amd import capi
from tests import hostcheck



@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    return hostcheck.build(tmp_path_factory, "hostcheck")


DUMMY = C.c_void_p(64)


def params(lib, d=4, dtype=capi.KVC_F64, wo=False):
    p = C.c_void_p()
    assert lib.kvc_params_create(d, dtype, DUMMY, DUMMY, DUMMY, DUMMY if wo else None, C.byref(p)) == 0
    return p


def layer(lib, p, heads=2, base=10000.0, max_pos=4, mode=capi.KVC_POS_ROPE):
    l = C.c_void_p()
    assert lib.kvc_layer_create(p, heads, mode, base, max_pos, C.byref(l)) == 0
    return l


def cache(lib, l, batch=1, cap=4, chunk=1):
    c = C.c_void_p()
    st = lib.kvc_cache_create(l, batch, cap, chunk, None, C.byref(c))
    assert st == 0, lib.kvc_last_error().contents.message
    return c


def append(lib, l, c, shape):
    arr = (C.c_int64 * len(shape))(*shape)
    w = capi.Work()
    return lib.kvc_append_and_attend(l, c, DUMMY, len(shape), arr, DUMMY, 0, C.byref(w))


def state(lib, c, batch=1):
    ln = np.zeros(batch, np.int32)
    npos = np.zeros(batch, np.int32)
    assert lib.kvc_lengths(c, ln.ctypes.data_as(capi.PI32), npos.ctypes.data_as(capi.PI32)) == 0
    k = C.c_void_p()
    v = C.c_void_p()
    n = C.c_int64()
    assert lib.kvc_storage_pointers(c, C.byref(k), C.byref(v), C.byref(n)) == 0
    kb = np.zeros(n.value, np.uint8)
    vb = np.zeros(n.value, np.uint8)
    assert lib.kvc_copy_storage(c, kb.ctypes.data_as(C.c_void_p), vb.ctypes.data_as(C.c_void_p)) == 0
    return ln.tolist(), npos.tolist(), k.value, v.value, kb.tobytes(), vb.tobytes()


def test_create_geometry_and_zeroed_storage(lib):
    p = params(lib)
    l = layer(lib, p)
    c = cache(lib, l, batch=3, cap=4, chunk=2)
    d = capi.CacheDesc()
    assert lib.kvc_cache_describe(c, C.byref(d)) == 0
    assert (d.batch, d.heads, d.head_width, d.model_width, d.capacity, d.max_chunk_rows) == (3, 2, 2, 4, 4, 2)
    ln, npos, kp, vp, kb, vb = state(lib, c, 3)
    assert ln == [0, 0, 0] and npos == [0, 0, 0]
    assert len(kb) == 3 * 2 * 4 * 2 * 8 and set(kb) == {0} and set(vb) == {0}
    lib.kvc_cache_destroy(c)


def test_create_checks_in_order(lib):
    """Chapter 37 constructor: zero batch, zero capacity, capacity over position capacity, overflow."""
    p = params(lib)
    l = layer(lib, p, max_pos=4)
    c = C.c_void_p()
    assert lib.kvc_cache_create(l, 0, 0, 1, None, C.byref(c)) == capi.KVC_ERR_ZERO_BATCH
    assert lib.kvc_cache_create(l, 1, 0, 1, None, C.byref(c)) == capi.KVC_ERR_ZERO_CAPACITY
    assert lib.kvc_cache_create(l, 1, 5, 1, None, C.byref(c)) == capi.KVC_ERR_CAPACITY_EXCEEDS_POSITIONS
    assert lib.kvc_cache_create(l, 1, 4, 0, None, C.byref(c)) == capi.KVC_ERR_BAD_ARGUMENT
    big = layer(lib, params(lib, d=128, dtype=capi.KVC_BF16), heads=1, max_pos=2 ** 31 - 1)
    assert lib.kvc_cache_create(big, 2 ** 31 - 1, 2 ** 31 - 1, 1, None, C.byref(c)) == \
        capi.KVC_ERR_ELEMENT_COUNT_OVERFLOW
    assert b"too large to index" in lib.kvc_last_error().contents.message


def test_request_checks_follow_the_chapter_order_and_leave_state_unchanged(lib):
    """Rank, one token, batch, width, binding, capacity -- each rejection leaves the
    cache's lengths, allocation and storage as they were."""
    p = params(lib)
    l = layer(lib, p)
    c = cache(lib, l)
    before = state(lib, c)
    cases = [
        ((1, 4), capi.KVC_ERR_INPUT_RANK),              # rank first, even with other faults
        ((2, 2, 8), capi.KVC_ERR_SINGLE_TOKEN_REQUIRED),  # two-token input (error evidence)
        ((2, 1, 8), capi.KVC_ERR_INPUT_BATCH_MISMATCH),
        ((1, 1, 8), capi.KVC_ERR_INPUT_WIDTH_MISMATCH),
    ]
    for shape, want in cases:
        assert append(lib, l, c, shape) == want, shape
        d = lib.kvc_last_error().contents
        assert d.status == want
        if want == capi.KVC_ERR_INPUT_WIDTH_MISMATCH:
            assert (d.expected, d.actual) == (4, 8)
        assert state(lib, c) == before
    # a valid request passes every host check and reaches the (absent) device
    assert append(lib, l, c, (1, 1, 4)) == capi.KVC_ERR_DEVICE
    assert state(lib, c) == before


def test_binding_cases_of_the_error_evidence(lib):
    """Chapter 37 error evidence: model-width mismatch, head mismatch, rebuilt layer,
    doubled RoPE base, one more max position; plus the in-place update case."""
    p = params(lib)
    l = layer(lib, p)
    x = (1, 1, 4)
    wider = layer(lib, params(lib, d=8), heads=2)
    c = cache(lib, wider)
    assert append(lib, l, c, x) == capi.KVC_ERR_CACHE_MODEL_WIDTH_MISMATCH
    one_head = layer(lib, params(lib, d=4), heads=1)
    c = cache(lib, one_head)
    assert append(lib, l, c, x) == capi.KVC_ERR_CACHE_HEAD_COUNT_MISMATCH
    rebuilt = layer(lib, params(lib))                 # same shapes, new parameter identity
    c = cache(lib, rebuilt)
    assert append(lib, l, c, x) == capi.KVC_ERR_CACHE_LAYER_MISMATCH
    c = cache(lib, l)
    doubled = layer(lib, p, base=20000.0)             # same parameters, different rotary base
    assert append(lib, doubled, c, x) == capi.KVC_ERR_CACHE_ROPE_MISMATCH
    d = lib.kvc_last_error().contents
    assert tuple(d.rope_base) == (10000.0, 20000.0)
    more = layer(lib, p, max_pos=5)
    assert append(lib, more, c, x) == capi.KVC_ERR_CACHE_ROPE_MISMATCH
    assert tuple(lib.kvc_last_error().contents.rope_max_positions) == (4, 5)
    none_mode = layer(lib, p, mode=capi.KVC_POS_NONE)
    assert append(lib, none_mode, c, x) == capi.KVC_ERR_CACHE_ROPE_MISMATCH
    # in-place update of W_v: identity kept, revision advanced; reset does not rebind
    assert lib.kvc_params_mark_updated(p, 2) == 0
    assert append(lib, l, c, x) == capi.KVC_ERR_CACHE_LAYER_REVISION_MISMATCH
    d = lib.kvc_last_error().contents
    assert (d.parameter, d.cache_revision, d.layer_revision) == (2, 0, 1)
    assert lib.kvc_reset(c) == 0
    assert append(lib, l, c, x) == capi.KVC_ERR_CACHE_LAYER_REVISION_MISMATCH
    fresh = cache(lib, l)                             # a new cache binds the new revision
    assert append(lib, l, fresh, x) == capi.KVC_ERR_DEVICE


def test_output_projection_is_a_bound_parameter(lib):
    """W_o is the fourth bound weight: its in-place update is reported as parameter 3;
    a set without W_o has only three weights to update."""
    p = params(lib, wo=True)
    l = layer(lib, p)
    c = cache(lib, l)
    assert append(lib, l, c, (1, 1, 4)) == capi.KVC_ERR_DEVICE
    assert lib.kvc_params_mark_updated(p, 3) == 0
    assert append(lib, l, c, (1, 1, 4)) == capi.KVC_ERR_CACHE_LAYER_REVISION_MISMATCH
    d = lib.kvc_last_error().contents
    assert (d.parameter, d.cache_revision, d.layer_revision) == (3, 0, 1)
    q = params(lib)
    assert lib.kvc_params_mark_updated(q, 3) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_params_mark_updated(q, -1) == 0


def test_binding_precedes_shape_of_geometry(lib):
    """Width mismatch of the *input* is checked before any cache binding check."""
    p = params(lib)
    l = layer(lib, p)
    other = cache(lib, layer(lib, params(lib)))
    assert append(lib, l, other, (1, 1, 3)) == capi.KVC_ERR_INPUT_WIDTH_MISMATCH
    assert append(lib, l, other, (1, 1, 4)) == capi.KVC_ERR_CACHE_LAYER_MISMATCH


def test_truncate_reset_and_snapshot_bookkeeping(lib):
    p = params(lib)
    l = layer(lib, p)
    c = cache(lib, l, batch=2)
    cut = np.array([0, 1], np.int32)
    assert lib.kvc_truncate(c, cut.ctypes.data_as(capi.PI32), 0) == capi.KVC_ERR_BAD_CUT
    d = lib.kvc_last_error().contents
    assert (d.sequence, d.expected, d.actual) == (1, 0, 1)
    cut = np.array([-1, 0], np.int32)
    assert lib.kvc_truncate(c, cut.ctypes.data_as(capi.PI32), 0) == capi.KVC_ERR_BAD_CUT
    cut = np.array([0, 0], np.int32)
    assert lib.kvc_truncate(c, cut.ctypes.data_as(capi.PI32), 4) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_truncate(c, cut.ctypes.data_as(capi.PI32), 0) == 0
    assert lib.kvc_truncate(c, cut.ctypes.data_as(capi.PI32), capi.KVC_TRUNCATE_KEEP_STALE_POSITION) == 0
    before = state(lib, c, 2)
    assert lib.kvc_reset(c) == 0
    after = state(lib, c, 2)
    assert after == before                            # same pointers and bytes
    rows = C.c_int32()
    assert lib.kvc_snapshot(c, 1, None, None, None, 0, C.byref(rows)) == 0 and rows.value == 0
    assert lib.kvc_snapshot(c, 2, None, None, None, 0, C.byref(rows)) == capi.KVC_ERR_BAD_ARGUMENT


def test_chunk_checks(lib):
    p = params(lib)
    l = layer(lib, p, max_pos=8)
    c = cache(lib, l, batch=2, cap=4, chunk=6)
    w = capi.Work()
    assert lib.kvc_continue_chunk(l, c, DUMMY, 7, None, DUMMY, 0, C.byref(w)) == capi.KVC_ERR_CHUNK_ROWS
    assert lib.kvc_continue_chunk(l, c, DUMMY, 0, None, DUMMY, 0, C.byref(w)) == capi.KVC_ERR_CHUNK_ROWS
    rows = np.array([2, 3], np.int32)
    assert lib.kvc_continue_chunk(l, c, DUMMY, 2, rows.ctypes.data_as(capi.PI32), DUMMY, 0,
                                  C.byref(w)) == capi.KVC_ERR_CHUNK_ROWS
    assert lib.kvc_last_error().contents.sequence == 1
    assert lib.kvc_continue_chunk(l, c, DUMMY, 5, None, DUMMY, 0, C.byref(w)) == capi.KVC_ERR_FULL
    rows = np.array([0, 0], np.int32)                 # nothing to do: OK with zero work
    assert lib.kvc_continue_chunk(l, c, DUMMY, 3, rows.ctypes.data_as(capi.PI32), DUMMY, 0, C.byref(w)) == 0
    assert w.incremental_rows_per_projection == 0
    assert lib.kvc_continue_chunk(l, c, DUMMY, 4, None, DUMMY, 0, C.byref(w)) == capi.KVC_ERR_DEVICE
    other = layer(lib, params(lib), max_pos=8)
    assert lib.kvc_continue_chunk(other, c, DUMMY, 2, None, DUMMY, 0, C.byref(w)) == capi.KVC_ERR_CACHE_LAYER_MISMATCH


def test_null_arguments(lib):
    assert lib.kvc_reset(None) == capi.KVC_ERR_NULL_ARGUMENT
    assert lib.kvc_sync(None) == capi.KVC_ERR_NULL_ARGUMENT
    assert lib.kvc_truncate(None, None, 0) == capi.KVC_ERR_NULL_ARGUMENT
    assert lib.kvc_append_and_attend(None, None, None, 3, None, None, 0, None) == capi.KVC_ERR_NULL_ARGUMENT
    out = C.c_int64()
    assert lib.kvc_lcp_cut(None, 2, None, 1, C.byref(out)) == capi.KVC_ERR_NULL_ARGUMENT


def test_stream_read_argument_checks(lib):
    """The bandwidth and matrix-core probes check their arguments on the host before any launch."""
    buf = C.c_void_p(4096)
    sink = C.c_void_p(8192)
    assert lib.kvc_stream_read(None, 32768, sink, None) == capi.KVC_ERR_NULL_ARGUMENT
    assert lib.kvc_stream_read(buf, 32768, None, None) == capi.KVC_ERR_NULL_ARGUMENT
    assert lib.kvc_stream_read(buf, 0, sink, None) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_stream_read(buf, 32768 + 16, sink, None) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_stream_read(C.c_void_p(4100), 32768, sink, None) == capi.KVC_ERR_BAD_ARGUMENT
    d = lib.kvc_last_error().contents
    assert (d.expected, d.actual) == (32768, 32768)
    assert lib.kvc_stream_read(buf, 65536, sink, None) == capi.KVC_ERR_DEVICE  # host-check library: no kernels
    flops = C.c_double()
    assert lib.kvc_mfma_rate(100, None, None, C.byref(flops)) == capi.KVC_ERR_NULL_ARGUMENT
    assert lib.kvc_mfma_rate(100, sink, None, None) == capi.KVC_ERR_NULL_ARGUMENT
    assert lib.kvc_mfma_rate(0, sink, None, C.byref(flops)) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_mfma_rate((1 << 24) + 1, sink, None, C.byref(flops)) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_mfma_rate(100, sink, None, C.byref(flops)) == capi.KVC_ERR_DEVICE


def _i32(v):
    a = np.ascontiguousarray(np.asarray(v, dtype=np.int32))
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def test_chunk_work_order_lists_every_item_heaviest_first(lib):
    """The chunk attention's work order: every (sequence, 256-row query tile) with
    rows appears once, the keys its last query reads never increase along the
    list, and equal loads keep sequence order."""
    tile = 256  # chunk rows per work item of the bf16 chunk attention
    lens, rows, n_max = [10, 500, 0, 37, 200], [600, 1, 0, 257, 512], 600
    la, lp = _i32(lens)
    ra, rp = _i32(rows)
    items = np.zeros(256, np.int32)
    qt = C.c_int32()
    n = lib.kvc_test_chunk_order(5, n_max, lp, rp, C.byref(qt), items.ctypes.data_as(C.POINTER(C.c_int32)))
    assert qt.value == 3
    got = [(int(i) >> 16, int(i) & 0xFFFF) for i in items[:n]]
    want = {(b, q) for b in range(5) for q in range(3) if q * tile < rows[b]}
    assert len(got) == len(want) and set(got) == want
    keys = [lens[b] + min(rows[b], tile * (q + 1)) for b, q in got]
    assert all(keys[k] >= keys[k + 1] for k in range(len(keys) - 1))
    for k in range(len(keys) - 1):
        if keys[k] == keys[k + 1]:
            assert got[k] < got[k + 1]
    # no per-sequence rows: every sequence has n_max rows
    n2 = lib.kvc_test_chunk_order(2, tile + 2, lp, None, C.byref(qt), items.ctypes.data_as(C.POINTER(C.c_int32)))
    assert n2 == 4 and qt.value == 2
    # more items than the table holds: natural order (count 0)
    big, bp = _i32(np.arange(300))
    assert lib.kvc_test_chunk_order(300, 1, bp, None, C.byref(qt), items.ctypes.data_as(C.POINTER(C.c_int32))) == 0


def test_decode_sequence_order_longest_first(lib):
    """The decode attention's sequence order: most retained rows first, ties in
    sequence order, dealt in rounds of per_round sequences with every other
    round reversed (a unit that takes a long lane in one round takes a short one
    in the next); a batch larger than the table keeps sequence order."""
    la, lp = _i32([3, 9, 9, 0, 4])
    seq = np.zeros(256, np.int32)
    sp = seq.ctypes.data_as(C.POINTER(C.c_int32))
    for per_round in (1, 5, 8):
        assert lib.kvc_test_seq_order(5, lp, per_round, sp) == 5 and list(seq[:5]) == [1, 2, 4, 0, 3]
    assert lib.kvc_test_seq_order(5, lp, 2, sp) == 5 and list(seq[:5]) == [1, 2, 0, 4, 3]
    # 32 sequences in rounds of 8 (32 heads on 256 units): rank sums per unit even out
    lens = np.random.default_rng(5).permutation(np.arange(1, 33) * 100)
    _, lp32 = _i32(lens)
    assert lib.kvc_test_seq_order(32, lp32, 8, sp) == 32
    ranks = np.argsort(np.argsort(-lens))[seq[:32]]
    assert list(ranks) == list(range(8)) + list(range(15, 7, -1)) + list(range(16, 24)) + list(range(31, 23, -1))
    assert len({int(ranks[k] + ranks[8 + k] + ranks[16 + k] + ranks[24 + k]) for k in range(8)}) == 1
    big, bp = _i32(np.arange(300))
    assert lib.kvc_test_seq_order(300, bp, 8, sp) == 0


# ------------------------------------------------------------- session ----

def session(lib, layers, vocab=10, pe=capi.KVC_PE_SINUSOIDAL, batch=2, cap=4, chunk=4):
    arr = (C.c_void_p * max(1, len(layers)))(*layers)
    s = C.c_void_p()
    st = lib.kvc_session_create(arr, len(layers), DUMMY, vocab, pe, batch, cap, chunk, None, C.byref(s))
    return st, s


def test_session_create_checks_and_names_the_layer(lib):
    """Session construction: null arguments, counts, encoding, layers of other width,
    then each layer's cache construction with detail.layer naming the layer."""
    p = params(lib)
    l0, l1 = layer(lib, p), layer(lib, p, max_pos=4)
    assert lib.kvc_session_create(None, 1, DUMMY, 10, 1, 1, 4, 1, None, C.byref(C.c_void_p())) == \
        capi.KVC_ERR_NULL_ARGUMENT
    assert session(lib, [])[0] == capi.KVC_ERR_BAD_ARGUMENT
    assert session(lib, [l0], vocab=0)[0] == capi.KVC_ERR_BAD_ARGUMENT
    assert session(lib, [l0], pe=7)[0] == capi.KVC_ERR_BAD_ARGUMENT
    st, _ = session(lib, [l0, None])
    assert st == capi.KVC_ERR_NULL_ARGUMENT and lib.kvc_last_error().contents.layer == 1
    wide = layer(lib, params(lib, d=8))
    st, _ = session(lib, [l0, wide])
    assert st == capi.KVC_ERR_BAD_ARGUMENT and lib.kvc_last_error().contents.layer == 1
    short = layer(lib, p, max_pos=3)
    st, _ = session(lib, [l0, l1, short])
    d = lib.kvc_last_error().contents
    assert st == capi.KVC_ERR_CAPACITY_EXCEEDS_POSITIONS and d.layer == 2 and (d.expected, d.actual) == (3, 4)
    st, s = session(lib, [l0, l1])
    assert st == capi.KVC_OK
    lib.kvc_session_destroy(s)


def test_session_layer_caches_are_read_only_views(lib):
    """A session's layer cache answers the read-only calls but refuses compute,
    truncate and reset (every layer must move together), and destroying it is a no-op."""
    p = params(lib)
    l0, l1 = layer(lib, p), layer(lib, p)
    st, s = session(lib, [l0, l1])
    assert st == 0
    c = C.c_void_p()
    assert lib.kvc_session_layer_cache(s, 2, C.byref(c)) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_session_layer_cache(s, 1, C.byref(c)) == 0
    cut, cp = np.zeros(2, np.int32), None
    cp = cut.ctypes.data_as(capi.PI32)
    assert lib.kvc_truncate(c, cp, 0) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_reset(c) == capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_continue_chunk(l1, c, DUMMY, 1, None, DUMMY, 0, None) == capi.KVC_ERR_BAD_ARGUMENT
    assert append(lib, l1, c, [2, 1, 4]) == capi.KVC_ERR_BAD_ARGUMENT
    assert state(lib, c, batch=2)[:2] == ([0, 0], [0, 0])
    lib.kvc_cache_destroy(c)  # ignored: the session owns it
    assert lib.kvc_lengths(c, None, None) == 0
    lib.kvc_session_destroy(s)


def test_session_request_checks(lib):
    """Session calls check rows, each layer's binding in layer order (detail.layer),
    then cuts; a valid request reaches the launch point (the host-check library has no kernels)."""
    p0, p1 = params(lib), params(lib)
    l0, l1 = layer(lib, p0), layer(lib, p1)
    st, s = session(lib, [l0, l1])
    assert st == 0
    w = capi.Work()
    assert lib.kvc_session_chunk(s, DUMMY, 0, None, DUMMY, 0, C.byref(w)) == capi.KVC_ERR_CHUNK_ROWS
    assert lib.kvc_session_chunk(s, DUMMY, 5, None, DUMMY, 0, C.byref(w)) == capi.KVC_ERR_CHUNK_ROWS
    rows = np.array([1, 3], np.int32)
    assert lib.kvc_session_chunk(s, DUMMY, 2, rows.ctypes.data_as(capi.PI32), DUMMY, 0, C.byref(w)) == \
        capi.KVC_ERR_CHUNK_ROWS
    assert lib.kvc_session_decode(s, DUMMY, DUMMY, 0, C.byref(w)) == capi.KVC_ERR_DEVICE
    assert lib.kvc_session_decode(s, None, DUMMY, 0, C.byref(w)) == capi.KVC_ERR_NULL_ARGUMENT
    assert lib.kvc_params_mark_updated(p1, 1) == 0
    assert lib.kvc_session_decode(s, DUMMY, DUMMY, 0, C.byref(w)) == capi.KVC_ERR_CACHE_LAYER_REVISION_MISMATCH
    d = lib.kvc_last_error().contents
    assert d.layer == 1 and d.parameter == 1
    cut = np.array([1, 0], np.int32)
    assert lib.kvc_session_truncate(s, cut.ctypes.data_as(capi.PI32), 0) == capi.KVC_ERR_BAD_CUT
    assert lib.kvc_last_error().contents.layer == 0
    cut[:] = 0
    assert lib.kvc_session_truncate(s, cut.ctypes.data_as(capi.PI32), 0) == 0
    assert lib.kvc_session_reset(s) == 0
    lib.kvc_session_destroy(s)


def test_grouped_parameters_layers_and_caches(lib):
    """Grouped key/value heads (Chapter 37, "From causal attention to managed LLM
    inference state": multi-query attention against the K/V reload bottleneck):
    W_k / W_v are [kv_width, D]; the layer has kv_width / d_h key/value heads,
    which must divide the query heads; the cache keeps [B, H_kv, C, d_h]; a
    layer with another key/value head count does not bind to the cache."""
    p = C.c_void_p()
    assert lib.kvc_params_create_grouped(8, 3, capi.KVC_F64, DUMMY, DUMMY, DUMMY, None, C.byref(p)) == \
        capi.KVC_ERR_BAD_ARGUMENT  # 3 does not divide 8
    assert lib.kvc_params_create_grouped(8, 0, capi.KVC_F64, DUMMY, DUMMY, DUMMY, None, C.byref(p)) == \
        capi.KVC_ERR_BAD_ARGUMENT
    assert lib.kvc_params_create_grouped(8, 4, capi.KVC_F64, DUMMY, DUMMY, DUMMY, None, C.byref(p)) == 0
    l = C.c_void_p()
    # 4 heads of width 2: 2 key/value heads
    assert lib.kvc_layer_create(p, 4, capi.KVC_POS_ROPE, 10000.0, 8, C.byref(l)) == 0
    # 1 head of width 8: the key/value width 4 is not a whole head
    bad = C.c_void_p()
    assert lib.kvc_layer_create(p, 1, capi.KVC_POS_ROPE, 10000.0, 8, C.byref(bad)) == capi.KVC_ERR_BAD_ARGUMENT
    p6 = C.c_void_p()
    assert lib.kvc_params_create_grouped(12, 6, capi.KVC_F64, DUMMY, DUMMY, DUMMY, None, C.byref(p6)) == 0
    # 3 heads of width 4 cannot share 6 / 4 heads; 6 heads of width 2 share 3 key/value heads
    assert lib.kvc_layer_create(p6, 3, capi.KVC_POS_ROPE, 10000.0, 8, C.byref(bad)) == capi.KVC_ERR_BAD_ARGUMENT
    c = cache(lib, l, batch=3, cap=4, chunk=2)
    d = capi.CacheDesc()
    assert lib.kvc_cache_describe(c, C.byref(d)) == 0
    assert (d.heads, d.kv_heads, d.head_width) == (4, 2, 2)
    *_, kb, vb = state(lib, c, 3)
    assert len(kb) == 3 * 2 * 4 * 2 * 8  # [B, H_kv, C, d_h] float64
    n = C.c_int32()
    assert lib.kvc_snapshot(c, 0, None, None, None, 0, C.byref(n)) == 0 and n.value == 0
    # the same query heads over the full key/value width: the head check comes first
    full = layer(lib, params(lib, d=8), heads=4, max_pos=8)
    assert append(lib, full, c, (3, 1, 8)) == capi.KVC_ERR_CACHE_HEAD_COUNT_MISMATCH
    e = lib.kvc_last_error().contents
    assert (e.expected, e.actual) == (4, 2)
    pf = params(lib, d=8)
    lf = layer(lib, pf, heads=4, max_pos=8)
    cf = cache(lib, lf, batch=3, cap=4)
    assert append(lib, l, cf, (3, 1, 8)) == capi.KVC_ERR_CACHE_HEAD_COUNT_MISMATCH
    e = lib.kvc_last_error().contents
    assert (e.expected, e.actual) == (2, 4)
    for h in (c, cf):
        lib.kvc_cache_destroy(h)
