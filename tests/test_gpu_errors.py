"""Rejected calls leave the cache unchanged (needs an MI355X).

Chapter 37, "Reset or reject without corrupting retained state" and its
error-evidence listing: two-token input, a full cache, model-width and
head-count mismatch, a rebuilt layer, a doubled RoPE base, one more max
position, and a finite input whose projection is not finite.  Also the
device-found errors' precedence and flat index, the deferred error of the
asynchronous mode, and a bound revision surviving reset.
"""
import numpy as np
import pytest

from incremental_kv_cache_amd import kvcache as K
from incremental_kv_cache_amd import synth

from tests.gpu_util import make_layer, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield


def _state(cache):
    ln, npos = K.kvc_lengths(cache)
    k, v = K.kvc_copy_storage(cache)
    return ln.tolist(), npos.tolist(), K.kvc_storage_pointers(cache), k.tobytes(), v.tobytes()


def _rejected_unchanged(fn, cache, want=None):
    before = _state(cache)
    with pytest.raises(K.KvcError) as e:
        fn()
    if want is not None:
        assert e.value.name == want, e.value
    assert _state(cache) == before
    return e.value


def _x(vals):
    import torch
    return torch.tensor(np.asarray(vals, np.float64).reshape(1, -1, 4), device="cuda:0")


def test_error_evidence_cases_leave_state_unchanged():
    import torch
    layer, _ = make_layer(37, 4, 2, "f64", std=0.5, max_positions=4)
    params = layer.params
    single = _x(synth.normal(37, 2, (4,)))
    # two tokens
    c = K.kvc_cache_create(layer, 1, 2)
    K.kvc_append_and_attend(layer, c, single)
    _rejected_unchanged(lambda: K.kvc_append_and_attend(layer, c, _x(synth.normal(37, 2, (8,)))), c,
                        "KVC_ERR_SINGLE_TOKEN_REQUIRED")
    # full cache (capacity 1 after one append)
    c = K.kvc_cache_create(layer, 1, 1)
    K.kvc_append_and_attend(layer, c, single)
    e = _rejected_unchanged(lambda: K.kvc_append_and_attend(layer, c, single), c, "KVC_ERR_FULL")
    assert e.detail["expected"] == 1
    # wider model
    wider, _ = make_layer(38, 8, 2, "f64", max_positions=4)
    c = K.kvc_cache_create(wider, 1, 4)
    _rejected_unchanged(lambda: K.kvc_append_and_attend(layer, c, single), c, "KVC_ERR_CACHE_MODEL_WIDTH_MISMATCH")
    # one head
    one_head, _ = make_layer(39, 4, 1, "f64", max_positions=4)
    c = K.kvc_cache_create(one_head, 1, 4)
    _rejected_unchanged(lambda: K.kvc_append_and_attend(layer, c, single), c, "KVC_ERR_CACHE_HEAD_COUNT_MISMATCH")
    # rebuilt, same-shaped and same-valued layer
    rebuilt, _ = make_layer(37, 4, 2, "f64", std=0.5, max_positions=4)
    c = K.kvc_cache_create(rebuilt, 1, 4)
    _rejected_unchanged(lambda: K.kvc_append_and_attend(layer, c, single), c, "KVC_ERR_CACHE_LAYER_MISMATCH")
    # same parameters, RoPE base doubled / one more max position
    c = K.kvc_cache_create(layer, 1, 4)
    K.kvc_append_and_attend(layer, c, single)
    doubled = K.kvc_layer_create(params, 2, K.KVC_POS_ROPE, 20000.0, 4)
    _rejected_unchanged(lambda: K.kvc_append_and_attend(doubled, c, single), c, "KVC_ERR_CACHE_ROPE_MISMATCH")
    more = K.kvc_layer_create(params, 2, K.KVC_POS_ROPE, 10000.0, 5)
    _rejected_unchanged(lambda: K.kvc_append_and_attend(more, c, single), c, "KVC_ERR_CACHE_ROPE_MISMATCH")
    # finite input whose projection is not finite
    c = K.kvc_cache_create(layer, 1, 4)
    K.kvc_append_and_attend(layer, c, single)
    big = _x([np.finfo(np.float64).max] * 4)
    e = _rejected_unchanged(lambda: K.kvc_append_and_attend(layer, c, big), c)
    assert e.name.startswith("KVC_ERR_NONFINITE_")
    # the cache still works afterwards
    out, work = K.kvc_append_and_attend(layer, c, single)
    assert work["position_min"] == 1 and np.all(np.isfinite(to_f64(out)))


def _crafted_layer(overflow):
    """Identity weights except one row of W_k or W_v that overflows for input (2, 2, 0, 0):
    row 3 (head 1, feature 1) of the chosen matrix."""
    import torch
    ws = [np.eye(4) for _ in range(3)]
    idx = {"key": 1, "value": 2}[overflow]
    ws[idx] = ws[idx].copy()
    ws[idx][3] = [1e308, 1e308, 0.0, 0.0]
    t = [torch.tensor(w, device="cuda:0") for w in ws]
    params = K.kvc_params_create(*t)
    return K.kvc_layer_create(params, 2, K.KVC_POS_NONE, 10000.0, 4)


@pytest.mark.parametrize("which", ["key", "value"])
def test_nonfinite_candidate_reports_first_flat_index(which):
    """Chapter 37 cache validation: the first non-finite flat index of the candidate key
    (then value) is reported with its value; nothing is appended."""
    layer = _crafted_layer(which)
    c = K.kvc_cache_create(layer, 1, 4)
    e = _rejected_unchanged(lambda: K.kvc_append_and_attend(layer, c, _x([2.0, 2.0, 0.0, 0.0])), c,
                            f"KVC_ERR_NONFINITE_{which.upper()}")
    assert e.detail["flat_index"] == 3 and np.isinf(e.detail["value"])


def test_async_failure_is_deferred_and_blocks_commits():
    """KVC_ASYNC: a device-found failure returns OK at enqueue, suppresses every later
    commit and length change, and the next synchronous call reports KVC_ERR_DEFERRED."""
    layer = _crafted_layer("value")
    c = K.kvc_cache_create(layer, 1, 4)
    good = _x([0.1, 0.2, 0.3, 0.4])
    K.kvc_append_and_attend(layer, c, good)
    before = _state(c)
    K.kvc_append_and_attend(layer, c, _x([2.0, 2.0, 0.0, 0.0]), flags=K.KVC_ASYNC)   # fails on device
    K.kvc_append_and_attend(layer, c, good, flags=K.KVC_ASYNC)                       # suppressed
    K.kvc_truncate(c, [1])                                                            # suppressed
    with pytest.raises(K.KvcError) as e:
        K.kvc_sync(c)
    assert e.value.name == "KVC_ERR_DEFERRED"
    assert e.value.detail["actual"] == K.capi.KVC_ERR_NONFINITE_VALUE
    assert _state(c) == before
    out, work = K.kvc_append_and_attend(layer, c, good)
    assert work["position_min"] == 1


def test_revision_mismatch_survives_reset_and_bad_cut():
    import torch
    layer, _ = make_layer(37, 4, 2, "f64", std=0.5, max_positions=4)
    c = K.kvc_cache_create(layer, 1, 4)
    x = torch.zeros(1, 1, 4, dtype=torch.float64, device="cuda:0")
    K.kvc_append_and_attend(layer, c, x)
    _rejected_unchanged(lambda: K.kvc_truncate(c, [2]), c, "KVC_ERR_BAD_CUT")
    K.kvc_params_mark_updated(layer.params, 0)
    e = _rejected_unchanged(lambda: K.kvc_append_and_attend(layer, c, x), c, "KVC_ERR_CACHE_LAYER_REVISION_MISMATCH")
    assert e.detail["parameter"] == 0
    K.kvc_reset(c)
    _rejected_unchanged(lambda: K.kvc_append_and_attend(layer, c, x), c, "KVC_ERR_CACHE_LAYER_REVISION_MISMATCH")
    fresh = K.kvc_cache_create(layer, 1, 4)
    K.kvc_append_and_attend(layer, fresh, x)


def test_stream_read_probe_reads_the_buffer():
    """The bandwidth probe reads every unit: a buffer whose first thread's words xor to
    the probe's marker makes it store the marker; an all-zero buffer leaves the sink."""
    import torch
    buf = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    K.kvc_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [0, 0, 0, 0]
    marker = np.array([0x9E3779B9], dtype=np.uint32).view(np.int32)[0]
    buf[(1 << 20) - 8192] = int(marker)  # first word of the last 32 KiB unit
    K.kvc_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [int(marker), 0, 0, 0]
