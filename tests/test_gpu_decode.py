"""Decode-step parity through the C ABI against the float64 oracle (needs an MI355X).

Covers the chapter's worked trace, the fixture-size seeded workload, reset and
replay evidence, multi-tile ragged lengths in float64 / float32 / bf16, and the
stored cache state and row counts after every step.
"""
import math

import numpy as np
import pytest

from incremental_kv_cache_amd import kvcache as K
from incremental_kv_cache_amd import synth
from oracle import attention as A
from oracle import prefix as P

from tests.gpu_util import assert_parity, hidden, make_layer, storage_f64, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield


def _trace_fixture():
    x = np.array([[1.0, 0.0, 1.0, 0.0],
                  [math.cos(1.0), -math.sin(1.0), 0.0, 1.0],
                  [math.cos(2.0), -math.sin(2.0), 1.0, 1.0]])
    return x


def _identity_layer(max_positions=4, base=10000.0, params=None):
    import torch
    if params is None:
        eye = [torch.eye(4, dtype=torch.float64, device="cuda:0") for _ in range(3)]
        params = K.kvc_params_create(*eye)
    return K.kvc_layer_create(params, 2, K.KVC_POS_ROPE, base, max_positions)


def _run_trace(layer, cache, x):
    import torch
    outs, works, snaps = [], [], []
    for p in range(3):
        xt = torch.tensor(x[p][None, None, :], dtype=torch.float64, device="cuda:0")
        out, work = K.kvc_append_and_attend(layer, cache, xt)
        outs.append(to_f64(out)[0, 0])
        works.append(work)
        snaps.append(K.kvc_snapshot(cache, 0))
    return outs, works, snaps


def test_chapter_trace_through_the_library():
    """Chapter 37 trace ('Advance the layer cache one position at a time'): printed outputs
    (9 d.p., after the fixture's block-swapping output projection, which this library
    leaves to the caller), printed rotated keys and values, positions, row counts; and
    cached == full-prefix oracle within 1e-12."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p2_trace.json")))
    x = _trace_fixture()
    layer = _identity_layer()
    cache = K.kvc_cache_create(layer, 1, 4)
    outs, works, snaps = _run_trace(layer, cache, x)
    eye = np.eye(4)
    for p, step in enumerate(g["steps"]):
        merged = outs[p]
        printed = np.array(step["output"])
        np.testing.assert_allclose(np.concatenate([merged[2:], merged[:2]]), printed, rtol=0, atol=5.1e-10)
        ref = A.full_prefix_decode(x[: p + 1], eye, eye, eye, heads=2)
        assert np.max(np.abs(merged - ref["out"])) <= 1e-12
        k, v, pos = snaps[p]
        assert k.shape == (2, p + 1, 2) and list(pos) == list(range(p + 1))
        for h, head in enumerate(step["heads"]):
            np.testing.assert_allclose(k[h], head["keys"], rtol=0, atol=5.1e-10)
            np.testing.assert_allclose(v[h], head["values"], rtol=0, atol=5.1e-10)
        assert works[p]["position_min"] == p == works[p]["position_max"]
    assert sum(w["full_prefix_rows_per_projection"] for w in works) == g["work"]["full_rows_per_projection"]
    assert sum(w["incremental_rows_per_projection"] for w in works) == g["work"]["incremental_rows_per_projection"]
    assert sum(w["reused_key_value_rows"] for w in works) == g["work"]["reused_rows_per_kv_projection"]


def test_chapter_trace_weights_read_out_of_the_library():
    """The trace's newest-query weights of each head (12 d.p.) after every step, read
    from the library (kvc_newest_weights recomputes them on the device from the
    step's rotated query and the stored keys); any later call that moves the cache
    ends the readout."""
    import json
    import os
    import torch
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p2_trace.json")))
    x = _trace_fixture()
    layer = _identity_layer()
    cache = K.kvc_cache_create(layer, 1, 4)
    for p, step in enumerate(g["steps"]):
        xt = torch.tensor(x[p][None, None, :], dtype=torch.float64, device="cuda:0")
        K.kvc_append_and_attend(layer, cache, xt)
        w = to_f64(K.kvc_newest_weights(cache, 0))
        assert w.shape == (2, p + 1)
        for h, head in enumerate(step["heads"]):
            np.testing.assert_allclose(w[h], head["weights"], rtol=0, atol=5.1e-13)
    K.kvc_truncate(cache, [2])
    with pytest.raises(K.KvcError) as e:
        K.kvc_newest_weights(cache, 0)
    assert e.value.name == "KVC_ERR_BAD_ARGUMENT"


def test_newest_weights_match_the_oracle_in_every_type():
    """Ragged lengths, several heads: the readout equals the oracle's weights of the
    newest row (float64 1e-12; float32 and bf16 storage within their bars)."""
    import torch
    for dtype in ("f64", "f32", "bf16"):
        B, H, dh, lens = 3, 4, 64, [0, 37, 300]
        D = H * dh
        layer, w = make_layer(17, D, H, dtype, max_positions=512)
        cache = K.kvc_cache_create(layer, B, 512, max_chunk_rows=max(lens))
        xp_dev, xp = hidden(17, synth.STREAM_PREFIX_X, B, max(lens), D, dtype)
        K.kvc_continue_chunk(layer, cache, xp_dev, n_rows=lens)
        xn_dev, xn = hidden(17, synth.STREAM_X, B, 1, D, dtype)
        K.kvc_append_and_attend(layer, cache, xn_dev)
        for b in range(B):
            got = to_f64(K.kvc_newest_weights(cache, b))
            rows = np.concatenate([xp[b, : lens[b]], xn[b]])
            ref = A.causal_layer(rows, *w, heads=H, rows=[lens[b]])["weights"][0]
            assert got.shape == ref.shape == (H, lens[b] + 1)
            tol = {"f64": 1e-12, "f32": 1e-5, "bf16": 2e-2}[dtype]
            assert float(np.max(np.abs(got - ref))) <= tol, (dtype, b)
            np.testing.assert_allclose(got.sum(axis=1), 1.0, rtol=0, atol=1e-6)
        torch.cuda.synchronize()


def test_reset_reuses_allocation_and_replays_identically():
    """Chapter 37 reset evidence: 3 -> 0, allocation reused, storage unchanged, replay identical."""
    x = _trace_fixture()
    layer = _identity_layer()
    cache = K.kvc_cache_create(layer, 1, 4)
    outs, works, snaps = _run_trace(layer, cache, x)
    ln, _ = K.kvc_lengths(cache)
    assert ln.tolist() == [3]
    ptrs = K.kvc_storage_pointers(cache)
    store = K.kvc_copy_storage(cache)
    K.kvc_reset(cache)
    assert K.kvc_lengths(cache)[0].tolist() == [0] and K.kvc_lengths(cache)[1].tolist() == [0]
    assert K.kvc_storage_pointers(cache) == ptrs
    after = K.kvc_copy_storage(cache)
    assert np.array_equal(after[0], store[0]) and np.array_equal(after[1], store[1])
    outs2, works2, snaps2 = _run_trace(layer, cache, x)
    for a, b in zip(outs, outs2):
        assert np.array_equal(a, b)
    assert works == works2
    for (k1, v1, p1), (k2, v2, p2) in zip(snaps, snaps2):
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2) and np.array_equal(p1, p2)


@pytest.mark.parametrize("seed", [37, 7, 11, 23])
def test_fixture_size_seeded_decode(seed):
    """Fixture-size workload: B=1, D=4, H=2, d_h=2, C=4, W ~ N(0, 1/4), one row per call.
    The first call returns its own value row exactly; every call equals the float64
    full-prefix recompute within 1e-12; the stored rows match the oracle's."""
    import torch
    layer, w = make_layer(seed, 4, 2, "f64", std=0.5, max_positions=4)
    cache = K.kvc_cache_create(layer, 1, 4)
    x = synth.normal(seed, synth.STREAM_X, (4, 4))
    for p in range(4):
        out, work = K.kvc_append_and_attend(layer, cache, torch.tensor(x[p][None, None], device="cuda:0"))
        o = to_f64(out)[0, 0]
        ref = A.full_prefix_decode(x[: p + 1], *w, heads=2)
        assert np.max(np.abs(o - ref["out"])) <= 1e-12
        assert work == {**P.decode_work([p]), "position_min": p, "position_max": p}
        k, v, pos = K.kvc_snapshot(cache, 0)
        if p == 0:
            # single retained key: weight exactly 1, output is the stored value row
            assert np.array_equal(o, np.concatenate([v[0, 0], v[1, 0]]))
        np.testing.assert_allclose(k, ref["keys"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(v, ref["values"], rtol=0, atol=1e-13)
    with pytest.raises(K.KvcError) as e:
        K.kvc_append_and_attend(layer, cache, torch.tensor(x[0][None, None], device="cuda:0"))
    assert e.value.name == "KVC_ERR_FULL"


def _decode_case(dtype, B, H, dh, lens, steps, seed, chunk_rows=512):
    """Prefill ragged prefixes through continue_chunk, then `steps` single-row decodes;
    each decode output and the final cache are compared with the float64 oracle."""
    D = H * dh
    cap = max(lens) + steps + 1
    layer, w = make_layer(seed, D, H, dtype, max_positions=cap)
    cache = K.kvc_cache_create(layer, B, cap, max_chunk_rows=chunk_rows)
    L = max(lens)
    xp_dev, xp = hidden(seed, synth.STREAM_PREFIX_X, B, L, D, dtype)
    if L > 0:
        for start in range(0, L, chunk_rows):
            n = min(chunk_rows, L - start)
            rows = [max(0, min(n, l - start)) for l in lens]
            K.kvc_continue_chunk(layer, cache, xp_dev[:, start:start + n].contiguous(), n_rows=rows)
    ln, npos = K.kvc_lengths(cache)
    assert ln.tolist() == list(lens) and npos.tolist() == list(lens)
    xd_dev, xd = hidden(seed, synth.STREAM_X, B, steps, D, dtype)
    worst = 0.0
    for s in range(steps):
        out, work = K.kvc_append_and_attend(layer, cache, xd_dev[:, s:s + 1].contiguous())
        cur = [l + s for l in lens]
        assert work["full_prefix_rows_per_projection"] == sum(c + 1 for c in cur)
        assert work["reused_key_value_rows"] == sum(cur)
        o = to_f64(out)[:, 0]
        for b in range(B):
            rows = np.concatenate([xp[b, : lens[b]], xd[b, : s + 1]])
            ref = A.full_prefix_decode(rows, *w, heads=H)
            worst = max(worst, assert_parity(o[b], ref["out"], dtype, f"seq {b} step {s}"))
    ln, npos = K.kvc_lengths(cache)
    assert ln.tolist() == [l + steps for l in lens] and npos.tolist() == ln.tolist()
    for b in range(B):
        rows = np.concatenate([xp[b, : lens[b]], xd[b]])
        full = A.causal_layer(rows, *w, heads=H, rows=[])
        k, v, pos = K.kvc_snapshot(cache, b)
        assert list(pos) == list(range(lens[b] + steps))
        assert_parity(storage_f64(k, dtype), full["keys"], dtype, f"keys seq {b}")
        assert_parity(storage_f64(v, dtype), full["values"], dtype, f"values seq {b}")
    return worst


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_multi_tile_ragged_decode(dtype):
    """Ragged lengths: an empty prefix, a single row, one partial tile and a lane of
    518 rows that crosses the 512-row split-K tile (two partials merged); H=4, d_h=64."""
    _decode_case(dtype, B=4, H=4, dh=64, lens=[0, 1, 300, 517], steps=3, seed=37)


@pytest.mark.parametrize("dtype,dh", [("f64", 16), ("f32", 128), ("bf16", 128), ("bf16", 32)])
def test_decode_head_widths(dtype, dh):
    _decode_case(dtype, B=2, H=2, dh=dh, lens=[255, 256], steps=2, seed=11)


def test_async_decode_matches_sync():
    """KVC_ASYNC enqueues without waiting; after kvc_sync the results and state equal
    the synchronous path."""
    import torch
    layer, w = make_layer(5, 64, 2, "f32", max_positions=64)
    xs_dev, _ = hidden(5, synth.STREAM_X, 2, 8, 64, "f32")
    outs = []
    for flags in (K.KVC_SYNC, K.KVC_ASYNC):
        cache = K.kvc_cache_create(layer, 2, 64)
        res = []
        for s in range(8):
            out, _ = K.kvc_append_and_attend(layer, cache, xs_dev[:, s:s + 1].contiguous(), flags=flags)
            res.append(out)
        K.kvc_sync(cache)
        torch.cuda.synchronize()
        outs.append(torch.stack(res).cpu())
        assert K.kvc_lengths(cache)[0].tolist() == [8, 8]
    assert torch.equal(outs[0], outs[1])


def test_split_tile_edges_bf16():
    """Lengths at the 512-row split boundaries: t = 512 (one full tile), 513 (a second
    tile holding only the candidate row), 1024, 1501 and 2049; three steps so the
    per-lane tile counters are reused after resetting themselves."""
    _decode_case("bf16", B=5, H=2, dh=128, lens=[511, 512, 1023, 1500, 2048], steps=3, seed=23)
