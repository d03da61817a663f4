"""Suffix-chunk continuation parity through the C ABI (needs an MI355X).

Prefix-reuse note: truncate to `cut`, set next_position = cut, compute the causal
suffix; the result must equal a full recompute of the new sequence, and the
stale-position negative control must not.
"""
import json
import os

import numpy as np
import pytest

from incremental_kv_cache_amd import kvcache as K
from incremental_kv_cache_amd import synth
from oracle import attention as A
from oracle import prefix as P
from oracle import toy_decoder as T

from tests.gpu_util import assert_parity, hidden, make_layer, storage_f64, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_truncate_and_chunk_match_full_recompute(dtype):
    """Ragged cuts (0, mid, whole prefix) and ragged chunk rows (including 0 and 1) on top
    of a multi-tile prefix; outputs, untouched padding rows, stored rows and positions."""
    import torch
    B, H, dh = 4, 4, 32
    D = H * dh
    lens, cuts, rows = [0, 40, 300, 37], [0, 17, 300, 37], [5, 64, 1, 0]
    n_max = 64
    cap = 400
    layer, w = make_layer(7, D, H, dtype, max_positions=cap)
    cache = K.kvc_cache_create(layer, B, cap, max_chunk_rows=512)
    xp_dev, xp = hidden(7, synth.STREAM_PREFIX_X, B, max(lens), D, dtype)
    K.kvc_continue_chunk(layer, cache, xp_dev, n_rows=lens)
    K.kvc_truncate(cache, cuts)
    ln, npos = K.kvc_lengths(cache)
    assert ln.tolist() == cuts and npos.tolist() == cuts
    xn_dev, xn = hidden(7, synth.STREAM_X, B, n_max, D, dtype)
    out, work = K.kvc_continue_chunk(layer, cache, xn_dev, n_rows=rows)
    assert {k: work[k] for k in P.chunk_work(cuts, rows)} == P.chunk_work(cuts, rows)
    o = to_f64(out)
    for b in range(B):
        seq = np.concatenate([xp[b, : cuts[b]], xn[b, : rows[b]]])
        if rows[b]:
            ref = A.causal_layer(seq, *w, heads=H, rows=range(cuts[b], cuts[b] + rows[b]))
            assert_parity(o[b, : rows[b]], ref["out"], dtype, f"seq {b}")
        assert not np.any(o[b, rows[b]:])  # rows past n_b untouched (zero-initialised)
        full = A.causal_layer(seq, *w, heads=H, rows=[])
        k, v, pos = K.kvc_snapshot(cache, b)
        assert list(pos) == list(range(cuts[b] + rows[b]))
        if len(seq):
            assert_parity(storage_f64(k, dtype), full["keys"], dtype, f"keys {b}")
            assert_parity(storage_f64(v, dtype), full["values"], dtype, f"values {b}")


def test_chunk_equals_sequential_decode_on_device():
    """An n-row chunk and n single-row decodes give the same outputs (float64, 1e-12)."""
    H, dh, n = 2, 16, 9
    D = H * dh
    layer, w = make_layer(3, D, H, "f64", max_positions=64)
    xp_dev, _ = hidden(3, synth.STREAM_PREFIX_X, 2, 20, D, "f64")
    xn_dev, _ = hidden(3, synth.STREAM_X, 2, n, D, "f64")
    a = K.kvc_cache_create(layer, 2, 64, max_chunk_rows=32)
    b = K.kvc_cache_create(layer, 2, 64, max_chunk_rows=32)
    for c in (a, b):
        K.kvc_continue_chunk(layer, c, xp_dev)
    out_chunk, _ = K.kvc_continue_chunk(layer, a, xn_dev)
    steps = [to_f64(K.kvc_append_and_attend(layer, b, xn_dev[:, i:i + 1].contiguous())[0])[:, 0] for i in range(n)]
    np.testing.assert_allclose(to_f64(out_chunk), np.stack(steps, axis=1), rtol=0, atol=1e-12)
    ka, va, pa = K.kvc_snapshot(a, 1)
    kb, vb, pb = K.kvc_snapshot(b, 1)
    np.testing.assert_allclose(ka, kb, rtol=0, atol=1e-13)
    assert np.array_equal(pa, pb)


def test_stale_next_position_negative_control():
    """Prefix-reuse note negative control with RoPE: same trim, same suffix, next_position
    left at the old length -- nothing raises, positions are stale, results diverge."""
    H, dh = 2, 16
    D = H * dh
    layer, w = make_layer(11, D, H, "f64", max_positions=64)
    old_dev, old = hidden(11, synth.STREAM_PREFIX_X, 1, 8, D, "f64")
    new_dev, new = hidden(11, synth.STREAM_X, 1, 8, D, "f64")
    seq = np.concatenate([old[0, :4], new[0]])
    ref = A.causal_layer(seq, *w, heads=H, rows=range(4, 12))["out"]
    errs = {}
    for stale in (False, True):
        c = K.kvc_cache_create(layer, 1, 64, max_chunk_rows=8)
        K.kvc_continue_chunk(layer, c, old_dev)
        K.kvc_truncate(c, [4], flags=K.KVC_TRUNCATE_KEEP_STALE_POSITION if stale else 0)
        out, work = K.kvc_continue_chunk(layer, c, new_dev)
        errs[stale] = float(np.max(np.abs(to_f64(out)[0] - ref)))
        _, _, pos = K.kvc_snapshot(c, 0)
        if stale:
            assert work["position_min"] == 8 and list(pos) == [0, 1, 2, 3] + list(range(8, 16))
        else:
            assert work["position_min"] == 4 and list(pos) == list(range(12))
    assert errs[False] <= 1e-12
    assert errs[True] > 1e-3


def _toy_layers(model):
    """One library layer per toy-decoder layer: one head, width 16, float64, no rotation."""
    import torch
    layers = []
    for wq, wk, wv in model.layers:
        t = [torch.tensor(np.ascontiguousarray(m), device="cuda:0") for m in (wq, wk, wv)]
        params = K.kvc_params_create(*t)
        layers.append(K.kvc_layer_create(params, 1, K.KVC_POS_NONE, 10000.0, 64))
    return layers


def _toy_chunk(model, layers, caches, tokens):
    """The toy decoder's suffix step with each layer's attention on the device:
    host glue adds embedding + sinusoidal PE at next_position + i (read from the
    library) and the tanh residual; attention, cache append and positions are the
    library's."""
    import torch
    start = int(K.kvc_lengths(caches[0])[1][0])
    pos = start + np.arange(len(tokens))
    h = T.embed(model, tokens, pos)
    works = []
    for layer, cache in zip(layers, caches):
        x = torch.tensor(h[None], device="cuda:0")
        a, work = K.kvc_continue_chunk(layer, cache, x)
        works.append(work)
        h = h + np.tanh(to_f64(a)[0])
    return h, works


@pytest.mark.parametrize("seed", [7, 11, 23])
def test_toy_decoder_prefix_reuse(seed):
    """Prefix-reuse note, the rows of its 27-case matrix covered here: append, edit first,
    edit fifth, edit eighth, shorten, the exercise, and the seeded edit.  Correct reuse is
    within 1e-12 of the float64 full recompute; projection rows are 6 x (len - cut); the
    stale-position control diverges whenever cut < 8."""
    e, ws = synth.toy_model_arrays(seed)
    model = T.ToyModel(e, ws)
    layers = _toy_layers(model)
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p3_cut_table.json")))
    cases = [(g["cached"], c["query"], c.get("cut")) for c in g["conditions"]]
    cs, qs, _ = synth.toy_edit_case(seed)
    cases.append((list(cs), list(qs), None))
    for cached, query, want_cut in cases:
        full, _ = T.full_forward(model, query)
        cut = K.kvc_lcp_cut(cached, query)
        if want_cut is not None:
            assert cut == want_cut
        assert cut == P.lcp_cut(cached, query)
        for stale in (False, True):
            caches = [K.kvc_cache_create(l, 1, 64, max_chunk_rows=16) for l in layers]
            _toy_chunk(model, layers, caches, cached)          # prefill the cached prefix
            for c in caches:
                K.kvc_truncate(c, [cut], flags=K.KVC_TRUNCATE_KEEP_STALE_POSITION if stale else 0)
            h, works = _toy_chunk(model, layers, caches, query[cut:])
            err = float(np.max(np.abs(h - full[cut:])))
            rows = sum(3 * w["incremental_rows_per_projection"] for w in works)
            assert rows == P.continuation_projection_rows(2, len(query), cut)[0]
            if not stale:
                assert err <= 1e-12, (cached, query)
                ref_cache = T.full_forward(model, query)[1]
                for c, (kf, vf, pf) in zip(caches, ref_cache["layers"]):
                    k, v, pos = K.kvc_snapshot(c, 0)
                    np.testing.assert_allclose(k[0], kf, rtol=0, atol=1e-12)
                    np.testing.assert_allclose(v[0], vf, rtol=0, atol=1e-12)
                    assert np.array_equal(pos, pf)
            elif cut < len(cached):
                assert err > 1e-3, (cached, query)
            else:
                assert err <= 1e-12
