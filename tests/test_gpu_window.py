"""Sliding-window layers and ring caches on the device (needs an MI355X).

A window layer's query at row r reads rows r - W + 1 .. r (prefix-reuse note,
"Why a sliding-window partial hit must fall back"); its cache is a ring of C
rows that keeps counting past C.  References: oracle.attention.causal_layer
with `window` over the whole history, oracle.toy_decoder with a window, and
oracle.prefix.window_continuable for which cuts can be continued.
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

from tests.gpu_util import assert_parity, storage_f64, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield


def window_layer(seed, D, heads, kv_heads, window, dtype, max_positions=8192):
    dh = D // heads
    ws = synth.grouped_weights(seed, D, kv_heads * dh, D ** -0.5, dtype)
    params = K.kvc_params_create_grouped(*[to_device(s, dtype) for s, _ in ws])
    return K.kvc_layer_create_windowed(params, heads, window, K.KVC_POS_ROPE, 10000.0, max_positions), \
        [f for _, f in ws]


def _rows(seed, B, n, D, dtype):
    s, f = synth.quantize(synth.normal(seed, synth.STREAM_X, (B, n, D)), dtype)
    return to_device(s, dtype), f


CASES = [  # dtype, d_h, H, H_kv, window, capacity
    ("bf16", 128, 4, 4, 300, 512), ("bf16", 128, 8, 2, 700, 1024), ("bf16", 64, 4, 1, 200, 256),
    ("f32", 32, 4, 2, 300, 512), ("f64", 16, 2, 2, 150, 256),
]


@pytest.mark.parametrize("dtype,dh,heads,kv_heads,window,cap", CASES)
def test_window_history_past_the_capacity_matches_the_oracle(dtype, dh, heads, kv_heads, window, cap):
    """Ragged chunks and decodes until every sequence has written several times
    the ring: each call's outputs (sampled chunk rows, every decode row) equal
    the float64 windowed layer over the whole history, and the held rows are
    the last ones with their keys and values."""
    D = heads * dh
    B = 3
    layer, w = window_layer(21, D, heads, kv_heads, window, dtype)
    cache = K.kvc_cache_create(layer, B, cap, max_chunk_rows=cap // 2)
    assert cache.desc["window"] == window
    hist = [np.zeros((0, D)) for _ in range(B)]
    rng = np.random.default_rng(22)
    for call in range(7):
        rows = [int(v) for v in rng.integers(0, cap // 2 + 1, B)]
        rows[call % B] = cap // 2
        x_dev, x = _rows(300 + call, B, cap // 2, D, dtype)
        out, _ = K.kvc_continue_chunk(layer, cache, x_dev, n_rows=rows)
        o = to_f64(out)
        for b in range(B):
            if not rows[b]:
                continue
            first = len(hist[b])
            hist[b] = np.concatenate([hist[b], x[b, : rows[b]]])
            pick = sorted({0, rows[b] // 2, rows[b] - 1})
            ref = A.causal_layer(hist[b], *w, heads=heads, kv_heads=kv_heads, window=window,
                                 rows=[first + i for i in pick])["out"]
            assert_parity(o[b, pick], ref, dtype, f"call {call} seq {b}")
        if call % 2:
            xd_dev, xd = _rows(400 + call, B, 1, D, dtype)
            out, _ = K.kvc_append_and_attend(layer, cache, xd_dev)
            for b in range(B):
                hist[b] = np.concatenate([hist[b], xd[b]])
                ref = A.causal_layer(hist[b], *w, heads=heads, kv_heads=kv_heads, window=window,
                                     rows=[len(hist[b]) - 1])["out"][0]
                assert_parity(to_f64(out)[b, 0], ref, dtype, f"decode {call} seq {b}")
    lens = K.kvc_lengths(cache)[0]
    assert max(lens) > 2 * cap
    for b in range(B):
        k, v, pos = K.kvc_snapshot(cache, b)
        L = len(hist[b])
        held = min(L, cap)
        assert list(pos) == list(range(L - held, L))
        full = A.causal_layer(hist[b], *w, heads=heads, kv_heads=kv_heads, rows=[])
        assert_parity(storage_f64(k, dtype), full["keys"][:, L - held:], dtype, f"keys {b}")
        assert_parity(storage_f64(v, dtype), full["values"][:, L - held:], dtype, f"values {b}")


@pytest.mark.parametrize("dtype", ["f64", "bf16"])
def test_window_reuse_cut_continues_exactly(dtype):
    """After a history past the ring's capacity, a common prefix whose window is
    still held is continued (kvc_reuse_cut returns it) and equals the recompute
    of the new history; a prefix that needs rows written over falls back to 0,
    and the recompute from an empty sequence equals it as well."""
    D, heads, window, cap = 256, 2, 200, 512
    layer, w = window_layer(23, D, heads, heads, window, dtype)
    cache = K.kvc_cache_create(layer, 1, cap, max_chunk_rows=256)
    x_dev, x = _rows(24, 1, 256, D, dtype)
    hist = np.zeros((0, D))
    for call in range(4):
        xc_dev, xc = _rows(25 + call, 1, 256, D, dtype)
        K.kvc_continue_chunk(layer, cache, xc_dev)
        hist = np.concatenate([hist, xc[0]])
    L = len(hist)  # 1024 rows, rows 512 .. 1023 held
    for lcp, want in ((900, 900), (L - cap + window - 1, L - cap + window - 1), (600, 0)):
        cut = K.kvc_reuse_cut(cache, 0, lcp)
        assert cut == want == (lcp if P.window_continuable(L, lcp, window, cap) else 0)
    # continue from 900 with a new 40-row suffix
    K.kvc_truncate(cache, [900])
    out, _ = K.kvc_continue_chunk(layer, cache, x_dev[:, :40].contiguous())
    new = np.concatenate([hist[:900], x[0, :40]])
    ref = A.causal_layer(new, *w, heads=heads, window=window, rows=range(900, 940))["out"]
    assert_parity(to_f64(out)[0], ref, dtype, "continued suffix")
    with pytest.raises(K.KvcError) as ei:
        K.kvc_truncate(cache, [600])
    assert ei.value.name == "KVC_ERR_BAD_CUT"
    # the fallback: recompute the whole new history from row 0
    K.kvc_truncate(cache, [0])
    other = np.concatenate([hist[:600], x[0, :40]])
    other_dev = to_device(synth.quantize(other, dtype)[0], dtype)[None]
    outs = []
    for first in range(0, len(other), 256):
        o, _ = K.kvc_continue_chunk(layer, cache, other_dev[:, first: first + 256].contiguous())
        outs.append(to_f64(o)[0, : min(256, len(other) - first)])
    ref = A.causal_layer(other, *w, heads=heads, window=window, rows=range(len(other) - 40, len(other)))["out"]
    assert_parity(np.concatenate(outs)[-40:], ref, dtype, "recomputed suffix")


def test_window_toy_decoder_session_follows_the_table():
    """The note's window rows through a library session: the toy decoder with a
    window of 4 (both layers), the cached prefix 1..8 and the note's two window
    queries.  kvc_reuse_cut keeps cut 8 for the append (24 projection rows) and,
    because this ring still holds every row, also the edit's cut 4 -- the finer
    strategy the note allows when rows are kept -- and both continuations equal
    the float64 windowed recompute within 1e-12."""
    import torch
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p3_window_table.json")))
    e, ws = synth.toy_model_arrays(7)
    model = T.ToyModel(e, ws, window=g["window"])
    for c in g["conditions"]:
        layers = []
        for wq, wk, wv in model.layers:
            t = [torch.tensor(np.ascontiguousarray(m), device="cuda:0") for m in (wq, wk, wv)]
            layers.append(K.kvc_layer_create_windowed(K.kvc_params_create(*t), 1, g["window"], K.KVC_POS_NONE,
                                                      10000.0, 256))
        emb = torch.tensor(model.embed, device="cuda:0")
        sess = K.kvc_session_create(layers, emb, emb.shape[0], K.KVC_PE_SINUSOIDAL, 1, 256, max_chunk_rows=16)
        K.kvc_session_chunk(sess, torch.tensor([g["cached"]], dtype=torch.int32, device="cuda:0"))
        lcp = K.kvc_lcp_cut(g["cached"], c["query"])
        cut = K.kvc_reuse_cut(sess.caches[0], 0, lcp)
        assert cut == lcp
        K.kvc_session_truncate(sess, [cut])
        out, work = K.kvc_session_chunk(sess, torch.tensor([c["query"][cut:]], dtype=torch.int32,
                                                           device="cuda:0"))
        full, _ = T.full_forward(model, c["query"])
        assert float(np.max(np.abs(to_f64(out)[0] - full[cut:]))) <= 1e-12
        assert 3 * work["incremental_rows_per_projection"] == P.continuation_projection_rows(2, len(c["query"]),
                                                                                             cut)[0]
        if c["cut"] == 8:
            assert P.continuation_projection_rows(2, len(c["query"]), cut) == (c["rows"], c["full_rows"])
