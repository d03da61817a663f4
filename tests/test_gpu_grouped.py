"""Grouped key/value heads on the device (needs an MI355X).

A grouped layer projects keys and values to H_kv < H heads and query head h
reads key/value head h // (H / H_kv) (Chapter 37, "From causal attention to
managed LLM inference state": multi-query attention as the answer to
reloading the retained keys and values; H_kv = 1 is that multi-query form).
The bf16 decode kernel scores every query head of a key/value head from one
read of its rows (up to eight per workgroup); the other kernels index the
shared head.  References: oracle.attention.causal_layer with kv_heads, and a
multi-head layer whose W_k / W_v repeat each key/value head, which must give
bit-identical results.
"""
import numpy as np
import pytest

from incremental_kv_cache_amd import kvcache as K
from incremental_kv_cache_amd import synth
from oracle import attention as A
from oracle import stack as S

from tests.gpu_util import TOL, assert_parity, storage_f64, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield


def _acc(dtype):
    return "f64" if dtype == "f64" else "f32"


def grouped_layer(seed, D, heads, kv_heads, dtype, max_positions, pos_mode=K.KVC_POS_ROPE):
    dh = D // heads
    ws = synth.grouped_weights(seed, D, kv_heads * dh, D ** -0.5, dtype)
    params = K.kvc_params_create_grouped(*[to_device(s, dtype) for s, _ in ws])
    return K.kvc_layer_create(params, heads, pos_mode, 10000.0, max_positions), [f for _, f in ws]


def _rows(seed, B, n, D, dtype):
    s, f = synth.quantize(synth.normal(seed, synth.STREAM_X, (B, n, D)), dtype)
    return to_device(s, dtype), f


CASES = [  # dtype, d_h, H, H_kv: decode workgroups serve 4, 8, 8 (MQA), 2 and 1 query heads
    ("bf16", 128, 8, 2), ("bf16", 128, 16, 2), ("bf16", 64, 8, 1), ("bf16", 64, 6, 3), ("bf16", 128, 6, 2),
    ("f32", 32, 8, 2), ("f64", 16, 4, 1),
]


@pytest.mark.parametrize("dtype,dh,heads,kv_heads", CASES)
def test_grouped_prefill_and_decode_match_the_oracle(dtype, dh, heads, kv_heads):
    """A ragged two-call prefill (the first large enough for the 256-wide MFMA
    projection in bf16, the second for the tiled one), then three decode steps
    over lengths past one 512-row split-K tile: outputs and the cached [H_kv]
    keys and values equal the float64 grouped layer."""
    D = heads * dh
    B, cap = 3, 1024
    layer, w = grouped_layer(31, D, heads, kv_heads, dtype, cap)
    cache = K.kvc_cache_create(layer, B, cap, max_chunk_rows=700)
    assert cache.desc["kv_heads"] == kv_heads
    x1_dev, x1 = _rows(32, B, 700, D, dtype)
    x2_dev, x2 = _rows(33, B, 100, D, dtype)
    n1, n2 = [700, 0, 650], [100, 37, 0]
    out1, _ = K.kvc_continue_chunk(layer, cache, x1_dev, n_rows=n1)
    out2, _ = K.kvc_continue_chunk(layer, cache, x2_dev, n_rows=n2)
    seqs = [np.concatenate([x1[b, : n1[b]], x2[b, : n2[b]]]) for b in range(B)]
    o1, o2 = to_f64(out1), to_f64(out2)
    for b in range(B):
        # sampled rows of each call: first, middle and last of the first, first and last of the second
        picks = [(o1[b], i, i) for i in sorted({0, n1[b] // 2, n1[b] - 1}) if n1[b]]
        picks += [(o2[b], i, n1[b] + i) for i in sorted({0, n2[b] - 1}) if n2[b]]
        if picks:
            ref = A.causal_layer(seqs[b], *w, heads=heads, kv_heads=kv_heads, rows=[r for _, _, r in picks])["out"]
            got = np.stack([o[i] for o, i, _ in picks])
            assert_parity(got, ref, dtype, f"chunk rows of seq {b}")
    xd_dev, xd = _rows(34, B, 3, D, dtype)
    for s in range(3):
        out, work = K.kvc_append_and_attend(layer, cache, xd_dev[:, s:s + 1].contiguous())
        for b in range(B):
            seqs[b] = np.concatenate([seqs[b], xd[b, s:s + 1]])
            ref = A.causal_layer(seqs[b], *w, heads=heads, kv_heads=kv_heads, rows=[len(seqs[b]) - 1])["out"][0]
            assert_parity(to_f64(out)[b, 0], ref, dtype, f"decode {s} seq {b}")
    for b in range(B):
        full = A.causal_layer(seqs[b], *w, heads=heads, kv_heads=kv_heads, rows=[])
        k, v, pos = K.kvc_snapshot(cache, b)
        assert k.shape == (kv_heads, len(seqs[b]), dh) and list(pos) == list(range(len(seqs[b])))
        assert_parity(storage_f64(k, dtype), full["keys"], dtype, f"keys {b}")
        assert_parity(storage_f64(v, dtype), full["values"], dtype, f"values {b}")


@pytest.mark.parametrize("dtype,dh,heads,kv_heads", [("bf16", 128, 8, 2), ("bf16", 128, 4, 1), ("f32", 32, 6, 3)])
def test_grouped_equals_multi_head_with_repeated_weights(dtype, dh, heads, kv_heads):
    """A multi-head layer whose W_k / W_v repeat each key/value head for its
    query heads computes the same keys and values per head and the same
    attention per query head: chunk and decode outputs are bit-identical to
    the grouped layer's, and its cache holds each key/value head repeated.
    (The bf16 decode of a grouped layer scores with q rounded to bf16 and packed
    dot products, so there the two agree within the bf16 bar; both are checked
    against the oracle above.)"""
    import torch
    D = heads * dh
    g = heads // kv_heads
    B, cap = 2, 1024
    lay_g, w = grouped_layer(41, D, heads, kv_heads, dtype, cap)
    ws = synth.grouped_weights(41, D, kv_heads * dh, D ** -0.5, dtype)
    rep = [np.repeat(s.reshape(kv_heads, dh, D), g, axis=0).reshape(D, D) for s, _ in ws[1:]]
    params_m = K.kvc_params_create(to_device(ws[0][0], dtype), to_device(rep[0], dtype), to_device(rep[1], dtype))
    lay_m = K.kvc_layer_create(params_m, heads, K.KVC_POS_ROPE, 10000.0, cap)
    cg = K.kvc_cache_create(lay_g, B, cap, max_chunk_rows=600)
    cm = K.kvc_cache_create(lay_m, B, cap, max_chunk_rows=600)
    x_dev, _ = _rows(42, B, 600, D, dtype)
    og, _ = K.kvc_continue_chunk(lay_g, cg, x_dev, n_rows=[600, 531])
    om, _ = K.kvc_continue_chunk(lay_m, cm, x_dev, n_rows=[600, 531])
    assert torch.equal(og, om)
    xd_dev, _ = _rows(43, B, 2, D, dtype)
    for s in range(2):
        og, _ = K.kvc_append_and_attend(lay_g, cg, xd_dev[:, s:s + 1].contiguous())
        om, _ = K.kvc_append_and_attend(lay_m, cm, xd_dev[:, s:s + 1].contiguous())
        if dtype == "bf16":
            # the grouped bf16 decode scores with q rounded to bf16 (packed dot products),
            # the one-head kernel with float32 q: equal within the bf16 bar
            assert float((og - om).abs().max()) <= TOL["bf16"], f"decode step {s}"
        else:
            assert torch.equal(og, om), f"decode step {s}"
    for b in range(B):
        kg, vg, _ = K.kvc_snapshot(cg, b)
        km, vm, _ = K.kvc_snapshot(cm, b)
        assert np.array_equal(np.repeat(kg, g, axis=0), km) and np.array_equal(np.repeat(vg, g, axis=0), vm)


def test_grouped_paged_equals_contiguous():
    """Grouped heads in a block-paged cache: outputs and rows bit-identical to the
    contiguous grouped cache, and the pool holds H_kv-head blocks."""
    import torch
    D, heads, kv_heads = 1024, 8, 2
    layer, _ = grouped_layer(51, D, heads, kv_heads, "bf16", 2048)
    p = K.kvc_cache_create_paged(layer, 3, 2048, 256, 24, max_chunk_rows=400)
    c = K.kvc_cache_create(layer, 3, 2048, max_chunk_rows=400)
    _, _, nbytes = K.kvc_storage_pointers(p)
    assert nbytes == 24 * kv_heads * 256 * 128 * 2
    for call, rows in enumerate(([400, 13, 300], [400, 400, 0], [0, 270, 399])):
        x, _ = _rows(60 + call, 3, 400, D, "bf16")
        op, _ = K.kvc_continue_chunk(layer, p, x, n_rows=rows)
        oc, _ = K.kvc_continue_chunk(layer, c, x, n_rows=rows)
        assert torch.equal(op, oc)
    for s in range(2):
        x, _ = _rows(70 + s, 3, 1, D, "bf16")
        op, _ = K.kvc_append_and_attend(layer, p, x)
        oc, _ = K.kvc_append_and_attend(layer, c, x)
        assert torch.equal(op, oc)
    for b in range(3):
        for a, bb in zip(K.kvc_snapshot(p, b), K.kvc_snapshot(c, b)):
            assert np.array_equal(a, bb)


@pytest.mark.parametrize("dtype", ["f64", "bf16"])
def test_session_with_grouped_layers_matches_the_stack(dtype):
    """A two-layer session whose layers group 4 query heads per key/value head and
    use multi-query attention: prefill and decode equal the float64 stack."""
    D, vocab, B, cap = 256, 40, 2, 64
    layers, olayers = [], []
    for l, (heads, kv_heads) in enumerate(((8, 2), (4, 1))):
        lay, w = grouped_layer(80 + l, D, heads, kv_heads, dtype, cap)
        layers.append(lay)
        olayers.append(S.Layer(*w, heads=heads, kv_heads=kv_heads))
    es, ef = synth.quantize(synth.normal(85, synth.STREAM_EMBED, (vocab, D)), _acc(dtype))
    sess = K.kvc_session_create(layers, to_device(es, _acc(dtype)), vocab, K.KVC_PE_SINUSOIDAL, B, cap,
                                max_chunk_rows=16)
    import torch
    toks = synth.uniform_int(86, synth.STREAM_TOKENS, B * 20, 0, vocab - 1).reshape(B, 20).astype(np.int32)
    out, _ = K.kvc_session_chunk(sess, torch.tensor(toks[:, :16], device="cuda:0"))
    tol = TOL[dtype] * (2 if dtype == "bf16" else 1)
    worst = 0.0
    for b in range(B):
        ref, _ = S.forward(ef, olayers, toks[b, :16])
        worst = max(worst, float(np.max(np.abs(to_f64(out)[b] - ref))))
        assert worst <= tol
    for s in range(16, 20):
        out, _ = K.kvc_session_decode(sess, torch.tensor(toks[:, s], device="cuda:0"))
        for b in range(B):
            ref, _ = S.forward(ef, olayers, toks[b, : s + 1])
            worst = max(worst, float(np.max(np.abs(to_f64(out)[b, 0] - ref[-1]))))
            assert worst <= tol
    print(f"{dtype} grouped two-layer stack: worst output error {worst:.3e} (bar {tol:.0e})", flush=True)
