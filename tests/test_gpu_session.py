"""Model-wide sessions on the device (needs an MI355X).

A session binds one cache per layer behind one token stream (Chapter 37, "Give
every decoder block its own state next"): the embedding, the sinusoidal
positions, each layer's attention and the tanh residual all run in the
library's kernels, every layer computes before any appends, and truncation
trims every layer with next_position (prefix-reuse note, "What must be trimmed
together").  References: oracle.stack (full recompute of the stack) and
oracle.toy_decoder (the note's two-layer model).
"""
import json
import os

import numpy as np
import pytest

from incremental_kv_cache_amd import kvcache as K
from incremental_kv_cache_amd import synth
from oracle import prefix as P
from oracle import stack as S
from oracle import toy_decoder as T

from tests.gpu_util import TOL, assert_parity, make_layer, storage_f64, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield


def _tokens(values):
    import torch
    return torch.tensor(np.asarray(values, np.int32), device="cuda:0")


def _acc(dtype):
    return "f64" if dtype == "f64" else "f32"


def _toy_session(model, cap=64):
    import torch
    layers = []
    for wq, wk, wv in model.layers:
        t = [torch.tensor(np.ascontiguousarray(m), device="cuda:0") for m in (wq, wk, wv)]
        layers.append(K.kvc_layer_create(K.kvc_params_create(*t), 1, K.KVC_POS_NONE, 10000.0, cap))
    emb = torch.tensor(model.embed, device="cuda:0")
    return K.kvc_session_create(layers, emb, emb.shape[0], K.KVC_PE_SINUSOIDAL, 1, cap, max_chunk_rows=16)


@pytest.mark.parametrize("seed", [7, 11, 23])
def test_toy_decoder_fully_on_device(seed):
    """The note's toy decoder with embedding, positions, both layers and the
    residual on the device: reuse after the longest-common-prefix cut equals the
    float64 full recompute within 1e-12 for every condition of the note's table
    and the seeded edit; each layer's keys, values and positions equal the
    recompute's; 6 x (len - cut) projection rows; the stale-position control
    diverges whenever cut < 8 (prefix-reuse note, 'Work and error over 27 cases')."""
    e, ws = synth.toy_model_arrays(seed)
    model = T.ToyModel(e, ws)
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p3_cut_table.json")))
    cases = [(g["cached"], c["query"]) for c in g["conditions"]]
    cs, qs, _ = synth.toy_edit_case(seed)
    cases.append((list(cs), list(qs)))
    for cached, query in cases:
        full, ref_cache = T.full_forward(model, query)
        cut = K.kvc_lcp_cut(cached, query)
        assert cut == P.lcp_cut(cached, query)
        for stale in (False, True):
            sess = _toy_session(model)
            K.kvc_session_chunk(sess, _tokens([cached]))
            K.kvc_session_truncate(sess, [cut], flags=K.KVC_TRUNCATE_KEEP_STALE_POSITION if stale else 0)
            out, work = K.kvc_session_chunk(sess, _tokens([query[cut:]]))
            err = float(np.max(np.abs(to_f64(out)[0] - full[cut:])))
            assert 3 * work["incremental_rows_per_projection"] == P.continuation_projection_rows(2, len(query), cut)[0]
            if not stale:
                assert err <= 1e-12, (cached, query, err)
                for c, (kf, vf, pf) in zip(sess.caches, ref_cache["layers"]):
                    k, v, pos = K.kvc_snapshot(c, 0)
                    np.testing.assert_allclose(k[0], kf, rtol=0, atol=1e-12)
                    np.testing.assert_allclose(v[0], vf, rtol=0, atol=1e-12)
                    assert np.array_equal(pos, pf)
            elif cut < len(cached):
                assert err > 1e-3, (cached, query)
            else:
                assert err <= 1e-12


def _stack_tol(dtype, layers):
    """Parity bar of an L-layer stack: the single-layer bars for float64 and float32;
    for bf16, L x 2e-2 -- every layer reads its input rows rounded to bf16 and the
    residual adds each layer's error to the next (tanh is 1-Lipschitz), so the
    per-layer bf16 bar accumulates once per layer."""
    return TOL[dtype] * (layers if dtype == "bf16" else 1)


def _parity(gpu, ref, dtype, layers, what):
    e = float(np.max(np.abs(np.asarray(gpu) - np.asarray(ref))))
    if dtype == "f32":
        e /= max(float(np.max(np.abs(ref))), 1e-300)
    assert e <= _stack_tol(dtype, layers), f"{what}: error {e:.3e} above {_stack_tol(dtype, layers):.0e} ({dtype})"
    return e


def _stack_session(dtype, B, cap, seed=61, D=128, vocab=50, specs=((2, True, False), (4, False, True), (2, True, False))):
    """Layers with different head counts, rotation and W_o; returns (session, oracle layers, embedding)."""
    layers, olayers = [], []
    for l, (heads, rope, wo) in enumerate(specs):
        lay, w = make_layer(seed + 10 * l, D, heads, dtype, max_positions=cap, wo=wo,
                            pos_mode=K.KVC_POS_ROPE if rope else K.KVC_POS_NONE)
        layers.append(lay)
        olayers.append(S.Layer(w[0], w[1], w[2], heads=heads, rope=rope, wo=w[3] if wo else None))
    es, ef = synth.quantize(synth.normal(seed, synth.STREAM_EMBED, (vocab, D)), _acc(dtype))
    sess = K.kvc_session_create(layers, to_device(es, _acc(dtype)), vocab, K.KVC_PE_SINUSOIDAL, B, cap,
                                max_chunk_rows=32)
    return sess, olayers, ef


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_session_prefill_and_decode_match_the_stack(dtype):
    """A three-layer session (2 and 4 heads, rotary and plain positions, one layer
    with W_o): a ragged prefill and three decode steps per sequence equal the
    float64 stack recomputed from scratch at every step, and each layer's cache
    holds the recompute's keys and values (bars: _stack_tol)."""
    B, cap, vocab = 3, 48, 50
    sess, olayers, ef = _stack_session(dtype, B, cap, vocab=vocab)
    lens = [10, 0, 23]
    toks = synth.uniform_int(62, synth.STREAM_TOKENS, B * 30, 0, vocab - 1).reshape(B, 30).astype(np.int32)
    pre = np.zeros((B, max(lens)), np.int32)
    for b in range(B):
        pre[b, : lens[b]] = toks[b, : lens[b]]
    out, work = K.kvc_session_chunk(sess, _tokens(pre), n_rows=lens)
    assert work["incremental_rows_per_projection"] == 3 * sum(lens)
    o = to_f64(out)
    worst_out = 0.0
    for b in range(B):
        if lens[b]:
            ref, _ = S.forward(ef, olayers, toks[b, : lens[b]])
            worst_out = max(worst_out, _parity(o[b, : lens[b]], ref, dtype, 3, f"prefill seq {b}"))
    for step in range(3):
        cur = [toks[b, lens[b] + step] for b in range(B)]
        out, work = K.kvc_session_decode(sess, _tokens(cur))
        assert work["incremental_rows_per_projection"] == 3 * B
        o = to_f64(out)[:, 0]
        for b in range(B):
            ref, _ = S.forward(ef, olayers, toks[b, : lens[b] + step + 1])
            worst_out = max(worst_out, _parity(o[b], ref[-1], dtype, 3, f"step {step} seq {b}"))
    worst_kv = [0.0] * len(sess.caches)
    for b in range(B):
        _, kv = S.forward(ef, olayers, toks[b, : lens[b] + 3])
        for l, (c, (kf, vf)) in enumerate(zip(sess.caches, kv)):
            k, v, pos = K.kvc_snapshot(c, b)
            assert list(pos) == list(range(lens[b] + 3))
            worst_kv[l] = max(worst_kv[l], _parity(storage_f64(k, dtype), kf, dtype, l + 1, f"layer {l} keys {b}"),
                              _parity(storage_f64(v, dtype), vf, dtype, l + 1, f"layer {l} values {b}"))
    # the measured errors beside the bars (reported with pytest -s)
    print(f"{dtype} stack: worst key/value error per layer "
          f"{', '.join(f'{e:.3e} (bar {_stack_tol(dtype, l + 1):.0e})' for l, e in enumerate(worst_kv))}; "
          f"worst output error {worst_out:.3e} (bar {_stack_tol(dtype, 3):.0e})", flush=True)


def _all_state(sess):
    return [(K.kvc_lengths(c)[0].tolist(), K.kvc_lengths(c)[1].tolist(), K.kvc_copy_storage(c)) for c in sess.caches]


def _same(a, b):
    return all(la == lb and na == nb and np.array_equal(ka, kb) and np.array_equal(va, vb)
               for (la, na, (ka, va)), (lb, nb, (kb, vb)) in zip(a, b))


def test_failure_in_one_layer_commits_no_layer():
    """Every layer prepares before any appends (Chapter 37, prepared-row listing):
    a non-finite key in the second layer is reported with its layer, and neither
    layer's lengths, positions or storage change."""
    import torch
    B, D, H = 2, 64, 2
    layers = []
    for l in range(2):
        ws = synth.decode_weights(70 + l, D, D ** -0.5, "f32")
        t = [to_device(s, "f32") for s, _ in ws]
        if l == 1:
            t[1][5, 7] = float("inf")
        layers.append(K.kvc_layer_create(K.kvc_params_create(*t), H, K.KVC_POS_ROPE, 10000.0, 16))
    emb = torch.randn(20, D, dtype=torch.float32, device="cuda:0")
    sess = K.kvc_session_create(layers, emb, 20, K.KVC_PE_SINUSOIDAL, B, 16, max_chunk_rows=4)
    before = _all_state(sess)
    with pytest.raises(K.KvcError) as ei:
        K.kvc_session_decode(sess, _tokens([1, 2]))
    assert ei.value.name == "KVC_ERR_NONFINITE_KEY" and ei.value.detail["layer"] == 1
    assert _same(before, _all_state(sess))


def test_token_outside_the_embedding_is_rejected_sync_and_deferred():
    """A token id outside [0, vocab) sets the session's token word: nothing is
    appended; in KVC_ASYNC mode the next kvc_session_sync reports it as DEFERRED;
    later calls run normally."""
    sess, olayers, ef = _stack_session("f32", 2, 16, vocab=50)
    before = _all_state(sess)
    with pytest.raises(K.KvcError) as ei:
        K.kvc_session_decode(sess, _tokens([3, 50]))
    assert ei.value.name == "KVC_ERR_TOKEN_RANGE" and ei.value.detail["flat_index"] == 1
    assert ei.value.detail["layer"] == 0
    assert _same(before, _all_state(sess))
    K.kvc_session_decode(sess, _tokens([-1, 4]), flags=K.KVC_ASYNC)
    with pytest.raises(K.KvcError) as ei:
        K.kvc_session_sync(sess)
    assert ei.value.name == "KVC_ERR_DEFERRED" and ei.value.detail["actual"] == K.capi.KVC_ERR_TOKEN_RANGE
    assert _same(before, _all_state(sess))
    out, _ = K.kvc_session_decode(sess, _tokens([3, 4]))
    for b, t in enumerate([3, 4]):
        ref, _ = S.forward(ef, olayers, [t])
        assert_parity(to_f64(out)[b, 0], ref[0], "f32", f"seq {b}")
