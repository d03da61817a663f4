"""Output projection W_o after the merged heads, through the C ABI (needs an MI355X).

Chapter 37 ("Bind the state, calculate completely, then commit") merges the heads
and applies the layer's output projection before anything is committed; its
worked trace prints outputs after a block-swapping W_o.  With W_o bound, the
library's output is merged heads through W_o, for decode and for suffix chunks.
"""
import json
import math
import os

import numpy as np
import pytest

from incremental_kv_cache_amd import kvcache as K
from incremental_kv_cache_amd import synth
from oracle import attention as A

from tests.gpu_util import assert_parity, hidden, make_layer, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield


def test_chapter_trace_printed_outputs_with_bound_output_projection():
    """The trace's printed outputs (9 d.p.) come straight out of the library once the
    fixture's swap W_o is bound; the oracle agrees within 1e-12."""
    import torch
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p2_trace.json")))
    x = np.array([[1.0, 0.0, 1.0, 0.0],
                  [math.cos(1.0), -math.sin(1.0), 0.0, 1.0],
                  [math.cos(2.0), -math.sin(2.0), 1.0, 1.0]])
    eye = np.eye(4)
    w_o = np.zeros((4, 4))
    w_o[0:2, 2:4] = np.eye(2)
    w_o[2:4, 0:2] = np.eye(2)
    t = [torch.tensor(m, device="cuda:0") for m in (eye, eye, eye, w_o)]
    params = K.kvc_params_create(*t)
    layer = K.kvc_layer_create(params, 2, K.KVC_POS_ROPE, 10000.0, 4)
    cache = K.kvc_cache_create(layer, 1, 4)
    for p, step in enumerate(g["steps"]):
        xt = torch.tensor(x[p][None, None, :], device="cuda:0")
        out, _ = K.kvc_append_and_attend(layer, cache, xt)
        y = to_f64(out)[0, 0]
        np.testing.assert_allclose(y, step["output"], rtol=0, atol=5.1e-10)
        ref = A.full_prefix_decode(x[: p + 1], eye, eye, eye, heads=2, wo=w_o)
        assert np.max(np.abs(y - ref["out"])) <= 1e-12


@pytest.mark.parametrize("dtype,H,dh", [("f64", 4, 64), ("f32", 4, 64), ("bf16", 4, 64), ("bf16", 16, 128)])
def test_decode_with_output_projection(dtype, H, dh):
    """Ragged multi-tile prefixes (one empty), two decode steps; every output against
    the full-prefix oracle followed by W_o."""
    D = H * dh
    lens = [0, 700, 1500]
    B = len(lens)
    cap = 1600
    layer, w = make_layer(31, D, H, dtype, max_positions=cap, wo=True)
    cache = K.kvc_cache_create(layer, B, cap, max_chunk_rows=max(lens))
    xp_dev, xp = hidden(31, synth.STREAM_PREFIX_X, B, max(lens), D, dtype)
    K.kvc_continue_chunk(layer, cache, xp_dev, n_rows=lens)
    xn_dev, xn = hidden(31, synth.STREAM_X, B, 2, D, dtype)
    for i in range(2):
        out, _ = K.kvc_append_and_attend(layer, cache, xn_dev[:, i:i + 1].contiguous())
        o = to_f64(out)[:, 0]
        for b in range(B):
            seq = np.concatenate([xp[b, : lens[b]], xn[b, : i + 1]])
            ref = A.full_prefix_decode(seq, w[0], w[1], w[2], heads=H, wo=w[3])
            assert_parity(o[b], ref["out"], dtype, f"step {i} seq {b}")
    ln, npos = K.kvc_lengths(cache)
    assert ln.tolist() == [n + 2 for n in lens] and npos.tolist() == ln.tolist()


@pytest.mark.parametrize("dtype,H,dh,n_max", [("f64", 4, 32, 64), ("f32", 4, 32, 64), ("bf16", 2, 64, 24),
                                              ("bf16", 16, 128, 96)])
def test_chunk_with_output_projection(dtype, H, dh, n_max):
    """Ragged cuts and ragged chunk rows (including 0 and 1): outputs against the causal
    oracle followed by W_o; padding rows stay untouched."""
    D = H * dh
    lens, cuts = [0, 40, 300, 37], [0, 17, 300, 37]
    rows = [5, n_max, 1, 0]
    B = len(lens)
    cap = 400
    layer, w = make_layer(13, D, H, dtype, max_positions=cap, wo=True)
    cache = K.kvc_cache_create(layer, B, cap, max_chunk_rows=512)
    xp_dev, xp = hidden(13, synth.STREAM_PREFIX_X, B, max(lens), D, dtype)
    K.kvc_continue_chunk(layer, cache, xp_dev, n_rows=lens)
    K.kvc_truncate(cache, cuts)
    xn_dev, xn = hidden(13, synth.STREAM_X, B, n_max, D, dtype)
    out, _ = K.kvc_continue_chunk(layer, cache, xn_dev, n_rows=rows)
    o = to_f64(out)
    for b in range(B):
        seq = np.concatenate([xp[b, : cuts[b]], xn[b, : rows[b]]])
        if rows[b]:
            ref = A.causal_layer(seq, w[0], w[1], w[2], heads=H, rows=range(cuts[b], cuts[b] + rows[b]), wo=w[3])
            assert_parity(o[b, : rows[b]], ref["out"], dtype, f"seq {b}")
        assert not np.any(o[b, rows[b]:])


@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_identity_output_projection_changes_nothing(dtype):
    """W_o = I reproduces the unprojected output bit for bit (every product is by 1 or 0)."""
    import torch
    H, dh = 4, 32
    D = H * dh
    ws = synth.decode_weights(5, D, D ** -0.5, dtype)
    t = [to_device(s, dtype) for s, _ in ws]
    eye = torch.eye(D, dtype=t[0].dtype, device="cuda:0")
    outs = []
    for with_wo in (False, True):
        params = K.kvc_params_create(*t, eye) if with_wo else K.kvc_params_create(*t)
        layer = K.kvc_layer_create(params, H, K.KVC_POS_ROPE, 10000.0, 256)
        cache = K.kvc_cache_create(layer, 2, 256, max_chunk_rows=64)
        xp_dev, _ = hidden(5, synth.STREAM_PREFIX_X, 2, 50, D, dtype)
        o1, _ = K.kvc_continue_chunk(layer, cache, xp_dev)
        xn_dev, _ = hidden(5, synth.STREAM_X, 2, 1, D, dtype)
        o2, _ = K.kvc_append_and_attend(layer, cache, xn_dev)
        outs.append((to_f64(o1), to_f64(o2)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_overflowing_output_projection_is_reported_and_not_committed(dtype):
    """A finite W_o whose row 5 overflows the accumulate type: the call fails with the
    first non-finite output's flat index, and no row is committed (Chapter 37:
    validate the result before publishing the new length)."""
    import torch
    D, H = 128, 2
    td = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    eye = torch.eye(D, dtype=td, device="cuda:0")
    wo = torch.eye(D, dtype=torch.float32)
    wo[5, 0] = 3.0e38
    wo[5, 1] = 3.0e38
    params = K.kvc_params_create(eye, eye, eye, wo.to(td).to("cuda:0"))
    layer = K.kvc_layer_create(params, H, K.KVC_POS_ROPE, 10000.0, 16)
    cache = K.kvc_cache_create(layer, 2, 16)
    x = torch.zeros((2, 1, D), dtype=td)
    x[:, 0, 0] = 1.0
    x[:, 0, 1] = 1.0
    with pytest.raises(K.KvcError) as e:
        K.kvc_append_and_attend(layer, cache, x.to("cuda:0"))
    assert e.value.name == "KVC_ERR_NONFINITE_OUTPUT"
    assert e.value.detail["flat_index"] == 5
    ln, npos = K.kvc_lengths(cache)
    assert ln.tolist() == [0, 0] and npos.tolist() == [0, 0]
