"""Parity of the bf16 matrix-core paths (needs an MI355X).

The projection switches to MFMA kernels for bf16 when D % 128 == 0 (a skinny
kernel for up to 64 rows, a tiled one above), and chunk attention uses the
flash kernel for d_h in {64, 128}.  Shapes here cross every tile edge: rows not
a multiple of 32 or 128, several query tiles of 256, key tiles straddling the
retained/chunk boundary, empty and single-row chunks.
"""
import numpy as np
import pytest

from incremental_kv_cache_amd import kvcache as K
from incremental_kv_cache_amd import synth
from oracle import attention as A

from tests.gpu_util import assert_parity, hidden, make_layer, storage_f64, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield


@pytest.mark.parametrize("B", [3, 40, 70])
def test_decode_projection_rows(B):
    """Skinny kernel with 3 and 40 rows (two 32-row tiles), tiled kernel at 70 rows:
    the stored candidate rows and outputs match the oracle."""
    H, dh = 2, 64
    D = H * dh
    layer, w = make_layer(13, D, H, "bf16", max_positions=8)
    cache = K.kvc_cache_create(layer, B, 8)
    x_dev, x = hidden(13, synth.STREAM_X, B, 2, D, "bf16")
    outs = []
    for s in range(2):
        out, _ = K.kvc_append_and_attend(layer, cache, x_dev[:, s:s + 1].contiguous())
        outs.append(to_f64(out)[:, 0])
    for b in range(B):
        full = A.causal_layer(x[b], *w, heads=H)
        for s in range(2):
            assert_parity(outs[s][b], full["out"][s], "bf16", f"seq {b} step {s}")
        k, v, pos = K.kvc_snapshot(cache, b)
        assert_parity(storage_f64(k, "bf16"), full["keys"], "bf16", f"keys {b}")
        assert_parity(storage_f64(v, "bf16"), full["values"], "bf16", f"values {b}")


@pytest.mark.parametrize("dh", [64, 128])
def test_flash_chunk_ragged(dh):
    """Two query tiles (n_max = 300), cuts that end inside a 128-key tile, rows 0/1/300/263."""
    H = 2
    D = H * dh
    B = 4
    lens, cuts, rows = [130, 70, 0, 257], [65, 70, 0, 3], [1, 300, 263, 0]
    n_max, cap = 300, 480
    layer, w = make_layer(17, D, H, "bf16", max_positions=cap)
    cache = K.kvc_cache_create(layer, B, cap, max_chunk_rows=512)
    xp_dev, xp = hidden(17, synth.STREAM_PREFIX_X, B, max(lens), D, "bf16")
    K.kvc_continue_chunk(layer, cache, xp_dev, n_rows=lens)
    K.kvc_truncate(cache, cuts)
    xn_dev, xn = hidden(17, synth.STREAM_X, B, n_max, D, "bf16")
    out, work = K.kvc_continue_chunk(layer, cache, xn_dev, n_rows=rows)
    o = to_f64(out)
    for b in range(B):
        seq = np.concatenate([xp[b, : cuts[b]], xn[b, : rows[b]]])
        if rows[b]:
            ref = A.causal_layer(seq, *w, heads=H, rows=range(cuts[b], cuts[b] + rows[b]))
            assert_parity(o[b, : rows[b]], ref["out"], "bf16", f"seq {b}")
        assert not np.any(o[b, rows[b]:])
        if len(seq):
            full = A.causal_layer(seq, *w, heads=H, rows=[])
            k, v, pos = K.kvc_snapshot(cache, b)
            assert list(pos) == list(range(len(seq)))
            assert_parity(storage_f64(k, "bf16"), full["keys"], "bf16", f"keys {b}")
            assert_parity(storage_f64(v, "bf16"), full["values"], "bf16", f"values {b}")


def test_flash_chunk_prefill_matches_causal_reference():
    """A 300-row bf16 prefill (two query tiles, five key tiles) through the tiled
    projection and the flash kernel matches the float64 causal reference."""
    H, dh, n = 4, 128, 300
    D = H * dh
    layer, w = make_layer(19, D, H, "bf16", max_positions=320)
    x_dev, x = hidden(19, synth.STREAM_PREFIX_X, 1, n, D, "bf16")
    cache = K.kvc_cache_create(layer, 1, 320, max_chunk_rows=512)
    out_chunk, _ = K.kvc_continue_chunk(layer, cache, x_dev)
    ref = A.causal_layer(x[0], *w, heads=H)["out"]
    assert_parity(to_f64(out_chunk)[0], ref, "bf16", "chunk")


def test_flash_chunk_more_items_than_the_order_table():
    """260 sequences x one query tile is more work items than the host's
    heaviest-first table holds: the kernel walks them in sequence order, and every
    ragged sequence (0..16 chunk rows over 0..30 retained rows) still matches."""
    H, dh, B, n_max, cap = 2, 64, 260, 16, 48
    D = H * dh
    layer, w = make_layer(29, D, H, "bf16", max_positions=cap)
    cache = K.kvc_cache_create(layer, B, cap, max_chunk_rows=32)
    cuts = [int(c) for c in synth.uniform_int(29, synth.STREAM_LENGTHS, B, 0, 30)]
    rows = [int(r) for r in synth.uniform_int(31, synth.STREAM_LENGTHS, B, 0, n_max)]
    xp_dev, xp = hidden(29, synth.STREAM_PREFIX_X, B, 30, D, "bf16")
    K.kvc_continue_chunk(layer, cache, xp_dev, n_rows=cuts)
    xn_dev, xn = hidden(29, synth.STREAM_X, B, n_max, D, "bf16")
    out, _ = K.kvc_continue_chunk(layer, cache, xn_dev, n_rows=rows)
    o = to_f64(out)
    for b in range(B):
        if rows[b]:
            seq = np.concatenate([xp[b, : cuts[b]], xn[b, : rows[b]]])
            ref = A.causal_layer(seq, *w, heads=H, rows=range(cuts[b], cuts[b] + rows[b]))
            assert_parity(o[b, : rows[b]], ref["out"], "bf16", f"seq {b}")
        assert not np.any(o[b, rows[b]:])


def test_flash_chunk_rescales_when_scores_rise():
    """Scores that climb by more than 2^8 from one key tile to the next force the
    running maximum up twice (retained keys 0..63 score about -10 in base 2, keys
    64..149 about 0, the chunk's own keys about +10): identity projections without
    rotation, so the oracle sees exactly these scores."""
    import torch
    H, dh, cut, n = 2, 128, 150, 40
    D = H * dh
    eye = torch.eye(D, dtype=torch.bfloat16, device="cuda")
    params = K.kvc_params_create(eye, eye.clone(), eye.clone())
    layer = K.kvc_layer_create(params, H, K.KVC_POS_NONE, 10000.0, 256)
    cache = K.kvc_cache_create(layer, 1, 256, max_chunk_rows=256)
    a = np.sqrt(10.0 * np.sqrt(dh) / 1.4426950408889634)  # a^2 / sqrt(d_h) = 10 / log2(e)
    e = np.full(D, a / np.sqrt(dh))
    noise = 0.3 * synth.normal(41, synth.STREAM_X, (cut + n, D))
    x = noise.copy()
    x[:64] -= e
    x[cut:] += e
    s, xf = synth.quantize(x, "bf16")
    xd = torch.from_numpy(s.view(np.int16).copy()).view(torch.bfloat16).cuda()
    K.kvc_continue_chunk(layer, cache, xd[None, :cut].contiguous())
    out, _ = K.kvc_continue_chunk(layer, cache, xd[None, cut:].contiguous())
    w = np.eye(D)
    ref = A.causal_layer(xf, w, w, w, heads=H, rope=False, rows=range(cut, cut + n))
    assert_parity(to_f64(out)[0], ref["out"], "bf16", "rising scores")


def test_flash_chunk_scores_far_above_the_first_keys():
    """Scores that climb by about 2^200 past the first keys (retained keys 0..63
    score about -100 in base 2, keys 64..149 about 0, the chunk's own keys about
    +100) in the first of two sequences, plain scores in the second: a kernel
    that keeps one reference per query from the first keys would overflow on the
    first sequence, which must still match the oracle like the second."""
    import torch
    H, dh, cut, n = 2, 128, 150, 40
    D = H * dh
    eye = torch.eye(D, dtype=torch.bfloat16, device="cuda")
    params = K.kvc_params_create(eye, eye.clone(), eye.clone())
    layer = K.kvc_layer_create(params, H, K.KVC_POS_NONE, 10000.0, 256)
    cache = K.kvc_cache_create(layer, 2, 256, max_chunk_rows=256)
    a = np.sqrt(100.0 * np.sqrt(dh) / 1.4426950408889634)  # a^2 / sqrt(d_h) = 100 / log2(e)
    e = np.full(D, a / np.sqrt(dh))
    x = 0.3 * synth.normal(43, synth.STREAM_X, (2, cut + n, D))
    x[0, :64] -= e
    x[0, cut:] += e
    s, xf = synth.quantize(x, "bf16")
    xd = torch.from_numpy(s.view(np.int16).copy()).view(torch.bfloat16).cuda()
    K.kvc_continue_chunk(layer, cache, xd[:, :cut].contiguous())
    out, _ = K.kvc_continue_chunk(layer, cache, xd[:, cut:].contiguous())
    w = np.eye(D)
    o = to_f64(out)
    for b in range(2):
        ref = A.causal_layer(xf[b], w, w, w, heads=H, rope=False, rows=range(cut, cut + n))
        assert np.all(np.isfinite(o[b]))
        assert_parity(o[b], ref["out"], "bf16", f"seq {b}")


@pytest.mark.parametrize("B,n_max,H,rows,cuts", [
    # 2250 rows: a partial last row tile, 54 tiles (not a multiple of the eight XCDs)
    (5, 450, 4, [450, 1, 0, 300, 449], [0, 5, 3, 100, 17]),
    # 2048 rows, 48 tiles: the XCD-grouped tile order
    (16, 128, 2, None, [3 * b for b in range(16)]),
])
def test_wide_projection_chunk(B, n_max, H, rows, cuts):
    """Chunks of >= 2048 bf16 rows take the 256 x 256 projection kernel: stored
    keys and values (rotated at next_position + i) and the attention outputs
    match the oracle for ragged rows and retained prefixes."""
    dh = 128
    D = H * dh
    cap = max(cuts) + n_max + 8
    layer, w = make_layer(43, D, H, "bf16", max_positions=cap)
    cache = K.kvc_cache_create(layer, B, cap, max_chunk_rows=n_max)
    xp_dev, xp = hidden(43, synth.STREAM_PREFIX_X, B, max(cuts), D, "bf16")
    K.kvc_continue_chunk(layer, cache, xp_dev, n_rows=cuts)
    xn_dev, xn = hidden(43, synth.STREAM_X, B, n_max, D, "bf16")
    out, _ = K.kvc_continue_chunk(layer, cache, xn_dev, n_rows=rows)
    o = to_f64(out)
    rows = rows or [n_max] * B
    for b in range(B):
        seq = np.concatenate([xp[b, : cuts[b]], xn[b, : rows[b]]])
        full = A.causal_layer(seq, *w, heads=H, rows=range(cuts[b], cuts[b] + rows[b]))
        if rows[b]:
            assert_parity(o[b, : rows[b]], full["out"], "bf16", f"seq {b}")
        assert not np.any(o[b, rows[b]:])
        if len(seq):
            k, v, pos = K.kvc_snapshot(cache, b)
            assert list(pos) == list(range(len(seq)))
            assert_parity(storage_f64(k, "bf16"), full["keys"], "bf16", f"keys {b}")
            assert_parity(storage_f64(v, "bf16"), full["values"], "bf16", f"values {b}")


def test_wide_projection_grouped_heads_and_output_projection():
    """2250 bf16 rows of a grouped layer (8 query heads over 2 key/value heads, d_h
    128, D 1024) with W_o bound: the 256 x 256 projection kernel takes W_q and the
    narrower W_k and W_v column tiles, and the float32 merged heads go through
    W_o; outputs (after W_o), stored keys and values match the float64 grouped
    layer for ragged rows and retained prefixes."""
    D, heads, kv_heads, dh = 1024, 8, 2, 128
    B, n_max = 5, 450
    rows, cuts = [450, 1, 0, 300, 449], [0, 5, 3, 100, 17]
    cap = max(cuts) + n_max + 8
    ws = synth.grouped_weights(61, D, kv_heads * dh, D ** -0.5, "bf16")
    wo_s, wo_f = synth.output_weight(61, D, D ** -0.5, "bf16")
    params = K.kvc_params_create_grouped(*[to_device(s, "bf16") for s, _ in ws], to_device(wo_s, "bf16"))
    layer = K.kvc_layer_create(params, heads, K.KVC_POS_ROPE, 10000.0, cap)
    w = [f for _, f in ws]
    cache = K.kvc_cache_create(layer, B, cap, max_chunk_rows=n_max)
    xp_dev, xp = hidden(62, synth.STREAM_PREFIX_X, B, max(cuts), D, "bf16")
    K.kvc_continue_chunk(layer, cache, xp_dev, n_rows=cuts)
    xn_dev, xn = hidden(62, synth.STREAM_X, B, n_max, D, "bf16")
    out, _ = K.kvc_continue_chunk(layer, cache, xn_dev, n_rows=rows)
    o = to_f64(out)
    for b in range(B):
        seq = np.concatenate([xp[b, : cuts[b]], xn[b, : rows[b]]])
        full = A.causal_layer(seq, *w, heads=heads, kv_heads=kv_heads, wo=wo_f,
                              rows=range(cuts[b], cuts[b] + rows[b]))
        if rows[b]:
            assert_parity(o[b, : rows[b]], full["out"], "bf16", f"seq {b}")
        assert not np.any(o[b, rows[b]:])
        if len(seq):
            k, v, pos = K.kvc_snapshot(cache, b)
            assert k.shape == (kv_heads, len(seq), dh) and list(pos) == list(range(len(seq)))
            assert_parity(storage_f64(k, "bf16"), full["keys"], "bf16", f"keys {b}")
            assert_parity(storage_f64(v, "bf16"), full["values"], "bf16", f"values {b}")


@pytest.mark.parametrize("D,heads,kv_heads,B,wo", [(2048, 16, 16, 5, True), (4096, 32, 8, 32, False),
                                                   (4096, 32, 32, 1, False)])
def test_split_decode_projection(D, heads, kv_heads, B, wo):
    """The decode projection of up to 32 rows at D = 2048 / 4096 splits its
    reduction axis over 4-8 blocks per column tile and adds the float32
    partials in a second kernel (W_o too): outputs, keys and values equal the
    float64 layer over two decode steps."""
    dh = D // heads
    ws = synth.grouped_weights(51, D, kv_heads * dh, D ** -0.5, "bf16")
    tens = [to_device(s, "bf16") for s, _ in ws]
    w = [f for _, f in ws]
    wo_f = None
    if wo:
        wo_s, wo_f = synth.output_weight(51, D, D ** -0.5, "bf16")
        tens.append(to_device(wo_s, "bf16"))
    params = K.kvc_params_create_grouped(*tens)
    layer = K.kvc_layer_create(params, heads, K.KVC_POS_ROPE, 10000.0, 64)
    cache = K.kvc_cache_create(layer, B, 64)
    x_dev, x = hidden(52, synth.STREAM_X, B, 2, D, "bf16")
    outs = []
    for s in range(2):
        out, _ = K.kvc_append_and_attend(layer, cache, x_dev[:, s:s + 1].contiguous())
        outs.append(to_f64(out)[:, 0])
    for b in range(B):
        full = A.causal_layer(x[b], *w, heads=heads, kv_heads=kv_heads, wo=wo_f)
        for s in range(2):
            assert_parity(outs[s][b], full["out"][s], "bf16", f"seq {b} step {s}")
        k, v, _ = K.kvc_snapshot(cache, b)
        assert_parity(storage_f64(k, "bf16"), full["keys"], "bf16", f"keys {b}")
        assert_parity(storage_f64(v, "bf16"), full["values"], "bf16", f"values {b}")


@pytest.mark.parametrize("which", ["key", "value"])
def test_wide_projection_reports_first_nonfinite_flat_index(which):
    """The 2048-row chunk projection (wide MFMA kernel): one W_k (then W_v) output row
    of 3e38 makes feature 5 of every row's key (value) overflow.  The call fails with
    the first non-finite flat index, 5 (sequence 0, head 0, row 0; Chapter 37 cache
    validation reports the first offending element in flat order), and the cache is
    unchanged; the same weights with that row restored project and commit."""
    import torch
    B, n, H, dh = 8, 256, 2, 128
    D = H * dh
    ws = synth.decode_weights(91, D, D ** -0.5, "bf16")
    idx = {"key": 1, "value": 2}[which]
    bad_w = ws[idx][1].copy()
    bad_w[5, :] = 3e38
    tensors = [to_device(s, "bf16") for s, _ in ws]
    tensors[idx] = to_device(synth.quantize(bad_w, "bf16")[0], "bf16")
    layer = K.kvc_layer_create(K.kvc_params_create(*tensors), H, K.KVC_POS_ROPE, 10000.0, 512)
    cache = K.kvc_cache_create(layer, B, 512, max_chunk_rows=n)
    x_dev, _ = hidden(92, synth.STREAM_X, B, n, D, "bf16")
    with pytest.raises(K.KvcError) as ei:
        K.kvc_continue_chunk(layer, cache, x_dev)
    assert ei.value.name == f"KVC_ERR_NONFINITE_{which.upper()}"
    assert ei.value.detail["flat_index"] == 5
    assert [a.tolist() for a in K.kvc_lengths(cache)] == [[0] * B, [0] * B]
    good = K.kvc_layer_create(K.kvc_params_create(*[to_device(s, "bf16") for s, _ in ws]), H, K.KVC_POS_ROPE,
                              10000.0, 512)
    cache = K.kvc_cache_create(good, B, 512, max_chunk_rows=n)
    out, _ = K.kvc_continue_chunk(good, cache, x_dev)
    assert torch.isfinite(out).all() and [a.tolist() for a in K.kvc_lengths(cache)] == [[n] * B, [n] * B]
