"""Full-size parity in the launch configuration bench.py times (needs an MI355X).

The decode workloads (B=32, H=32, d_h=128, C=4096 with t=4096 or ragged t; B=4,
C=32768) and the suffix-chunk workload (B=8, C=16384, cut uniform on
[0, 8192], 512-row chunk) are prefilled and stepped exactly as the bench does.
The float64 oracle is too slow for every output, so sampled sequences are
recomputed from their hidden rows in full (projection of every row plus the
newest rows' attention), and sampled stored rows are compared with their
float64 projections.  Tolerance: bf16 storage with float32 accumulation,
2e-2 max-abs.
"""
import numpy as np
import pytest

import bench
from incremental_kv_cache_amd import kvcache as K
from incremental_kv_cache_amd import synth
from oracle import attention as A

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield


def _weights(env):
    return [synth.bf16_bits_to_f64(b) for b in env["weights_bits"]]


def _prefix_rows(b, n, D, stride):
    return synth.bf16_bits_to_f64(synth.round_to_bf16_bits(
        synth.hidden_rows(bench.SEED, synth.STREAM_PREFIX_X, b, 0, n, D, stride)))


@pytest.mark.parametrize("workload,samples", [("headline", [0, 31]), ("ragged", [0, 7, 29]), ("long", [3])])
def test_fullsize_decode_sampled(workload, samples):
    import torch
    wl = bench.WORKLOADS[workload]
    env = bench.setup(wl)
    B, H, D, C = wl["B"], wl["H"], env["D"], wl["C"]
    layer, cache, start = env["layer"], env["cache"], env["start"]
    x_bits = np.stack([synth.round_to_bf16_bits(synth.hidden_rows(bench.SEED, synth.STREAM_X, b, 0, 1, D, 1))
                       for b in range(B)])
    x = bench.to_dev_bf16(x_bits.reshape(B, 1, D).copy())
    out, work = K.kvc_append_and_attend(layer, cache, x)
    o = out.double().cpu().numpy()[:, 0]
    assert work["full_prefix_rows_per_projection"] == sum(s + 1 for s in start)
    ln, npos = K.kvc_lengths(cache)
    assert ln.tolist() == [s + 1 for s in start] and npos.tolist() == ln.tolist()
    w = _weights(env)
    rng = np.random.default_rng(5)
    for b in samples:
        rows = np.concatenate([_prefix_rows(b, start[b], D, C), synth.bf16_bits_to_f64(x_bits[b])])
        ref = A.full_prefix_decode(rows, *w, heads=H)
        err = float(np.max(np.abs(o[b] - ref["out"])))
        assert err <= TOL, (workload, b, err)
        k, v, pos = K.kvc_snapshot(cache, b)
        t = start[b] + 1
        assert list(pos[[0, t - 1]]) == [0, t - 1]
        pick = np.unique(np.concatenate([[0, t - 1], rng.integers(0, t, 62)]))
        kr = synth.bf16_bits_to_f64(k[:, pick])
        vr = synth.bf16_bits_to_f64(v[:, pick])
        assert float(np.max(np.abs(kr - ref["keys"][:, pick]))) <= TOL
        assert float(np.max(np.abs(vr - ref["values"][:, pick]))) <= TOL
    torch.cuda.synchronize()


def test_fullsize_chunk_sampled():
    import torch
    wl = bench.WORKLOADS["chunk"]
    env = bench.setup(wl)
    B, H, D, C, n = wl["B"], wl["H"], env["D"], wl["C"], wl["n"]
    layer, cache, cuts = env["layer"], env["cache"], env["start"]
    bits = bench.gen_rows_bf16(synth.STREAM_X, B, 0, n, D, n)
    x = bench.to_dev_bf16(bits)
    K.kvc_truncate(cache, cuts)
    out, work = K.kvc_continue_chunk(layer, cache, x)
    o = out.double().cpu().numpy()
    assert work["incremental_rows_per_projection"] == B * n
    assert work["reused_key_value_rows"] == sum(cuts)
    assert K.kvc_lengths(cache)[0].tolist() == [c + n for c in cuts]
    w = _weights(env)
    # every chunk row (both 256-query tiles, every 128-key tile edge) of the
    # sequences with the shortest, the median and the longest cut
    order = np.argsort(cuts, kind="stable")
    for b in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        print(f"chunk parity: sequence {b}, cut {cuts[b]}, rows 0..{n - 1}", flush=True)
        rows = np.concatenate([_prefix_rows(b, cuts[b], D, C), synth.bf16_bits_to_f64(bits[b])])
        ref = A.causal_layer(rows, *w, heads=H, rows=range(cuts[b], cuts[b] + n))
        err = np.abs(o[b] - ref["out"])
        worst = np.unravel_index(int(np.argmax(err)), err.shape)
        assert float(err.max()) <= TOL, (b, cuts[b], worst, float(err.max()))
        k, v, pos = K.kvc_snapshot(cache, b)
        assert pos.tolist() == list(range(cuts[b] + n))
        tail = slice(cuts[b], cuts[b] + n)
        assert float(np.max(np.abs(synth.bf16_bits_to_f64(k[:, tail]) - ref["keys"][:, tail]))) <= TOL
        assert float(np.max(np.abs(synth.bf16_bits_to_f64(v[:, tail]) - ref["values"][:, tail]))) <= TOL
    torch.cuda.synchronize()
