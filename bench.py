"""Decode-step throughput of the layer-bound KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one cached decode step of one layer over the whole batch: the new
rows' Q/K/V projection with RoPE, split-K attention over every retained row
plus the candidate row, the log-sum-exp merge, and the predicated append
(kvc_append_and_attend).  Each step is timed with HIP events recorded on the
cache's stream around that call alone; before each step, outside the event
pair, kvc_truncate cuts the cache back to its starting length so that every
timed step sees the same t (the wall-clock time of the whole loop, truncation
included, is reported beside it).  Inputs (weights, hidden rows, the
prefilled cache) are seeded synthetic data resident in HBM before timing.

The default run (headline workload) also measures the ragged-length decode,
the long-context decode and the suffix-chunk workloads and reports them under
"other_configs" of the same line, with the achievable streaming-read
bandwidth and matrix-core rate of the box as yardsticks.

Workloads (default: headline):
  headline  B=32, H=32, d_h=128, C=4096, t=4096 for every sequence, bf16 K/V
  ragged    same shape, t_b uniform on [1, 4096]
  long      B=4, C=32768, t=32768 for every sequence
  chunk     B=8, C=16384, cut_b uniform on [0, 8192], 512-row suffix chunk per
            sequence (step = truncate to cut + kvc_continue_chunk)
  session   a 4-layer model-wide session of headline-shaped layers (vocab 8192,
            sinusoidal positions, tanh residual), t=4096: step = kvc_session_truncate
            + kvc_session_decode of the whole stack
  paged     headline with block-paged K/V (kvc_cache_create_paged, 512-row blocks,
            pool = B x C / 512 blocks, handed out across sequences by the prefill)
  paged_ragged  ragged lengths with a pool of exactly sum_b ceil(t_b / 512) blocks
  grouped   headline with 8 key/value heads for the 32 query heads (W_k, W_v
            [1024 x 4096]); each decode workgroup serves the 4 query heads of one
            key/value head from one read of its rows

Prints one JSON line (rank 0).  `roofline` describes the dominant kernel, timed
with HIP events recorded by the library on the cache's stream.  `cpu_baseline`
times the float64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/s + KV-read GB/s (% of HBM peak) at B=32,H=32,d_h=128,t=4096"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
SEED = 37

# HBM bytes per launch of each workload's dominant kernel, measured with
# `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` on this bench (KiB per
# dispatch, a timed step's dispatch) and scaled by what the same counters read
# for a plain 1 GiB device copy (bench.py --calibrate-copy-mib 1024):
# FETCH_SIZE reported 0.5 x the bytes the copy read, WRITE_SIZE 1.0 x the bytes
# it wrote.  The figures belong to the kernel source they were taken on; once
# that file changes the bench reports traffic as null until they are measured
# again.
MEASURED_TRAFFIC = {
    # attend_decode_bf16_kernel, headline decode (B=32, t=4096)
    "headline": {"source": "decode", "fetch_kib": 1048893.0, "fetch_scale": 2.0, "write_kib": 512.0, "write_scale": 1.0,
                 "kernel_source_sha256": "ff3b3a9411d402a8edf4b3a8f93d5def7cd1c117ebc40b471aaa0ac8c98fb43f"},
    # project_wide_kernel, suffix chunk (B=8, n=512)
    "chunk": {"source": "mfma", "fetch_kib": 299386.8, "fetch_scale": 2.0, "write_kib": 98304.3, "write_scale": 1.0,
              "kernel_source_sha256": "5e828e7b7beca4c6421b041f2b511451a73ca3425226d96f4f1cf33dd184128b"},
    # attend_split_kernel, suffix chunk (B=8, n=512); the general kernel's launch
    # for handed-back work items (none on this workload) writes nothing and
    # fetches about 30 KiB
    "chunk_attention": {"source": "mfma", "fetch_kib": 338571.3, "fetch_scale": 2.0, "write_kib": 65557.2,
                        "write_scale": 1.0,
                        "kernel_source_sha256": "5e828e7b7beca4c6421b041f2b511451a73ca3425226d96f4f1cf33dd184128b"},
}
KERNEL_SOURCES = {"decode": os.path.join(ROOT, "incremental_kv_cache_amd", "csrc", "kvc_decode.hip"),
                  "mfma": os.path.join(ROOT, "incremental_kv_cache_amd", "csrc", "kvc_mfma.hip")}

WORKLOADS = {
    "headline": dict(B=32, H=32, dh=128, C=4096, t="full", kind="decode"),
    "ragged": dict(B=32, H=32, dh=128, C=4096, t="uniform", kind="decode"),
    "long": dict(B=4, H=32, dh=128, C=32768, t="full", kind="decode"),
    "chunk": dict(B=8, H=32, dh=128, C=16384, cut_max=8192, n=512, kind="chunk"),
    "session": dict(B=32, H=32, dh=128, C=4096, layers=4, vocab=8192, kind="session"),
    "paged": dict(B=32, H=32, dh=128, C=4096, t="full", kind="decode", block_rows=512),
    "paged_ragged": dict(B=32, H=32, dh=128, C=4096, t="uniform", kind="decode", block_rows=512),
    "grouped": dict(B=32, H=32, dh=128, C=4096, t="full", kind="decode", kv_heads=8),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _pool():
    return cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def gen_rows_bf16(stream, B, first, n, D, row_stride, lens=None):
    """[B, n, D] bf16 bit patterns of hidden rows first..first+n-1 (rows beyond lens[b] zero)."""
    from incremental_kv_cache_amd import synth
    out = np.zeros((B, n, D), np.uint16)

    def one(b):
        m = n if lens is None else max(0, min(n, lens[b] - first))
        if m > 0:
            out[b, :m] = synth.round_to_bf16_bits(synth.hidden_rows(SEED, stream, b, first, m, D, row_stride))

    with _pool() as ex:
        list(ex.map(one, range(B)))
    return out


def to_dev_bf16(bits):
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def setup(wl, max_chunk=512):
    """Weights, layer, cache prefilled to each sequence's starting length."""
    import torch
    from incremental_kv_cache_amd import kvcache as K
    from incremental_kv_cache_amd import synth

    B, H, dh, C = wl["B"], wl["H"], wl["dh"], wl["C"]
    D = H * dh
    KVW = wl.get("kv_heads", H) * dh
    t0 = time.time()
    shapes = {synth.STREAM_WQ: (D, D), synth.STREAM_WK: (KVW, D), synth.STREAM_WV: (KVW, D)}
    with _pool() as ex:
        ws = list(ex.map(lambda s: synth.round_to_bf16_bits(synth.normal(SEED, s, shapes[s], std=D ** -0.5)),
                         (synth.STREAM_WQ, synth.STREAM_WK, synth.STREAM_WV)))
    wdev = [to_dev_bf16(w) for w in ws]
    params = K.kvc_params_create_grouped(*wdev) if KVW != D else K.kvc_params_create(*wdev)
    layer = K.kvc_layer_create(params, H, K.KVC_POS_ROPE, 10000.0, C)
    if wl["kind"] == "decode":
        if wl["t"] == "full":
            start = [C - 1] * B
        else:
            start = [int(v) - 1 for v in synth.uniform_int(SEED, synth.STREAM_LENGTHS, B, 1, C)]
    else:
        start = [int(v) for v in synth.uniform_int(SEED, synth.STREAM_LENGTHS, B, 0, wl["cut_max"])]
    br = wl.get("block_rows")
    if br:
        # blocks for every row a step holds (start + the appended row)
        pool = sum((s + 1 + br - 1) // br for s in start)
        cache = K.kvc_cache_create_paged(layer, B, C, br, pool, max_chunk_rows=max_chunk)
    else:
        cache = K.kvc_cache_create(layer, B, C, max_chunk_rows=max_chunk)
    L = max(start)
    pre_out = torch.empty(B, max_chunk, D, dtype=torch.float32, device="cuda")
    for first in range(0, L, max_chunk):
        n = min(max_chunk, L - first)
        rows = [max(0, min(n, s - first)) for s in start]
        bits = gen_rows_bf16(synth.STREAM_PREFIX_X, B, first, n, D, C, start)
        K.kvc_continue_chunk(layer, cache, to_dev_bf16(bits), n_rows=rows,
                             out=pre_out[:, :n] if n == max_chunk else None, flags=K.KVC_ASYNC)
    K.kvc_sync(cache)
    torch.cuda.synchronize()
    ln, _ = K.kvc_lengths(cache)
    assert ln.tolist() == start, "prefill lengths differ"
    log(f"setup: prefilled {sum(start)} rows in {time.time() - t0:.1f}s")
    return dict(weights_bits=ws, wdev=wdev, params=params, layer=layer, cache=cache, start=start, D=D)


def paging_summary(env, wl):
    """Pool geometry of a paged workload next to the contiguous footprint."""
    from incremental_kv_cache_amd import kvcache as K
    cache = env["cache"]
    d = cache.desc
    used, free = K.kvc_pool_usage(cache)
    row_bytes = 2 * wl.get("kv_heads", wl["H"]) * wl["dh"] * 2  # K and V, bf16
    return {"block_rows": d["block_rows"], "pool_blocks": d["pool_blocks"], "blocks_in_use": used,
            "pool_bytes": d["pool_blocks"] * d["block_rows"] * row_bytes,
            "contiguous_bytes": wl["B"] * wl["C"] * row_bytes}


def measured_traffic(name):
    """Counter-derived HBM bytes per launch of the workload's dominant kernel, or
    None if not measured for the current kernel source."""
    import hashlib
    m = MEASURED_TRAFFIC.get(name)
    if not m:
        return None
    with open(KERNEL_SOURCES[m["source"]], "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != m["kernel_source_sha256"]:
            return None
    return m["fetch_kib"] * 1024 * m["fetch_scale"] + m["write_kib"] * 1024 * m["write_scale"]


def decode_kv_bytes(rows, kv_heads, head_width):
    """Algorithmic bytes of one decode attention launch: every row a newest query
    reads (the retained rows plus the candidate, `rows` per sequence), K and V of
    every key/value head, bf16."""
    return sum(2 * kv_heads * t * head_width * 2 for t in rows)


def chunk_attention_flops(cuts, n, heads, head_width):
    """Algorithmic flops of the chunk attention: chunk row i of a sequence cut at c
    attends keys 0 .. c + i; each (query, key) pair costs q.k and p v, 2 d_h flops
    each, per head."""
    return sum(4 * heads * head_width * sum(c + i + 1 for i in range(n)) for c in cuts)


def chunk_projection_flops(rows, model_width, kv_width):
    """Algorithmic flops of the chunk projection: every row through W_q [D, D] and
    W_k, W_v [kv_width, D]."""
    return 2 * rows * model_width * (model_width + 2 * kv_width)


def time_steps(pre, call, steps, warmup):
    """W untimed warm-up steps, then K steps, each `pre()` (outside the timing)
    then `call()` between two HIP events on the current stream (the cache's).
    Returns (mean event ms per step, p10/p50/p90 of the event ms, wall-clock ms
    per step of the whole loop, `pre` and host time included)."""
    import torch
    for _ in range(warmup):
        pre()
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        pre()
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    pct = {"p10": float(np.percentile(ms, 10)), "p50": float(np.percentile(ms, 50)),
           "p90": float(np.percentile(ms, 90))}
    return float(ms.mean()), pct, wall


def stage_times(cache, pre, call, steps):
    """Average per-stage kernel time (ms) from the library's HIP events."""
    import torch
    from incremental_kv_cache_amd import kvcache as K
    K.kvc_profile_enable(cache, steps)
    for _ in range(steps):
        pre()
        call()
    torch.cuda.synchronize()
    ms, calls = K.kvc_profile_read(cache)
    K.kvc_profile_enable(cache, 0)
    return [m / c if c else 0.0 for m, c in zip(ms, calls)][:4]


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def _blas_threads():
    """Threads of the BLAS library numpy calls (the oracle's matrix products)."""
    try:
        from threadpoolctl import threadpool_info
        return {i.get("internal_api", "?"): i.get("num_threads") for i in threadpool_info()
                if i.get("user_api") == "blas"}
    except Exception:
        return {}


def host_info():
    return {"cpu_count": os.cpu_count(), "blas_threads": _blas_threads()}


def cpu_baseline_decode(env, wl, out_gpu, x_bits, budget_s=25.0, step_budget_s=10.0):
    """Float64 oracle on the host, for as many sequences as fit the time budget:
    the full-prefix recompute of the newest row (projection of all t rows plus the
    newest row's attention) and the oracle's own cached step (project the new row,
    attend over its float64 cache of the t-1 retained rows, append).  The cached
    step is short, so each sequence's is repeated (the cache cut back to its t-1
    rows in between, as the oracle's truncate does) until the steps add up to about
    step_budget_s.  Returns the baseline record and the worst difference of those
    rows from the GPU output."""
    from incremental_kv_cache_amd import synth
    from oracle import attention as A
    D, H, dh = env["D"], wl["H"], wl["dh"]
    HK = wl.get("kv_heads", H)
    w = [synth.bf16_bits_to_f64(b) for b in env["weights_bits"]]
    done, t_full, t_inc, worst, steps, reps = 0, 0.0, 0.0, 0.0, 0, 1
    for b in range(wl["B"]):
        s = env["start"][b]
        prefix = synth.bf16_bits_to_f64(synth.round_to_bf16_bits(
            synth.hidden_rows(SEED, synth.STREAM_PREFIX_X, b, 0, s, D, wl["C"])))
        x_new = synth.bf16_bits_to_f64(x_bits[b])
        rows = np.concatenate([prefix, x_new])
        t0 = time.perf_counter()
        ref = A.full_prefix_decode(rows, *w, heads=H, kv_heads=HK)
        t_full += time.perf_counter() - t0
        cache = A.DecodeCache(HK, dh, s + 1)
        cache.keys[:, :s] = ref["keys"][:, :s]
        cache.values[:, :s] = ref["values"][:, :s]
        cache.positions[:s] = np.arange(s)
        cache.len = cache.next_position = s
        t0 = time.perf_counter()
        inc, _, _ = A.incremental_step(cache, x_new[0], *w, heads=H, kv_heads=HK)
        dt = time.perf_counter() - t0
        t_inc += dt
        steps += 1
        if b == 0:
            reps = max(1, int(step_budget_s / (wl["B"] * dt)))
        for _ in range(reps - 1):
            cache.len = cache.next_position = s
            t0 = time.perf_counter()
            A.incremental_step(cache, x_new[0], *w, heads=H, kv_heads=HK)
            t_inc += time.perf_counter() - t0
            steps += 1
        worst = max(worst, float(np.max(np.abs(out_gpu[b] - ref["out"]))),
                    float(np.max(np.abs(out_gpu[b] - inc))))
        done += 1
        if t_full + t_inc >= budget_s:
            break
    return {"value": steps / t_inc, "unit": "tokens/s", "cores": int(_cores()), "kind": "oracle",
            "sample": f"float64 oracle cached step (new-row projection + attention over its float64 cache + "
                      f"append) for sequences 0..{done - 1} of {wl['B']} (t = "
                      f"{', '.join(str(env['start'][b] + 1) for b in range(done))}), {steps} steps "
                      f"({reps} per sequence), {t_inc:.2f}s of CPU work",
            "full_prefix_recompute": {"value": done / t_full, "unit": "tokens/s",
                                      "sample": f"same sequences, projection of all t rows + newest-row "
                                                f"attention, {t_full:.1f}s of CPU work",
                                      "seconds_per_sequence": t_full / done,
                                      "scaled_step_seconds": wl["B"] * t_full / done,
                                      "scaled": f"one sequence's measured time x B = {wl['B']} "
                                                f"(a whole-batch step, not measured)"},
            **host_info()}, worst, done


def cpu_baseline_chunk(env, wl, out_gpu, x_bits, budget_rows=512):
    """Float64 oracle suffix chunk for the sequence with the shortest cut: its retained
    rows go into an oracle cache (untimed), then the oracle's continue_chunk computes
    the chunk rows (timed).  Returns the baseline record and the worst difference
    from the GPU rows."""
    from incremental_kv_cache_amd import synth
    from oracle import attention as A
    D, H, dh = env["D"], wl["H"], wl["dh"]
    w = [synth.bf16_bits_to_f64(b) for b in env["weights_bits"]]
    b = int(np.argmin(env["start"]))
    cut = env["start"][b]
    n = min(budget_rows, wl["n"])
    prefix = synth.bf16_bits_to_f64(synth.round_to_bf16_bits(
        synth.hidden_rows(SEED, synth.STREAM_PREFIX_X, b, 0, cut, D, wl["C"])))
    pre = A.causal_layer(prefix, *w, heads=H, rows=[])
    cache = A.DecodeCache(H, dh, cut + n)
    cache.keys[:, :cut] = pre["keys"]
    cache.values[:, :cut] = pre["values"]
    cache.positions[:cut] = np.arange(cut)
    cache.len = cache.next_position = cut
    xn = synth.bf16_bits_to_f64(x_bits[b, :n])
    t0 = time.perf_counter()
    out, _ = A.continue_chunk(cache, xn, *w, heads=H)
    dt = time.perf_counter() - t0
    worst = float(np.max(np.abs(out_gpu[b, :n] - out)))
    return {"value": n / dt, "unit": "tokens/s", "cores": int(_cores()), "kind": "oracle",
            "sample": f"float64 oracle continue_chunk of {n} rows on sequence {b} (cut {cut}), "
                      f"{dt:.1f}s of CPU work", **host_info()}, worst


def achievable_read_gbps(nbytes=4 << 30, reps=10):
    """Streaming-read bandwidth of a plain read of a 4 GiB buffer (kvc_stream_read),
    timed with events on the current stream."""
    import torch
    from incremental_kv_cache_amd import kvcache as K
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(3):
        K.kvc_stream_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        K.kvc_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbps = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return gbps


def achievable_mfma_tflops(iters=5000, reps=5):
    """bf16 matrix-core rate of a register-only MFMA loop over every compute unit
    (kvc_mfma_rate), timed with events on the current stream."""
    import torch
    from incremental_kv_cache_amd import kvcache as K
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    K.kvc_mfma_rate(iters // 10, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = sum(K.kvc_mfma_rate(iters, sink) for _ in range(reps))
    e1.record()
    torch.cuda.synchronize()
    return flops / (e0.elapsed_time(e1) * 1e-3) / 1e12


def inputs_sha256(env, *arrays):
    """SHA-256 of the workload's synthetic inputs: weight bits, starting lengths,
    and the step's input rows."""
    from incremental_kv_cache_amd import synth
    return synth.sha256(*env["weights_bits"], np.asarray(env["start"], np.int64), *arrays)


def run_decode(name, wl, steps, warmup, cpu):
    import torch
    from incremental_kv_cache_amd import kvcache as K
    from incremental_kv_cache_amd import synth

    env = setup(wl)
    B, H, dh = wl["B"], wl["H"], wl["dh"]
    D = env["D"]
    layer, cache, start = env["layer"], env["cache"], env["start"]
    x_bits = np.stack([synth.round_to_bf16_bits(synth.hidden_rows(SEED, synth.STREAM_X, b, 0, 1, D, 1))
                       for b in range(B)])
    x = to_dev_bf16(x_bits.reshape(B, 1, D).copy())
    out = torch.empty(B, 1, D, dtype=torch.float32, device="cuda")

    def pre():
        K.kvc_truncate(cache, start)

    def call():
        K.kvc_append_and_attend(layer, cache, x, out=out, flags=K.KVC_ASYNC)

    ms, pct, wall_ms = time_steps(pre, call, steps, warmup)
    sec = ms * 1e-3
    K.kvc_sync(cache)
    st = stage_times(cache, pre, call, steps)
    K.kvc_sync(cache)
    paging = paging_summary(env, wl) if wl.get("block_rows") else None
    torch.cuda.synchronize()
    achievable = achievable_read_gbps()
    t = [s + 1 for s in start]
    HK = wl.get("kv_heads", H)
    kv_bytes = decode_kv_bytes(t, HK, dh)
    attend_ms = st[1]
    att_gbps = kv_bytes / (attend_ms * 1e-3) / 1e9
    attn_merge_gbps = kv_bytes / ((st[1] + st[2]) * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": B / sec, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": sec * 1e3, "wall_ms_per_step": wall_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "inputs_sha256": inputs_sha256(env, x_bits),
        "config": {"workload": f"{name}: one-layer cached decode, B={B} H={H} d_h={dh} C={wl['C']} "
                               f"t={'uniform[1,%d]' % wl['C'] if wl['t'] == 'uniform' else t[0]}, bf16 K/V"
                               f"{', block-paged %d-row blocks' % wl['block_rows'] if paging else ''}"
                               f"{', %d key/value heads' % HK if HK != H else ''}, "
                               f"fp32 accumulate", "batch": B, "heads": H, "kv_heads": HK, "head_width": dh,
                   "capacity": wl["C"], "t_mean": float(np.mean(t)), "seed": SEED},
        "kv_read_GBps": attn_merge_gbps, "kv_read_frac_of_peak": attn_merge_gbps / HBM_PEAK_GBPS,
        "step_ms_percentiles": pct,
        "stage_ms": {"project": st[0], "attend": st[1], "merge": st[2], "commit": st[3]},
        "roofline": {"bound": "hbm", "kernel": "attend_decode_bf16_kernel", "achieved": att_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": att_gbps / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(name), "algorithmic_bytes_per_launch": kv_bytes,
                     "achievable_read_GBps": achievable, "frac_of_achievable": att_gbps / achievable},
    }
    if paging:
        res["paging"] = paging
    out_np = out.double().cpu().numpy()[:, 0]
    if cpu:
        cb, worst, n = cpu_baseline_decode(env, wl, out_np, x_bits)
        res["cpu_baseline"] = cb
        res["parity"] = {"sequences": n, "max_abs_err_vs_oracle": worst, "tolerance": 2e-2}
    return res


def run_chunk(name, wl, steps, warmup, cpu):
    import torch
    from incremental_kv_cache_amd import kvcache as K
    from incremental_kv_cache_amd import synth

    env = setup(wl)
    B, H, dh, n = wl["B"], wl["H"], wl["dh"], wl["n"]
    D = env["D"]
    layer, cache, start = env["layer"], env["cache"], env["start"]
    # the chunk rows are the rows that follow each cut (stream X, row-addressable)
    bits = gen_rows_bf16(synth.STREAM_X, B, 0, n, D, n)
    x = to_dev_bf16(bits)
    out = torch.zeros(B, n, D, dtype=torch.float32, device="cuda")

    def pre():
        K.kvc_truncate(cache, start)

    def call():
        K.kvc_continue_chunk(layer, cache, x, out=out, flags=K.KVC_ASYNC)

    ms, pct, wall_ms = time_steps(pre, call, steps, warmup)
    sec = ms * 1e-3
    K.kvc_sync(cache)
    st = stage_times(cache, pre, call, steps)
    K.kvc_sync(cache)
    torch.cuda.synchronize()
    mfma_tf = achievable_mfma_tflops()
    attn_flops = chunk_attention_flops(start, n, H, dh)
    proj_flops = chunk_projection_flops(B * n, D, wl.get("kv_heads", H) * dh)
    att_tf = attn_flops / (st[1] * 1e-3) / 1e12
    proj_tf = proj_flops / (st[0] * 1e-3) / 1e12
    res = {
        "metric": "suffix-chunk tokens/s (MFMA utilisation)", "value": B * n / sec, "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": sec * 1e3, "wall_ms_per_step": wall_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "inputs_sha256": inputs_sha256(env, bits),
        "config": {"workload": f"{name}: suffix chunk n={n}, B={B} H={H} d_h={dh} C={wl['C']} "
                               f"cut uniform[0,{wl['cut_max']}], bf16", "cuts": start, "seed": SEED},
        "step_ms_percentiles": pct,
        "stage_ms": {"project": st[0], "attend": st[1], "merge": st[2], "commit": st[3]},
        # the projection is the step's largest kernel; the attention's figures follow it
        "roofline": {"bound": "mfma", "kernel": "project_wide_kernel", "achieved": proj_tf,
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": proj_tf / BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic(name), "algorithmic_flops_per_launch": proj_flops,
                     "achievable_tflops": mfma_tf, "frac_of_achievable": proj_tf / mfma_tf},
        # the attention stage: the role-split kernel and the general kernel's
        # launch for the work items it hands back (none here)
        "attention_roofline": {"bound": "mfma", "kernel": "attend_split_kernel", "achieved": att_tf,
                               "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": att_tf / BF16_PEAK_TFLOPS,
                               "traffic": measured_traffic("chunk_attention"),
                               "algorithmic_flops_per_launch": attn_flops,
                               "achievable_tflops": mfma_tf, "frac_of_achievable": att_tf / mfma_tf},
    }
    if cpu:
        cb, worst = cpu_baseline_chunk(env, wl, out.double().cpu().numpy(), bits)
        res["cpu_baseline"] = cb
        res["parity"] = {"sequences": 1, "max_abs_err_vs_oracle": worst, "tolerance": 2e-2}
    return res


def run_session(name, wl, steps, warmup, cpu):
    """Whole-stack decode through a kvc_session: embedding, L layers of headline
    shape, residuals, all-layer commit.  The CPU baseline is omitted: the oracle's
    stack recomputes every row of every layer (no cached step)."""
    import torch
    from incremental_kv_cache_amd import kvcache as K
    from incremental_kv_cache_amd import synth

    B, H, dh, C, L, V = wl["B"], wl["H"], wl["dh"], wl["C"], wl["layers"], wl["vocab"]
    D = H * dh
    t0 = time.time()
    layers = []
    with _pool() as ex:
        for l in range(L):
            ws = list(ex.map(lambda st: synth.round_to_bf16_bits(
                synth.normal(SEED + 100 * l, st, (D, D), std=D ** -0.5)),
                (synth.STREAM_WQ, synth.STREAM_WK, synth.STREAM_WV)))
            params = K.kvc_params_create(*[to_dev_bf16(w) for w in ws])
            layers.append(K.kvc_layer_create(params, H, K.KVC_POS_ROPE, 10000.0, C))
    emb = torch.from_numpy(synth.normal(SEED, synth.STREAM_EMBED, (V, D)).astype(np.float32)).cuda()
    sess = K.kvc_session_create(layers, emb, V, K.KVC_PE_SINUSOIDAL, B, C, max_chunk_rows=512)
    start = C - 1
    toks = synth.uniform_int(SEED, synth.STREAM_TOKENS, B * C, 0, V - 1).reshape(B, C).astype(np.int32)
    for first in range(0, start, 512):
        n = min(512, start - first)
        K.kvc_session_chunk(sess, torch.from_numpy(np.ascontiguousarray(toks[:, first:first + n])).cuda(),
                            flags=K.KVC_ASYNC)
    K.kvc_session_sync(sess)
    log(f"setup: {L} layers, prefilled {B * start} rows per layer in {time.time() - t0:.1f}s")
    tok = torch.from_numpy(np.ascontiguousarray(toks[:, start])).cuda()
    out = torch.empty(B, 1, D, dtype=torch.float32, device="cuda")

    def pre():
        K.kvc_session_truncate(sess, [start] * B)

    def call():
        K.kvc_session_decode(sess, tok, out=out, flags=K.KVC_ASYNC)

    ms, pct, wall_ms = time_steps(pre, call, steps, warmup)
    sec = ms * 1e-3
    K.kvc_session_sync(sess)
    for c in sess.caches:
        K.kvc_profile_enable(c, steps)
    for _ in range(steps):
        pre()
        call()
    torch.cuda.synchronize()
    att = []
    for c in sess.caches:
        ms, calls = K.kvc_profile_read(c)
        att.append(ms[1] / calls[1])
        K.kvc_profile_enable(c, 0)
    K.kvc_session_sync(sess)
    kv_bytes = decode_kv_bytes([C] * B, H, dh)  # per layer: t = C rows per lane
    attend_ms = float(np.mean(att))
    att_gbps = kv_bytes / (attend_ms * 1e-3) / 1e9
    return {
        "metric": f"model-wide decode tokens/s ({L} layers)", "value": B / sec, "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": sec * 1e3, "wall_ms_per_step": wall_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{name}: {L}-layer session, B={B} H={H} d_h={dh} C={C} t={C}, vocab {V}, "
                               f"sinusoidal positions, tanh residual, bf16 K/V", "layers": L, "seed": SEED},
        "step_ms_percentiles": pct,
        "attend_ms_per_layer": att,
        "roofline": {"bound": "hbm", "kernel": "attend_decode_bf16_kernel", "achieved": att_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": att_gbps / HBM_PEAK_GBPS,
                     "traffic": None, "algorithmic_bytes_per_launch": kv_bytes},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="headline only: skip the ragged, long-context and suffix-chunk measurements")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times), to scale HBM byte counters")
    a = ap.parse_args()
    if a.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if a.calibrate_copy_mib:
        n = a.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n}))
        return
    from incremental_kv_cache_amd import capi
    capi.lib()  # fails loudly if the HIP library is missing
    wl = WORKLOADS[a.workload]
    fn = {"decode": run_decode, "chunk": run_chunk, "session": run_session}[wl["kind"]]
    res = fn(a.workload, wl, a.steps, a.warmup, not a.no_cpu_baseline)
    if a.workload == "headline" and not a.no_other_configs:
        # the other measured workloads, one after the other on the same GPU
        # (each cache freed before the next is built); no CPU baselines for them
        import gc
        res["other_configs"] = {}
        for other in ("ragged", "long", "chunk"):
            gc.collect()
            torch.cuda.empty_cache()
            log(f"other config: {other}")
            r = {"decode": run_decode, "chunk": run_chunk}[WORKLOADS[other]["kind"]](
                other, WORKLOADS[other], a.steps, a.warmup, False)
            res["other_configs"][other] = {k: r[k] for k in (
                "metric", "value", "unit", "ms_per_step", "wall_ms_per_step", "step_ms_percentiles", "stage_ms",
                "roofline", "attention_roofline", "kv_read_GBps", "kv_read_frac_of_peak", "config",
                "inputs_sha256") if k in r}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
