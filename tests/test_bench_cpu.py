"""Host logic of bench.py (no GPU): the algorithmic work each roofline divides
by, the measured-traffic table's source-hash check, and the one-GPU refusal."""
import hashlib
import itertools
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_kv_bytes_counts_every_row_read():
    # brute force: each row of each sequence is one K and one V row per key/value head, d_h bf16 values
    rows, kv_heads, dh = [1, 5, 4096], 3, 64
    reads = sum(1 for t in rows for _ in range(t) for _ in range(kv_heads) for _ in ("k", "v"))
    assert bench.decode_kv_bytes(rows, kv_heads, dh) == reads * dh * 2
    # the headline: 32 sequences of 4096 rows, 32 heads of 128: 2 GiB
    assert bench.decode_kv_bytes([4096] * 32, 32, 128) == 2 ** 31


def test_chunk_attention_flops_counts_causal_pairs():
    cuts, n, heads, dh = [0, 3, 7], 5, 2, 16
    pairs = sum(1 for c in cuts for i in range(n) for j in range(c + n) if j <= c + i)
    assert bench.chunk_attention_flops(cuts, n, heads, dh) == pairs * heads * 4 * dh
    # no chunk rows, no work
    assert bench.chunk_attention_flops([10, 20], 0, 4, 64) == 0


def test_chunk_projection_flops():
    rows, D, kv = 6, 8, 4
    macs = rows * (D * D + 2 * kv * D)  # W_q [D, D], W_k and W_v [kv, D]
    assert bench.chunk_projection_flops(rows, D, kv) == 2 * macs
    # the suffix-chunk workload: 4096 rows at D = 4096, all heads: 412.3 GFLOP
    assert bench.chunk_projection_flops(8 * 512, 4096, 4096) == 412316860416


def test_measured_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_bytes(b"// a kernel\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"k": str(src)})
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", {
        "w": {"source": "k", "fetch_kib": 10.0, "fetch_scale": 2.0, "write_kib": 3.0, "write_scale": 1.0,
              "kernel_source_sha256": digest}})
    assert bench.measured_traffic("w") == 10.0 * 1024 * 2.0 + 3.0 * 1024
    assert bench.measured_traffic("other") is None
    src.write_bytes(b"// the kernel changed\n")
    assert bench.measured_traffic("w") is None


def test_committed_traffic_entries_name_existing_sources():
    for name, m in bench.MEASURED_TRAFFIC.items():
        assert m["source"] in bench.KERNEL_SOURCES, name
        assert os.path.exists(bench.KERNEL_SOURCES[m["source"]]), name
        assert len(m["kernel_source_sha256"]) == 64


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
