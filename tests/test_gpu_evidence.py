"""The library's Chapter 37 evidence report against the chapter's printed report (needs an MI355X).

Chapter 37, section "Assemble cached matches, row counts, reset replay, and error
evidence": the report's step, work, reset and errors lines, every figure produced
by the library's own calls (decode steps, a chunk-path full recompute, work
counters, reset and rejected calls read back from the device).  Outputs agree
with the printed nine-decimal values within half a unit of the last printed
place; every other field matches the printed text exactly.
"""
import json
import os
import re

import pytest

from incremental_kv_cache_amd import evidence

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield


def _split_output(line):
    m = re.match(r"^(.*output:\[)([^\]]*)(\])$", line)
    if not m:
        return line, None
    return m.group(1) + m.group(3), [float(v) for v in m.group(2).split(",")]


def test_report_matches_the_printed_report():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p2_trace.json")))
    report = evidence.chapter_report("cuda:0")
    print(report, flush=True)
    got = report.splitlines()
    want = g["report"]
    assert len(got) == len(want)
    for a, b in zip(got, want):
        ta, va = _split_output(a)
        tb, vb = _split_output(b)
        assert ta == tb, (a, b)
        if vb is not None:
            assert len(va) == len(vb)
            assert max(abs(x - y) for x, y in zip(va, vb)) <= 5.1e-10, (a, b)
