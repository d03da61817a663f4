"""Line format of the evidence report (host only): the chapter's printed step line
is reproduced from its own figures (Chapter 37, "Assemble cached matches, row
counts, reset replay, and error evidence"), and values that round to zero print
without a sign."""
import json
import os

import numpy as np

from incremental_kv_cache_amd import evidence


def test_step_line_reproduces_the_printed_lines():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p2_trace.json")))
    for p, step in enumerate(g["steps"]):
        rec = dict(position=p, before=p, after=p + 1, shape=[1, 2, p + 1, 2], diff=-1e-17,
                   output=np.array(step["output"]))
        assert evidence._step_line(rec) == g["report"][p]


def test_signless_zero():
    assert evidence._fmt(-4e-13, 12) == "0.000000000000"
    assert evidence._fmt(-0.0, 9) == "0.000000000"
    assert evidence._fmt(-0.420735492, 9) == "-0.420735492"


def test_trace_inputs_are_the_chapter_rows():
    x = evidence.trace_inputs()
    assert x.shape == (3, 4)
    np.testing.assert_allclose(x[1], [np.cos(1.0), -np.sin(1.0), 0.0, 1.0], rtol=0, atol=0)
