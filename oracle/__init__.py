"""Float64 CPU oracle for the incremental KV-cache hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The library under ``incremental_kv_cache_amd`` never imports it and
shares no code with it; the two meet only through the seeded inputs of
``incremental_kv_cache_amd.synth``, which holds no arithmetic of the method.

Sources ("the pages"):

* "Keep the prefix, project only the new row" -- incremental-attention course
  chapter 37 (intale.github.io learn_llm, English and Russian editions),
  cited below as *Chapter 37* with the section heading.
* "LLM mechanism experiment (5): can only the changed suffix be recomputed?"
  (huhohoo.com, longest-prefix-reuse lab note), cited as *Prefix-reuse note*
  with its section heading.

Everything is plain NumPy in float64, written for a reader to check by eye:

* ``attention``   -- rotary position embedding, projections, and the full-prefix
  causal attention that every cached result must reproduce; plus the
  incremental decode and prefix-continuation steps in the pages' order, used
  only to pin the invariants the pages state.
* ``toy_decoder`` -- the prefix-reuse note's two-layer, one-head decoder.
* ``stack``       -- the model-wide stack (embedding, positions, several layers
  with the tanh residual) that a session of per-layer caches must reproduce.
* ``prefix``      -- longest-common-prefix cut and projection-row counts.

Parity status of each function is given in its docstring; the pins live in
``tests/test_oracle_pins.py``.  Functions with no pin say "parity unpinned".
"""
from . import attention, prefix, stack, toy_decoder  # noqa: F401
