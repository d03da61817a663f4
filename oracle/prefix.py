"""Longest-common-prefix cut and projection-row accounting (float-free, exact integers).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numbers


def validate_token_ids(ids) -> list[int]:
    """Non-empty sequence of integer token IDs (prefix-reuse note, "Lookup flow and
    cache ownership", step 1): a float such as 1.0 never counts as ID 1."""
    ids = list(ids)
    if not ids:
        raise ValueError("token IDs must be non-empty")
    for t in ids:
        if isinstance(t, bool) or not isinstance(t, numbers.Integral):
            raise TypeError(f"token ID {t!r} is not an integer")
    return [int(t) for t in ids]


def lcp_cut(cached, query) -> int:
    """Reusable prefix length for a new query over a cached token sequence.

    The reusable part is the *contiguous* common prefix from the start (equal IDs
    after the first difference do not count: prefix-reuse note, "First, one history
    edit"), capped at len(query) - 1 so the last query token is always recomputed
    and yields an output (same note, end of "Lookup flow and cache ownership").
    """
    cached = validate_token_ids(cached) if len(cached) else []
    query = validate_token_ids(query)
    n = 0
    for a, b in zip(cached, query):
        if a != b:
            break
        n += 1
    return min(n, len(query) - 1)


def decode_work(lens_before) -> dict:
    """Projection-row counts of one single-row decode step over a batch (per Q, K or V projection).

    Chapter 37, "Count projection rows, not hardware time": a full-prefix call
    projects len+1 rows, the incremental call projects 1 row and reuses len
    earlier key and value rows.
    """
    lens = [int(x) for x in lens_before]
    return {"full_prefix_rows_per_projection": sum(l + 1 for l in lens),
            "incremental_rows_per_projection": len(lens),
            "reused_key_value_rows": sum(lens)}


def chunk_work(cuts, rows) -> dict:
    """Row counts of a suffix-chunk continuation: cut_b rows reused, n_b rows projected."""
    cuts = [int(x) for x in cuts]
    rows = [int(x) for x in rows]
    return {"full_prefix_rows_per_projection": sum(c + n for c, n in zip(cuts, rows)),
            "incremental_rows_per_projection": sum(rows),
            "reused_key_value_rows": sum(cuts)}


def continuation_projection_rows(layers: int, query_len: int, cut: int) -> tuple[int, int]:
    """(rows this call, rows of a full recompute): layers x {Q,K,V} x tokens
    (prefix-reuse note, the 27-case table and the formula under it)."""
    return 3 * layers * (query_len - cut), 3 * layers * query_len


def window_reuse_cut(cached, query) -> int:
    """The note's conservative rule for a sliding-window cache (prefix-reuse note,
    "Why a sliding-window partial hit must fall back"): the rows before the
    window are gone, so the existing window is reused only when the whole
    cached prefix matches and the query adds a suffix; any partial hit
    recomputes from the start (cut 0)."""
    cut = lcp_cut(cached, query)
    return cut if cut == len(cached) else 0


def window_continuable(length: int, cut: int, window: int, retained: int) -> bool:
    """Whether a window cache holding the last ``retained`` of ``length`` rows can
    continue from ``cut``: the continuation's first row reads rows
    cut - window + 1 .. cut - 1, which must all still be held (or cut = 0,
    a recompute).  The note's rule above is the case that demands cut = length."""
    return cut == 0 or (0 <= cut <= length and cut - window + 1 >= length - retained)
