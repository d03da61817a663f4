"""Float64 attention oracle: projection, rotary embedding, full-prefix causal attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation follows Chapter 37 ("Keep layer, logical length, and capacity
separate"): batch B, heads H, head width d_h, model width D = H * d_h,
capacity C.  A layer has three projection matrices used on this path,
W_q, W_k, W_v, each stored [D_out, D_in] so that a projected row is
``y[j] = sum_i x[i] * W[j, i]``.  (The chapter never prints its weights; its
fixture uses identity matrices, so the orientation is a convention of ours,
used identically by the library.)

Readings taken where the pages leave a step open:

* Rotary pairing is "rotate half": feature ``i`` pairs with ``i + d_h/2``,
  and pair ``i`` turns by ``p * base**(-2 i / d_h)`` radians at position p.
  Chapter 37 pins the direction only through its d_h = 2 trace, where the
  single pair turns by exactly p radians.
* Scores are scaled by 1/sqrt(d_h) and the softmax subtracts the row maximum
  (Chapter 37, "Bind the state, calculate completely, then commit" and the
  incremental-attention listing's scoring loop).
* The newest query scores itself: the candidate key is the last scored row.
* Grouped key/value heads (Chapter 37, "From causal attention to managed LLM
  inference state": Shazeer's analysis of reloading the retained keys and
  values as the bandwidth bottleneck, and multi-query attention as its remedy).
  A layer may project keys and values to H_kv heads, H_kv dividing H; W_k and
  W_v are then [H_kv * d_h, D] and query head h reads key/value head
  h // (H / H_kv), so consecutive query heads share one key/value head.
  H_kv = 1 is multi-query attention, H_kv = H the chapter's layer.
* Sliding window (prefix-reuse note, "Why a sliding-window partial hit must
  fall back"): with window W, the row at index p reads rows
  max(0, p - W + 1) .. p, and a window cache only needs (and keeps) the most
  recent rows.  W = None reads the whole prefix.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def project(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Rows of ``x`` through one projection: ``y[..., j] = sum_i x[..., i] * w[j, i]``."""
    return np.asarray(x, F64) @ np.asarray(w, F64).T


def split_heads(y: np.ndarray, heads: int) -> np.ndarray:
    """[..., D] -> [..., H, d_h]: head h owns columns h*d_h .. (h+1)*d_h - 1."""
    d = y.shape[-1]
    return y.reshape(y.shape[:-1] + (heads, d // heads))


def merge_heads(o: np.ndarray) -> np.ndarray:
    """[..., H, d_h] -> [..., H*d_h], head blocks in head order."""
    return o.reshape(o.shape[:-2] + (o.shape[-2] * o.shape[-1],))


def rope_angles(position, head_width: int, base: float) -> np.ndarray:
    """Angles p * base**(-2 i / d_h) for the d_h/2 pairs (float64, computed directly)."""
    half = head_width // 2
    i = np.arange(half, dtype=F64)
    inv_freq = np.power(F64(base), -2.0 * i / head_width)
    return np.multiply.outer(np.asarray(position, F64), inv_freq)


def rotate(u: np.ndarray, position, base: float) -> np.ndarray:
    """Rotary embedding of the last axis of ``u`` at ``position`` (scalar or per-row array).

    Pair (a_i, b_i) = (u_i, u_{i+half}) becomes
    (a_i cos t_i - b_i sin t_i, b_i cos t_i + a_i sin t_i).
    Chapter 37, "Append along the position axis": queries and keys are rotated
    at their absolute position, values are never rotated.
    """
    u = np.asarray(u, F64)
    d = u.shape[-1]
    half = d // 2
    ang = rope_angles(position, d, base)
    # broadcast the angle rows against any head axes sitting between them and d
    while ang.ndim < u.ndim:
        ang = np.expand_dims(ang, axis=-2)
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(scores: np.ndarray) -> np.ndarray:
    """Numerically stable softmax over the last axis."""
    s = np.asarray(scores, F64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray):
    """One query over t rows: weights = softmax(q.k_j / sqrt(d_h)), output = sum_j w_j v_j.

    ``q`` [d_h], ``keys``/``values`` [t, d_h].  Returns (output [d_h], weights [t]).
    Chapter 37, incremental-attention listing: scaled dot products, stable
    softmax over the prefix, value mixture.
    """
    d = q.shape[-1]
    w = softmax(keys @ q / np.sqrt(F64(d)))
    return w @ values, w


def layer_projections(x_rows, wq, wk, wv, heads: int, positions, base: float, rope: bool, kv_heads=None):
    """Per-row rotated queries, rotated keys and values for one layer.

    ``x_rows`` [L, D] at absolute ``positions`` [L].  Returns q as [L, H, d_h]
    and k, v as [L, H_kv, d_h] (H_kv = ``kv_heads``, default H).  With
    ``rope=False`` (the prefix-reuse note's absolute-position model) no
    rotation is applied.
    """
    kv_heads = heads if kv_heads is None else kv_heads
    q = split_heads(project(x_rows, wq), heads)
    k = split_heads(project(x_rows, wk), kv_heads)
    v = split_heads(project(x_rows, wv), kv_heads)
    if rope:
        pos = np.asarray(positions, F64)
        q = rotate(q, pos, base)
        k = rotate(k, pos, base)
    return q, k, v


def causal_layer(x_rows, wq, wk, wv, heads: int, base: float = 10000.0,
                 rope: bool = True, positions=None, rows=None, wo=None, kv_heads=None, window=None):
    """Full-prefix causal attention of one layer, recomputed from hidden rows.

    This is the reference every cached result must reproduce (Chapter 37,
    "From causal attention to managed LLM inference state": Vaswani-style
    masked attention; row p reads rows 0..p).  ``x_rows`` [L, D]; positions
    default to 0..L-1.  ``rows`` selects which output rows to compute (default
    all).  ``wo``: the layer's output projection, applied to the merged heads
    (Chapter 37, "Bind the state, calculate completely, then commit": merge
    heads, then the output projection); None returns the merged heads.
    ``kv_heads``: key/value heads H_kv (default H); query head h reads
    key/value head h // (H / H_kv).  ``window``: row p reads rows
    max(0, p - window + 1) .. p only (None: rows 0 .. p).
    Returns dict with ``out`` [len(rows), D], ``keys`` / ``values``
    [H_kv, L, d_h] (the layer's full logical cache), ``weights`` (list per row
    of [H, p+1]).
    """
    x_rows = np.asarray(x_rows, F64)
    n = x_rows.shape[0]
    kv_heads = heads if kv_heads is None else kv_heads
    if heads % kv_heads:
        raise ValueError("key/value heads must divide the query heads")
    group = heads // kv_heads
    if positions is None:
        positions = np.arange(n)
    q, k, v = layer_projections(x_rows, wq, wk, wv, heads, positions, base, rope, kv_heads)
    if rows is None:
        rows = range(n)
    outs, weights = [], []
    for p in rows:
        lo = 0 if window is None else max(0, p - window + 1)
        o_heads, w_heads = [], []
        for h in range(heads):
            o, w = attend(q[p, h], k[lo: p + 1, h // group], v[lo: p + 1, h // group])
            o_heads.append(o)
            w_heads.append(w)
        outs.append(np.concatenate(o_heads))
        weights.append(np.stack(w_heads))
    out = np.stack(outs) if outs else np.zeros((0, x_rows.shape[1]))
    if wo is not None:
        out = project(out, wo)
    return {
        "out": out,
        "keys": np.transpose(k, (1, 0, 2)),
        "values": np.transpose(v, (1, 0, 2)),
        "weights": weights,
    }


def full_prefix_decode(x_rows, wq, wk, wv, heads: int, base: float = 10000.0, rope: bool = True, wo=None,
                       kv_heads=None):
    """Output of the newest row t-1 of a t-row prefix, recomputed from scratch.

    Equivalent to ``causal_layer(...)`` restricted to the last row; returns the
    same dict (``out`` [D], ``weights`` [H, t]).
    """
    n = np.asarray(x_rows).shape[0]
    r = causal_layer(x_rows, wq, wk, wv, heads, base, rope, rows=[n - 1], wo=wo, kv_heads=kv_heads)
    r["out"] = r["out"][0]
    r["weights"] = r["weights"][0]
    return r


# ------------------------------------------------------------------------------
# The incremental steps in the pages' order.  These are NOT what the GPU path is
# compared with (that is the full-prefix definition above); they exist to pin the
# pages' invariants: cached == full prefix, single key -> its value, stale
# next_position diverges.
# ------------------------------------------------------------------------------

class DecodeCache:
    """A one-sequence, one-layer cache as Chapter 37 describes it.

    Fixed capacity, rotated keys and unrotated values stored [H, C, d_h] (H: the
    layer's key/value heads), a
    logical length, and (prefix-reuse note, "What must be trimmed together")
    the absolute position of every row plus ``next_position``.
    """

    def __init__(self, heads: int, head_width: int, capacity: int):
        self.keys = np.zeros((heads, capacity, head_width), F64)
        self.values = np.zeros((heads, capacity, head_width), F64)
        self.positions = np.zeros(capacity, np.int64)
        self.len = 0
        self.next_position = 0
        self.capacity = capacity

    def logical(self):
        return (self.keys[:, : self.len].copy(), self.values[:, : self.len].copy(),
                self.positions[: self.len].copy())


def incremental_step(cache: DecodeCache, x_row, wq, wk, wv, heads: int,
                     base: float = 10000.0, rope: bool = True, kv_heads=None):
    """One checked append-and-attend step (Chapter 37, "Bind the state, calculate
    completely, then commit").

    Projects only the new row, rotates q and k at ``cache.next_position`` (the
    old logical length unless a caller broke that invariant), scores the new
    query against the retained rows plus its own candidate row, mixes values,
    and only then appends the candidate pair and advances the length.  With
    ``kv_heads`` the cache holds H_kv heads and query head h reads h // (H / H_kv).
    Returns (output [D], weights [H, len+1], work dict).
    """
    if cache.len == cache.capacity:
        raise OverflowError("cache is full")
    kv_heads = heads if kv_heads is None else kv_heads
    group = heads // kv_heads
    pos = cache.next_position
    q, k, v = layer_projections(np.asarray(x_row, F64)[None], wq, wk, wv, heads, [pos], base, rope, kv_heads)
    q, k, v = q[0], k[0], v[0]
    outs, ws = [], []
    for h in range(heads):
        j = h // group
        keys = np.concatenate([cache.keys[j, : cache.len], k[j][None]])
        vals = np.concatenate([cache.values[j, : cache.len], v[j][None]])
        o, w = attend(q[h], keys, vals)
        outs.append(o)
        ws.append(w)
    work = {"position": pos, "full_prefix_rows_per_projection": cache.len + 1,
            "incremental_rows_per_projection": 1, "reused_key_value_rows": cache.len}
    # commit
    cache.keys[:, cache.len] = k
    cache.values[:, cache.len] = v
    cache.positions[cache.len] = pos
    cache.len += 1
    cache.next_position += 1
    return np.concatenate(outs), np.stack(ws), work


def truncate(cache: DecodeCache, cut: int, keep_stale_position: bool = False) -> None:
    """Keep rows 0..cut-1 and set next_position = cut (prefix-reuse note, "What
    must be trimmed together").  ``keep_stale_position`` is the note's negative
    control: rows are trimmed but next_position keeps the old length."""
    if not 0 <= cut <= cache.len:
        raise ValueError("cut out of range")
    cache.len = cut
    if not keep_stale_position:
        cache.next_position = cut


def continue_chunk(cache: DecodeCache, x_rows, wq, wk, wv, heads: int,
                   base: float = 10000.0, rope: bool = True):
    """Prefix-reuse note, "What must be trimmed together": compute the suffix rows
    from ``next_position`` on top of the retained rows, then append them.

    New row i sits at position next_position + i and reads the retained rows
    plus new rows 0..i.  Returns (outputs [n, D], work dict).
    """
    x_rows = np.asarray(x_rows, F64)
    n = x_rows.shape[0]
    if cache.len + n > cache.capacity:
        raise OverflowError("chunk exceeds capacity")
    pos = cache.next_position + np.arange(n)
    q, k, v = layer_projections(x_rows, wq, wk, wv, heads, pos, base, rope)
    outs = []
    for i in range(n):
        o_heads = []
        for h in range(heads):
            keys = np.concatenate([cache.keys[h, : cache.len], k[: i + 1, h]])
            vals = np.concatenate([cache.values[h, : cache.len], v[: i + 1, h]])
            o_heads.append(attend(q[i, h], keys, vals)[0])
        outs.append(np.concatenate(o_heads))
    work = {"full_prefix_rows_per_projection": cache.len + n,
            "incremental_rows_per_projection": n, "reused_key_value_rows": cache.len}
    cache.keys[:, cache.len: cache.len + n] = np.transpose(k, (1, 0, 2))
    cache.values[:, cache.len: cache.len + n] = np.transpose(v, (1, 0, 2))
    cache.positions[cache.len: cache.len + n] = pos
    cache.len += n
    cache.next_position += n
    return (np.stack(outs) if n else np.zeros((0, x_rows.shape[1]))), work
