"""The prefix-reuse note's untrained toy decoder, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Prefix-reuse note, "Work and error over 27 cases": two layers, one head,
width 16, vocabulary 32, float64, absolute sinusoidal position encoding and a
tanh residual; no training, feed-forward block, LayerNorm or tokenizer.  The
article that defines the model is not among the pages, so this is the plainest
model those facts allow:

    h0[p] = E[token_p] + PE(p)
    for each layer:  q, k, v = h @ W^T (one head, d_h = 16, no rotation)
                     a[p]    = sum_{j <= p} softmax_j(q_p . k_j / 4) v_j
                     h[p]    = h[p] + tanh(a[p])
    PE(p, 2i) = sin(p / 10000**(2i/16)),  PE(p, 2i+1) = cos(p / 10000**(2i/16))

The cache keeps, per layer, K, V and the absolute position of every row, plus
``next_position`` (note, "What must be trimmed together").  A model with a
sliding window W (note, "Why a sliding-window partial hit must fall back")
lets the row at position p read positions p - W + 1 .. p only, and its cache
keeps only the most recent rows (``retain``).  Parity of this
model to the note's own model is unpinned (its weights and random generator
are not published); what is pinned is the note's invariants: the reuse path
equals a full recompute and the stale-position path does not.
"""
from __future__ import annotations

import numpy as np

from . import attention as A

F64 = np.float64
WIDTH = 16
VOCAB = 32
LAYERS = 2


def sinusoidal(positions, width: int = WIDTH) -> np.ndarray:
    """Absolute sinusoidal position encoding [len(positions), width] (Vaswani et al.)."""
    p = np.asarray(positions, F64)[:, None]
    i = np.arange(width // 2, dtype=F64)[None, :]
    ang = p / np.power(10000.0, 2.0 * i / width)
    pe = np.zeros((p.shape[0], width), F64)
    pe[:, 0::2] = np.sin(ang)
    pe[:, 1::2] = np.cos(ang)
    return pe


class ToyModel:
    """Embedding [VOCAB, WIDTH] and per layer (W_q, W_k, W_v), each [WIDTH, WIDTH] as [out, in];
    ``window``: sliding-window width W, or None for full causal attention."""

    def __init__(self, embed, layers, window=None):
        self.embed = np.asarray(embed, F64)
        self.layers = [tuple(np.asarray(w, F64) for w in ws) for ws in layers]
        self.window = window


def embed(model: ToyModel, tokens, positions) -> np.ndarray:
    return model.embed[np.asarray(tokens, np.int64)] + sinusoidal(positions, model.embed.shape[1])


def full_forward(model: ToyModel, tokens):
    """Full recompute over ``tokens`` from position 0.

    Returns (final hidden rows [L, WIDTH], cache) where cache is
    ``{'next_position': L, 'layers': [(K [L,16], V [L,16], positions [L]) per layer]}``.
    """
    n = len(tokens)
    pos = np.arange(n)
    h = embed(model, tokens, pos)
    layers = []
    for wq, wk, wv in model.layers:
        r = A.causal_layer(h, wq, wk, wv, heads=1, rope=False, positions=pos, window=model.window)
        layers.append((r["keys"][0].copy(), r["values"][0].copy(), pos.copy()))
        h = h + np.tanh(r["out"])
    return h, {"next_position": n, "layers": layers}


def retain(cache, rows: int):
    """A window cache: keep only the last ``rows`` rows of every layer (their
    positions say which); next_position is unchanged."""
    return {
        "next_position": cache["next_position"],
        "layers": [(k[-rows:].copy(), v[-rows:].copy(), p[-rows:].copy()) for k, v, p in cache["layers"]],
    }


def trim(cache, cut: int, keep_stale_position: bool = False):
    """Copy rows 0..cut-1 of every layer's K, V and positions; next_position = cut.

    With ``keep_stale_position`` the rows are trimmed but next_position keeps the
    old length: the note's negative control, where shapes still agree and
    nothing raises but the suffix is encoded at the wrong positions.
    """
    return {
        "next_position": cache["next_position"] if keep_stale_position else cut,
        "layers": [(k[:cut].copy(), v[:cut].copy(), p[:cut].copy()) for k, v, p in cache["layers"]],
    }


def trim_window(cache, cut: int):
    """A window cache (rows in position order, the oldest ones gone) cut back to
    positions 0..cut-1: it keeps the rows it still holds below ``cut``;
    next_position = cut."""
    out = []
    for k, v, p in cache["layers"]:
        keep = p < cut
        out.append((k[keep].copy(), v[keep].copy(), p[keep].copy()))
    return {"next_position": cut, "layers": out}


def chunk(model: ToyModel, tokens, cache):
    """Compute ``tokens`` as a suffix after the cached rows, from ``next_position``.

    New row i is encoded at position next_position + i and, in each layer,
    reads the cached rows plus new rows 0..i.  Returns (hidden rows [n, 16],
    updated cache).
    """
    n = len(tokens)
    start = cache["next_position"]
    pos = start + np.arange(n)
    h = embed(model, tokens, pos)
    new_layers = []
    for (wq, wk, wv), (kc, vc, pc) in zip(model.layers, cache["layers"]):
        q = A.project(h, wq)
        k = A.project(h, wk)
        v = A.project(h, wv)
        a = np.zeros_like(h)
        for i in range(n):
            keys = np.concatenate([kc, k[: i + 1]])
            vals = np.concatenate([vc, v[: i + 1]])
            if model.window is not None:
                # rows by position: the window of position pos[i]
                seen = np.concatenate([pc, pos[: i + 1]]) > pos[i] - model.window
                keys, vals = keys[seen], vals[seen]
            a[i] = A.attend(q[i], keys, vals)[0]
        new_layers.append((np.concatenate([kc, k]), np.concatenate([vc, v]), np.concatenate([pc, pos])))
        h = h + np.tanh(a)
    return h, {"next_position": start + n, "layers": new_layers}
