"""Float64 model-wide stack: embedding, absolute positions and several attention layers.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Chapter 37, "Give every decoder block its own state next": a model-wide
session binds one cache per decoder block and threads them through prefill
and one-token decode.  The block is the prefix-reuse note's toy decoder block
("Work and error over 27 cases": absolute sinusoidal positions, tanh
residual, no feed-forward block or LayerNorm), generalised to layers with
several heads, optional rotary positions and an optional output projection:

    h0[p] = E[token_p] (+ PE(p))
    for each layer:  a = causal attention of h (the layer's own heads, rotary
                         configuration and W_o, as attention.causal_layer)
                     h = h + tanh(a)
    PE(p, 2i) = sin(p / 10000**(2i/D)),  PE(p, 2i+1) = cos(p / 10000**(2i/D))

The plain definition is a full recompute from position 0; a cached session
must equal it row for row.  Pins (tests/test_oracle_pins.py): it reduces to
the toy decoder for two one-head layers of width 16; zero value weights leave
h0 unchanged exactly; a row does not depend on later tokens; the first
layer's keys and values are those of causal_layer on h0.
"""
from __future__ import annotations

import numpy as np

from . import attention as A

F64 = np.float64


def sinusoidal(positions, width: int) -> np.ndarray:
    """Absolute sinusoidal encoding [len(positions), width] (Vaswani et al.)."""
    p = np.asarray(positions, F64)[:, None]
    i = np.arange(width // 2, dtype=F64)[None, :]
    ang = p / np.power(10000.0, 2.0 * i / width)
    pe = np.zeros((p.shape[0], width), F64)
    pe[:, 0::2] = np.sin(ang)
    pe[:, 1::2] = np.cos(ang)
    return pe


class Layer:
    """One attention layer: W_q (and W_o or None) [D, D], W_k and W_v [H_kv * d_h, D], as [out, in]."""

    def __init__(self, wq, wk, wv, heads: int, rope: bool = True, base: float = 10000.0, wo=None, kv_heads=None,
                 window=None):
        self.w = tuple(np.asarray(m, F64) for m in (wq, wk, wv))
        self.wo = None if wo is None else np.asarray(wo, F64)
        self.heads = heads
        self.kv_heads = heads if kv_heads is None else kv_heads
        self.window = window
        self.rope = rope
        self.base = base


def forward(embed, layers, tokens, sinusoidal_pe: bool = True):
    """Full recompute of ``tokens`` from position 0.

    Returns (rows [L, D] after the last layer, per-layer list of (K [H, L, d_h],
    V [H, L, d_h])).
    """
    embed = np.asarray(embed, F64)
    n = len(tokens)
    pos = np.arange(n)
    h = embed[np.asarray(tokens, np.int64)].copy()
    if sinusoidal_pe:
        h = h + sinusoidal(pos, embed.shape[1])
    kv = []
    for lay in layers:
        r = A.causal_layer(h, *lay.w, heads=lay.heads, base=lay.base, rope=lay.rope, positions=pos, wo=lay.wo,
                           kv_heads=lay.kv_heads, window=lay.window)
        kv.append((r["keys"], r["values"]))
        h = h + np.tanh(r["out"])
    return h, kv
