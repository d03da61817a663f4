"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds input generation only: counter-based random draws, their
mapping to normal and uniform-integer values, and the one-time rounding of
inputs to bfloat16.  It contains none of the attention, projection, rotary or
cache arithmetic, so the HIP path and the float64 oracle can both consume its
output without sharing any of the method's code.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), the generator the incremental-attention
chapter seeds its demo layers with ("Exercise incompatible and invalid calls",
the error-evidence listing).  It is counter based: draw ``i`` of a stream is
``mix(state0 + (i + 1) * GAMMA)``, so any row of any tensor can be regenerated
on its own (the full-shape parity checks regenerate sampled rows this way).

Normals use the Box-Muller transform on one 64-bit draw per value: the high
32 bits give ``u1`` in (0, 1], the low 32 bits give ``u2`` in [0, 1), and the
value is ``sqrt(-2 ln u1) * cos(2 pi u2)``.
"""
from __future__ import annotations

import hashlib

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MUL1 = np.uint64(0xBF58476D1CE4E5B9)
_MUL2 = np.uint64(0x94D049BB133111EB)
_MASK32 = np.uint64(0xFFFFFFFF)

# Stream identifiers: every tensor a workload draws has its own stream so that
# changing one shape never shifts the values of another.
STREAM_LENGTHS = 1
STREAM_X = 2
STREAM_WQ = 3
STREAM_WK = 4
STREAM_WV = 5
STREAM_EMBED = 6
STREAM_TOKENS = 7
STREAM_PREFIX_X = 8
STREAM_EDIT = 9
STREAM_WO = 10
STREAM_TOY_W = 16  # + 3 * layer + {0, 1, 2}


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _MUL1
    z = (z ^ (z >> np.uint64(27))) * _MUL2
    return z ^ (z >> np.uint64(31))


def _stream_state(seed: int, stream: int) -> np.uint64:
    """Initial state of stream ``stream`` under ``seed`` (a mixed seed/stream pair)."""
    with np.errstate(over="ignore"):
        a = np.array([np.uint64(seed & 0xFFFFFFFFFFFFFFFF)], dtype=np.uint64)
        b = np.array([np.uint64(stream & 0xFFFFFFFFFFFFFFFF)], dtype=np.uint64)
        s = _mix(a + _GAMMA) ^ _mix(b * _MUL2 + _GAMMA)
    return s[0]


def splitmix64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Draws ``start .. start+count-1`` of stream ``stream`` (uint64 array)."""
    state0 = _stream_state(seed, stream)
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(state0 + idx * _GAMMA)


def normal(seed: int, stream: int, shape, std: float = 1.0, start: int = 0) -> np.ndarray:
    """float64 N(0, std^2) values, one draw each, laid out row-major in ``shape``."""
    shape = tuple(int(s) for s in np.atleast_1d(shape)) if not isinstance(shape, tuple) else shape
    count = int(np.prod(shape)) if len(shape) else 1
    z = splitmix64(seed, stream, start, count)
    u1 = ((z >> np.uint64(32)).astype(np.float64) + 1.0) * (1.0 / 4294967296.0)
    u2 = (z & _MASK32).astype(np.float64) * (1.0 / 4294967296.0)
    v = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    if std != 1.0:
        v = v * std
    return v.reshape(shape)


def uniform_int(seed: int, stream: int, count: int, low: int, high: int, start: int = 0) -> np.ndarray:
    """Integers uniform on the closed range [low, high] (int64), by 128-bit multiply-shift."""
    span = high - low + 1
    if span <= 0:
        raise ValueError("empty range")
    z = splitmix64(seed, stream, start, count)
    hi = (z >> np.uint64(32)).astype(np.uint64)
    lo = (z & _MASK32).astype(np.uint64)
    # floor(z * span / 2^64) computed exactly from 32-bit halves.
    sp = np.uint64(span)
    with np.errstate(over="ignore"):
        top = hi * sp + ((lo * sp) >> np.uint64(32))
    return (top >> np.uint64(32)).astype(np.int64) + low


# ---------------------------------------------------------------- bfloat16 ---

def round_to_bf16_bits(values: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of ``values``: float64 -> float32 -> bf16, both round-to-nearest-even."""
    f = np.ascontiguousarray(values, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    u = (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16))
    return u.view(np.float32).astype(np.float64)


def quantize(values: np.ndarray, dtype: str) -> tuple[np.ndarray, np.ndarray]:
    """Returns (storage array, exact float64 value) of ``values`` in ``dtype``.

    ``dtype`` is "f64", "f32" or "bf16"; the storage array is what the device
    receives (bf16 as uint16 bit patterns), the float64 array is exactly the
    value those bits hold, which is what the oracle consumes.
    """
    if dtype == "f64":
        s = np.ascontiguousarray(values, dtype=np.float64)
        return s, s.copy()
    if dtype == "f32":
        s = np.ascontiguousarray(values, dtype=np.float32)
        return s, s.astype(np.float64)
    if dtype == "bf16":
        s = round_to_bf16_bits(values)
        return s, bf16_bits_to_f64(s)
    raise ValueError(f"unknown dtype {dtype!r}")


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# --------------------------------------------------------------- workloads ---

def output_weight(seed: int, model_width: int, std: float, dtype: str):
    """W_o as a [D_out, D_in] array: (storage, float64 value)."""
    return quantize(normal(seed, STREAM_WO, (model_width, model_width), std=std), dtype)


def decode_weights(seed: int, model_width: int, std: float, dtype: str):
    """W_q, W_k, W_v as [D_out, D_in] arrays: (storage, float64 value) pairs."""
    out = []
    for stream in (STREAM_WQ, STREAM_WK, STREAM_WV):
        w = normal(seed, stream, (model_width, model_width), std=std)
        out.append(quantize(w, dtype))
    return out


def grouped_weights(seed: int, model_width: int, kv_width: int, std: float, dtype: str):
    """W_q [D, D] and W_k, W_v [kv_width, D] ([D_out, D_in]): (storage, float64 value) pairs."""
    shapes = ((model_width, model_width), (kv_width, model_width), (kv_width, model_width))
    return [quantize(normal(seed, stream, shape, std=std), dtype)
            for stream, shape in zip((STREAM_WQ, STREAM_WK, STREAM_WV), shapes)]


def hidden_rows(seed: int, stream: int, seq: int, first_row: int, rows: int,
                model_width: int, row_stride: int) -> np.ndarray:
    """float64 N(0,1) hidden rows ``first_row .. first_row+rows-1`` of sequence ``seq``.

    Row ``r`` of sequence ``seq`` is draw block ``seq * row_stride + r``, so a
    row can be regenerated alone.
    """
    start = (seq * row_stride + first_row) * model_width
    return normal(seed, stream, (rows, model_width), start=start)


def toy_tokens(seed: int, count: int, vocab: int = 32, start: int = 0) -> np.ndarray:
    return uniform_int(seed, STREAM_TOKENS, count, 0, vocab - 1, start=start)


def toy_model_arrays(seed: int, vocab: int = 32, width: int = 16, layers: int = 2):
    """N(0,1) embedding [vocab, width] and per-layer (W_q, W_k, W_v) [width, width] (float64)."""
    e = normal(seed, STREAM_EMBED, (vocab, width))
    ws = [tuple(normal(seed, STREAM_TOY_W + 3 * l + j, (width, width)) for j in range(3))
          for l in range(layers)]
    return e, ws


def toy_edit_case(seed: int, cached_len: int = 8, query_len: int = 12, vocab: int = 32):
    """Cached token IDs, a query that extends them by ``query_len - cached_len`` IDs and
    replaces one seeded position e in [0, cached_len) by a different ID, and e itself."""
    cached = uniform_int(seed, STREAM_TOKENS, cached_len, 0, vocab - 1)
    extra = uniform_int(seed, STREAM_TOKENS, query_len - cached_len, 0, vocab - 1, start=cached_len)
    e = int(uniform_int(seed, STREAM_EDIT, 1, 0, cached_len - 1)[0])
    shift = int(uniform_int(seed, STREAM_EDIT, 1, 1, vocab - 1, start=1)[0])
    query = np.concatenate([cached, extra]).copy()
    query[e] = (query[e] + shift) % vocab
    return cached, query, e
