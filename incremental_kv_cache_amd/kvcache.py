"""Python binding of libkvcache with the C ABI's names (argument marshalling only).

Every compute step runs in the HIP kernels of libkvcache.so; this module only
turns torch device tensors and numpy host arrays into pointers and sizes, and
failing statuses into ``KvcError``.  PyTorch provides device memory and the
stream (``torch.cuda.current_stream()``), nothing else.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import capi
from .capi import (KVC_ASYNC, KVC_BF16, KVC_F32, KVC_F64, KVC_PE_NONE, KVC_PE_SINUSOIDAL,  # noqa: F401
                   KVC_POS_NONE, KVC_POS_ROPE, KVC_STAGES, KVC_SYNC, KVC_TRUNCATE_KEEP_STALE_POSITION)


class KvcError(RuntimeError):
    """A non-OK status; ``detail`` mirrors kvc_error_detail."""

    def __init__(self, status: int, name: str, detail: dict):
        super().__init__(f"{name}: {detail.get('message', '')}")
        self.status = status
        self.name = name
        self.detail = detail


def _detail(lib) -> dict:
    d = lib.kvc_last_error().contents
    return {
        "status": d.status, "parameter": d.parameter, "sequence": d.sequence, "layer": d.layer,
        "expected": d.expected, "actual": d.actual,
        "cache_revision": d.cache_revision, "layer_revision": d.layer_revision,
        "flat_index": d.flat_index, "value": d.value,
        "rope_feature_width": tuple(d.rope_feature_width), "rope_max_positions": tuple(d.rope_max_positions),
        "rope_base": tuple(d.rope_base), "message": d.message.decode(errors="replace"),
    }


def _check(lib, st: int) -> None:
    if st != capi.KVC_OK:
        raise KvcError(st, lib.kvc_status_name(st).decode(), _detail(lib))


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float64:
        return KVC_F64
    if t.dtype == torch.float32:
        return KVC_F32
    if t.dtype == torch.bfloat16:
        return KVC_BF16
    raise TypeError(f"unsupported tensor type {t.dtype}")


def _out_dtype(code: int):
    torch = _torch()
    return torch.float64 if code == KVC_F64 else torch.float32


def _check_out(out, shape, code: int, like) -> None:
    """A caller-supplied output must be exactly what the kernels write: the
    accumulate type, the call's shape, on the input's device."""
    want = _out_dtype(code)
    if out.dtype != want:
        raise TypeError(f"out must be {want}, got {out.dtype}")
    if tuple(out.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"out must have shape {tuple(int(v) for v in shape)}, got {tuple(out.shape)}")
    if out.device != like.device:
        raise ValueError(f"out is on {out.device}, the input on {like.device}")


def _rows_arg(n_rows, batch: int):
    """Host int32 [B] row counts (or None) as a pointer; the array is returned to keep it alive."""
    if n_rows is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(n_rows, dtype=np.int32))
    if arr.shape != (batch,):
        raise ValueError(f"n_rows must hold one count per sequence ({batch}), got shape {arr.shape}")
    return arr, arr.ctypes.data_as(capi.PI32)


def _dev_ptr(t) -> int:
    if not t.is_cuda:
        raise TypeError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


class _Handle:
    _destroy = ""

    def __init__(self, lib, ptr):
        self._lib = lib
        self.ptr = ptr

    def close(self):
        if self.ptr:
            getattr(self._lib, self._destroy)(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Params(_Handle):
    _destroy = "kvc_params_destroy"


class Layer(_Handle):
    _destroy = "kvc_layer_destroy"


class Cache(_Handle):
    _destroy = "kvc_cache_destroy"


class Session(_Handle):
    _destroy = "kvc_session_destroy"


class _CacheView(Cache):
    """A session's layer cache: borrowed, never destroyed through this handle."""

    def close(self):
        self.ptr = None


def _lib(lib):
    return lib if lib is not None else capi.lib()


def kvc_params_create(w_q, w_k, w_v, w_o=None, *, lib=None) -> Params:
    """W_q, W_k, W_v (and optionally W_o): contiguous device tensors [D, D] as [out, in], one dtype."""
    lib = _lib(lib)
    code = _dtype_code(w_q)
    ws = (w_q, w_k, w_v) + ((w_o,) if w_o is not None else ())
    if any(_dtype_code(w) != code or tuple(w.shape) != tuple(w_q.shape) for w in ws):
        raise TypeError("weights must share dtype and shape")
    if w_q.dim() != 2 or w_q.shape[0] != w_q.shape[1]:
        raise ValueError("weights must be square [D, D]")
    out = C.c_void_p()
    _check(lib, lib.kvc_params_create(int(w_q.shape[0]), code, _dev_ptr(w_q), _dev_ptr(w_k), _dev_ptr(w_v),
                                      _dev_ptr(w_o) if w_o is not None else None, C.byref(out)))
    h = Params(lib, out)
    h.tensors = ws
    h.dtype_code = code
    h.model_width = int(w_q.shape[0])
    return h


def kvc_params_create_grouped(w_q, w_k, w_v, w_o=None, *, lib=None) -> Params:
    """Grouped key/value heads: W_q (and W_o) [D, D], W_k and W_v [kv_width, D]
    (contiguous device tensors, one dtype); kv_width = H_kv * d_h."""
    lib = _lib(lib)
    code = _dtype_code(w_q)
    ws = (w_q, w_k, w_v) + ((w_o,) if w_o is not None else ())
    if any(_dtype_code(w) != code or w.dim() != 2 for w in ws):
        raise TypeError("weights must be matrices of one dtype")
    d, kvw = int(w_q.shape[0]), int(w_k.shape[0])
    if tuple(w_q.shape) != (d, d) or tuple(w_k.shape) != (kvw, d) or tuple(w_v.shape) != (kvw, d) or (
            w_o is not None and tuple(w_o.shape) != (d, d)):
        raise ValueError("W_q and W_o must be [D, D], W_k and W_v [kv_width, D]")
    out = C.c_void_p()
    _check(lib, lib.kvc_params_create_grouped(d, kvw, code, _dev_ptr(w_q), _dev_ptr(w_k), _dev_ptr(w_v),
                                              _dev_ptr(w_o) if w_o is not None else None, C.byref(out)))
    h = Params(lib, out)
    h.tensors = ws
    h.dtype_code = code
    h.model_width = d
    return h


def kvc_params_mark_updated(params: Params, which: int = -1) -> None:
    _check(params._lib, params._lib.kvc_params_mark_updated(params.ptr, which))


def kvc_layer_create(params: Params, heads: int, pos_mode: int = KVC_POS_ROPE, rope_base: float = 10000.0,
                     rope_max_positions: int = 4096) -> Layer:
    lib = params._lib
    out = C.c_void_p()
    _check(lib, lib.kvc_layer_create(params.ptr, heads, pos_mode, float(rope_base), rope_max_positions,
                                     C.byref(out)))
    h = Layer(lib, out)
    h.params = params
    h.heads = heads
    return h


def _stream_arg(stream):
    if stream is None:
        try:
            stream = _torch().cuda.current_stream().cuda_stream
        except Exception:
            stream = 0
    return C.c_void_p(stream or 0)


def kvc_layer_create_windowed(params: Params, heads: int, window: int, pos_mode: int = KVC_POS_ROPE,
                              rope_base: float = 10000.0, rope_max_positions: int = 4096) -> Layer:
    """A layer whose queries read only the last ``window`` rows (itself included)."""
    lib = params._lib
    out = C.c_void_p()
    _check(lib, lib.kvc_layer_create_windowed(params.ptr, heads, pos_mode, float(rope_base), rope_max_positions,
                                              window, C.byref(out)))
    h = Layer(lib, out)
    h.params = params
    h.heads = heads
    return h


def kvc_reuse_cut(cache: Cache, seq: int, lcp_cut: int) -> int:
    """The cut to continue sequence ``seq`` from, given its longest common prefix."""
    out = C.c_int64()
    _check(cache._lib, cache._lib.kvc_reuse_cut(cache.ptr, seq, int(lcp_cut), C.byref(out)))
    return out.value


def kvc_cache_create(layer: Layer, batch: int, capacity: int, max_chunk_rows: int = 1, stream=None) -> Cache:
    """Allocates the cache on the current device; its work runs on ``stream``
    (default: torch's current stream)."""
    lib = layer._lib
    out = C.c_void_p()
    _check(lib, lib.kvc_cache_create(layer.ptr, batch, capacity, max_chunk_rows, _stream_arg(stream),
                                     C.byref(out)))
    h = Cache(lib, out)
    h.layer = layer
    h.desc = kvc_cache_describe(h)
    return h


def kvc_cache_create_paged(layer: Layer, batch: int, capacity: int, block_rows: int, pool_blocks: int,
                           max_chunk_rows: int = 1, stream=None) -> Cache:
    """A cache whose K/V rows live in a shared pool of ``pool_blocks`` blocks of
    ``block_rows`` rows (same calls and results as kvc_cache_create)."""
    lib = layer._lib
    out = C.c_void_p()
    _check(lib, lib.kvc_cache_create_paged(layer.ptr, batch, capacity, max_chunk_rows, block_rows, pool_blocks,
                                           _stream_arg(stream), C.byref(out)))
    h = Cache(lib, out)
    h.layer = layer
    h.desc = kvc_cache_describe(h)
    return h


def kvc_fork(cache: Cache, src: int, dst: int, rows: int) -> None:
    """Sequence ``dst`` becomes the first ``rows`` rows of ``src`` (next position = rows)."""
    _check(cache._lib, cache._lib.kvc_fork(cache.ptr, src, dst, rows))


def kvc_pool_usage(cache: Cache):
    """(blocks in use, free blocks) of a paged cache's pool."""
    used, free = C.c_int32(), C.c_int32()
    _check(cache._lib, cache._lib.kvc_pool_usage(cache.ptr, C.byref(used), C.byref(free)))
    return used.value, free.value


def kvc_cache_describe(cache: Cache) -> dict:
    d = capi.CacheDesc()
    _check(cache._lib, cache._lib.kvc_cache_describe(cache.ptr, C.byref(d)))
    return {f: getattr(d, f) for f, _ in capi.CacheDesc._fields_}


def kvc_append_and_attend(layer: Layer, cache: Cache, x, out=None, flags: int = KVC_SYNC):
    """x: device tensor [B, 1, D] (any rank is passed through for the rank check).
    Returns (out [B, 1, D], work dict)."""
    return _decode_call("kvc_append_and_attend", layer, cache, x, out, flags)


def kvc_append_and_attend_static(layer: Layer, cache: Cache, x, out=None, flags: int = KVC_SYNC):
    """kvc_append_and_attend whose scratch is the library's static device array:
    the call allocates nothing (pass ``out`` to keep the binding from allocating
    either).  Returns (out [B, 1, D], work dict)."""
    return _decode_call("kvc_append_and_attend_static", layer, cache, x, out, flags)


def _decode_call(name: str, layer: Layer, cache: Cache, x, out, flags: int):
    lib = cache._lib
    code = cache.desc["kv_dtype"]
    if _dtype_code(x) != code:
        raise TypeError("input type differs from the cache's type")
    out_shape = (cache.desc["batch"], 1, cache.desc["model_width"])
    if out is None:
        torch = _torch()
        out = torch.empty(out_shape, dtype=_out_dtype(code), device=x.device)
    _check_out(out, out_shape, code, x)
    shape = (C.c_int64 * max(1, x.dim()))(*[int(s) for s in x.shape])
    w = capi.Work()
    _check(lib, getattr(lib, name)(layer.ptr, cache.ptr, _dev_ptr(x), x.dim(), shape, _dev_ptr(out), flags,
                                   C.byref(w)))
    return out, w.as_dict()


def kvc_continue_chunk(layer: Layer, cache: Cache, x, n_rows=None, out=None, flags: int = KVC_SYNC):
    """x: device tensor [B, n_max, D]; n_rows: host ints [B] or None.  Returns (out, work)."""
    lib = cache._lib
    code = cache.desc["kv_dtype"]
    if _dtype_code(x) != code:
        raise TypeError("input type differs from the cache's type")
    if x.dim() != 3 or x.shape[0] != cache.desc["batch"] or x.shape[2] != cache.desc["model_width"]:
        raise ValueError(f"chunk input must be [B, n, D], got {tuple(x.shape)}")
    n_max = int(x.shape[1])
    arr, rows_ptr = _rows_arg(n_rows, cache.desc["batch"])
    if out is None:
        torch = _torch()
        out = torch.zeros((x.shape[0], n_max, x.shape[2]), dtype=_out_dtype(code), device=x.device)
    _check_out(out, (x.shape[0], n_max, x.shape[2]), code, x)
    w = capi.Work()
    _check(lib, lib.kvc_continue_chunk(layer.ptr, cache.ptr, _dev_ptr(x), n_max, rows_ptr, _dev_ptr(out), flags,
                                       C.byref(w)))
    return out, w.as_dict()


def kvc_newest_weights(cache: Cache, seq: int):
    """Softmax weights [H, rows] (device tensor, accumulate type) of the last
    decode call's query of each head of sequence ``seq`` over its committed rows."""
    torch = _torch()
    lib = cache._lib
    rows = C.c_int32()
    _check(lib, lib.kvc_newest_weights(cache.ptr, seq, None, 0, C.byref(rows)))
    w = torch.zeros((cache.desc["heads"], rows.value), dtype=_out_dtype(cache.desc["kv_dtype"]),
                    device=f"cuda:{cache.desc['device']}")
    _check(lib, lib.kvc_newest_weights(cache.ptr, seq, _dev_ptr(w), rows.value, C.byref(rows)))
    return w


def kvc_truncate(cache: Cache, cut, flags: int = 0) -> None:
    arr = np.ascontiguousarray(np.broadcast_to(np.asarray(cut, dtype=np.int32), (cache.desc["batch"],)))
    _check(cache._lib, cache._lib.kvc_truncate(cache.ptr, arr.ctypes.data_as(capi.PI32), flags))


def kvc_reset(cache: Cache) -> None:
    _check(cache._lib, cache._lib.kvc_reset(cache.ptr))


def kvc_sync(cache: Cache) -> None:
    _check(cache._lib, cache._lib.kvc_sync(cache.ptr))


def kvc_lengths(cache: Cache):
    b = cache.desc["batch"]
    ln = np.zeros(b, np.int32)
    npos = np.zeros(b, np.int32)
    _check(cache._lib, cache._lib.kvc_lengths(cache.ptr, ln.ctypes.data_as(capi.PI32), npos.ctypes.data_as(capi.PI32)))
    return ln, npos


_NP_STORAGE = {KVC_F64: np.float64, KVC_F32: np.float32, KVC_BF16: np.uint16}


def kvc_snapshot(cache: Cache, seq: int):
    """Logical rows of sequence ``seq``: keys, values [H_kv, len, d_h] in the storage
    type (bf16 as uint16 bit patterns) and positions [len]."""
    lib = cache._lib
    rows = C.c_int32()
    _check(lib, lib.kvc_snapshot(cache.ptr, seq, None, None, None, 0, C.byref(rows)))
    n = rows.value
    h, dh = cache.desc["kv_heads"], cache.desc["head_width"]
    dt = _NP_STORAGE[cache.desc["kv_dtype"]]
    k = np.zeros((h, n, dh), dt)
    v = np.zeros((h, n, dh), dt)
    pos = np.zeros(n, np.int32)
    _check(lib, lib.kvc_snapshot(cache.ptr, seq, k.ctypes.data_as(C.c_void_p), v.ctypes.data_as(C.c_void_p),
                                 pos.ctypes.data_as(capi.PI32), n, C.byref(rows)))
    if rows.value != n:
        raise RuntimeError("cache length changed during snapshot")
    return k, v, pos


def kvc_storage_pointers(cache: Cache):
    k, v, n = C.c_void_p(), C.c_void_p(), C.c_int64()
    _check(cache._lib, cache._lib.kvc_storage_pointers(cache.ptr, C.byref(k), C.byref(v), C.byref(n)))
    return k.value, v.value, n.value


def kvc_copy_storage(cache: Cache):
    """Whole physical K and V storage as raw bytes (uint8 arrays)."""
    _, _, n = kvc_storage_pointers(cache)
    k = np.zeros(n, np.uint8)
    v = np.zeros(n, np.uint8)
    _check(cache._lib, cache._lib.kvc_copy_storage(cache.ptr, k.ctypes.data_as(C.c_void_p),
                                                   v.ctypes.data_as(C.c_void_p)))
    return k, v


def kvc_profile_enable(cache: Cache, slots: int) -> None:
    _check(cache._lib, cache._lib.kvc_profile_enable(cache.ptr, slots))


def kvc_profile_read(cache: Cache):
    ms = (C.c_float * KVC_STAGES)()
    calls = (C.c_int32 * KVC_STAGES)()
    _check(cache._lib, cache._lib.kvc_profile_read(cache.ptr, ms, calls))
    return list(ms), list(calls)


def kvc_stream_read(buf, sink, stream=None, *, lib=None) -> None:
    """Launches one streaming read of the whole contiguous device tensor ``buf`` on
    ``stream`` (default: torch's current stream); ``sink`` is a >= 16-byte device tensor."""
    lib = _lib(lib)
    if stream is None:
        stream = _torch().cuda.current_stream().cuda_stream
    nbytes = buf.numel() * buf.element_size()
    _check(lib, lib.kvc_stream_read(_dev_ptr(buf), nbytes, _dev_ptr(sink), C.c_void_p(stream or 0)))


def kvc_mfma_rate(iterations: int, sink, stream=None, *, lib=None) -> float:
    """Launches the matrix-core rate probe on ``stream`` (default: torch's current
    stream); returns the launch's floating-point operations.  ``sink``: >= 16-byte
    device tensor."""
    lib = _lib(lib)
    if stream is None:
        stream = _torch().cuda.current_stream().cuda_stream
    flops = C.c_double()
    _check(lib, lib.kvc_mfma_rate(int(iterations), _dev_ptr(sink), C.c_void_p(stream or 0), C.byref(flops)))
    return flops.value


def kvc_lcp_cut(cached, query, *, lib=None) -> int:
    lib = _lib(lib)
    a = np.ascontiguousarray(np.asarray(cached, dtype=np.int32))
    b = np.ascontiguousarray(np.asarray(query, dtype=np.int32))
    out = C.c_int64()
    _check(lib, lib.kvc_lcp_cut(a.ctypes.data_as(capi.PI32) if a.size else None, a.size,
                                b.ctypes.data_as(capi.PI32) if b.size else None, b.size, C.byref(out)))
    return out.value


def kvc_status_name(status: int, *, lib=None) -> str:
    return _lib(lib).kvc_status_name(status).decode()


def kvc_last_error(*, lib=None) -> dict:
    return _detail(_lib(lib))


# ---- model-wide session ----------------------------------------------------

def kvc_session_create(layers, embedding, vocab: int, position_encoding: int, batch: int, capacity: int,
                       max_chunk_rows: int = 1, stream=None) -> Session:
    """One cache per layer of ``layers`` behind one token stream.  embedding:
    device tensor [vocab, D] in the accumulate type (float64 for f64 layers,
    float32 otherwise)."""
    lib = layers[0]._lib
    if stream is None:
        try:
            stream = _torch().cuda.current_stream().cuda_stream
        except Exception:
            stream = 0
    arr = (C.c_void_p * len(layers))(*[l.ptr for l in layers])
    out = C.c_void_p()
    _check(lib, lib.kvc_session_create(arr, len(layers), _dev_ptr(embedding), vocab, position_encoding, batch,
                                       capacity, max_chunk_rows, C.c_void_p(stream or 0), C.byref(out)))
    h = Session(lib, out)
    h.layers = list(layers)
    h.embedding = embedding
    h.caches = [kvc_session_layer_cache(h, l) for l in range(len(layers))]
    h.desc = h.caches[0].desc
    return h


def kvc_session_layer_cache(session: Session, layer: int) -> Cache:
    """A borrowed view of the session's cache of ``layer`` (read-only calls)."""
    out = C.c_void_p()
    _check(session._lib, session._lib.kvc_session_layer_cache(session.ptr, layer, C.byref(out)))
    c = _CacheView(session._lib, out)
    c.desc = kvc_cache_describe(c)
    c.session = session
    return c


def kvc_session_chunk(session: Session, tokens, n_rows=None, out=None, flags: int = KVC_SYNC):
    """tokens: device int32 tensor [B, n_max]; n_rows: host ints [B] or None.
    Returns (last layer's rows [B, n_max, D], work summed over the layers)."""
    lib = session._lib
    torch = _torch()
    if tokens.dtype != torch.int32 or tokens.dim() != 2:
        raise TypeError("tokens must be a device int32 tensor [B, n]")
    n_max = int(tokens.shape[1])
    batch = session.desc["batch"]
    if tokens.shape[0] != batch:
        raise ValueError(f"tokens must be [B={batch}, n], got {tuple(tokens.shape)}")
    arr, rows_ptr = _rows_arg(n_rows, batch)
    out_shape = (batch, n_max, session.desc["model_width"])
    if out is None:
        out = torch.zeros(out_shape, dtype=_out_dtype(session.desc["kv_dtype"]), device=tokens.device)
    _check_out(out, out_shape, session.desc["kv_dtype"], tokens)
    w = capi.Work()
    _check(lib, lib.kvc_session_chunk(session.ptr, _dev_ptr(tokens), n_max, rows_ptr, _dev_ptr(out), flags,
                                      C.byref(w)))
    return out, w.as_dict()


def kvc_session_decode(session: Session, tokens, out=None, flags: int = KVC_SYNC):
    """tokens: device int32 tensor [B].  Returns (last layer's rows [B, 1, D], work)."""
    lib = session._lib
    torch = _torch()
    if tokens.dtype != torch.int32:
        raise TypeError("tokens must be a device int32 tensor [B]")
    batch = session.desc["batch"]
    if tuple(tokens.shape) != (batch,):
        raise ValueError(f"tokens must be [B={batch}], got {tuple(tokens.shape)}")
    out_shape = (batch, 1, session.desc["model_width"])
    if out is None:
        out = torch.empty(out_shape, dtype=_out_dtype(session.desc["kv_dtype"]), device=tokens.device)
    _check_out(out, out_shape, session.desc["kv_dtype"], tokens)
    w = capi.Work()
    _check(lib, lib.kvc_session_decode(session.ptr, _dev_ptr(tokens), _dev_ptr(out), flags, C.byref(w)))
    return out, w.as_dict()


def kvc_session_truncate(session: Session, cut, flags: int = 0) -> None:
    arr = np.ascontiguousarray(np.broadcast_to(np.asarray(cut, dtype=np.int32), (session.desc["batch"],)))
    _check(session._lib, session._lib.kvc_session_truncate(session.ptr, arr.ctypes.data_as(capi.PI32), flags))


def kvc_session_reset(session: Session) -> None:
    _check(session._lib, session._lib.kvc_session_reset(session.ptr))


def kvc_session_sync(session: Session) -> None:
    _check(session._lib, session._lib.kvc_session_sync(session.ptr))
