"""Evidence report of the library on the Chapter 37 trace, produced by the library's own calls.

Chapter 37 ("Keep the prefix, project only the new row") ends with a report
(section "Assemble cached matches, row counts, reset replay, and error
evidence") of four kinds of facts about its layer cache on the worked trace of
"Advance the layer cache one position at a time":

* one ``step=`` line per decode step: the position, the cache length before and
  after, the shape of the stored keys ``[batch, heads, rows, head_width]``, the
  largest difference between the cached output and a full recompute of the
  prefix, and the output (nine decimals);
* a ``work=`` line: rows projected by full recomputes and by the cached steps,
  rows reused per key/value projection, and the rows the reuse avoided across the
  key and value projections (twice the reused rows);
* a ``reset=`` line: the length before and after a reset, whether the storage
  allocation and its bytes stayed as they were, and whether replaying the steps
  gives identical records;
* an ``errors=`` line: each rejected call the chapter lists, and whether every
  one left the cache as it was.

Here every figure comes from the library on the device: the steps are
``kvc_append_and_attend`` calls, the full recompute is ``kvc_continue_chunk`` of
the whole prefix into a fresh cache (whose last output row is the newest
position's recomputed output), the row counts are the calls' work counters, and
the reset and error facts are read back with ``kvc_lengths``,
``kvc_storage_pointers`` and ``kvc_copy_storage``.  The trace's layer has
identity W_q, W_k, W_v on a width-4 model with two heads of width 2 and rotary
positions (base 10000, four positions); its printed outputs are after an output
projection that swaps the two heads' blocks, which is bound here as W_o.  The
line format follows the chapter's report so that the two can be compared line by
line; a value that rounds to zero prints without a sign.

Run ``python -m incremental_kv_cache_amd.evidence`` on a machine with the GPU.
"""
import math

import numpy as np

from . import kvcache as K

WIDTH, HEADS, HEAD_WIDTH, POSITIONS, ROPE_BASE = 4, 2, 2, 4, 10000.0


def _fmt(x: float, places: int) -> str:
    s = f"{x:.{places}f}"
    return s[1:] if s.startswith("-") and float(s) == 0.0 else s


def _flag(b: bool) -> str:
    return "true" if b else "false"


def trace_inputs() -> np.ndarray:
    """The trace's three input rows (positions 0, 1, 2)."""
    return np.array([[1.0, 0.0, 1.0, 0.0],
                     [math.cos(1.0), -math.sin(1.0), 0.0, 1.0],
                     [math.cos(2.0), -math.sin(2.0), 1.0, 1.0]])


def _tensor(a, device):
    import torch
    return torch.tensor(np.asarray(a, np.float64), dtype=torch.float64, device=device)


def _params(device, width=WIDTH, w_o=True):
    eye = np.eye(width)
    swap = np.roll(eye, width // 2, axis=1) if w_o else None  # out[i] = merged[(i + width/2) % width]
    return K.kvc_params_create(_tensor(eye, device), _tensor(eye, device), _tensor(eye, device),
                               _tensor(swap, device) if w_o else None)


def _layer(params, heads=HEADS, base=ROPE_BASE, positions=POSITIONS):
    return K.kvc_layer_create(params, heads, K.KVC_POS_ROPE, base, positions)


def _state(cache):
    ln, npos = K.kvc_lengths(cache)
    k, v = K.kvc_copy_storage(cache)
    return ln.tolist(), npos.tolist(), K.kvc_storage_pointers(cache), k.tobytes(), v.tobytes()


def _steps(layer, cache, x, device):
    """Runs the trace's decode steps; returns one record per step."""
    records = []
    for p in range(len(x)):
        before = int(K.kvc_lengths(cache)[0][0])
        out, work = K.kvc_append_and_attend(layer, cache, _tensor(x[p][None, None, :], device))
        after = int(K.kvc_lengths(cache)[0][0])
        keys = K.kvc_snapshot(cache, 0)[0]
        # full recompute of the prefix 0..p through the chunk path, into a fresh cache
        fresh = K.kvc_cache_create(layer, 1, POSITIONS, max_chunk_rows=len(x))
        full, _ = K.kvc_continue_chunk(layer, fresh, _tensor(x[None, : p + 1, :], device))
        cached = out.double().cpu().numpy()[0, 0]
        recomputed = full.double().cpu().numpy()[0, p]
        records.append(dict(position=p, before=before, after=after, shape=[1] + list(keys.shape),
                            diff=float(np.max(np.abs(cached - recomputed))), output=cached, work=work))
    return records


def _step_line(r) -> str:
    shape = ",".join(str(n) for n in r["shape"])
    out = ",".join(_fmt(float(v), 9) for v in r["output"])
    return (f"step=position:{r['position']} cache:{r['before']}->{r['after']} shape:[{shape}] "
            f"max_abs_diff:{_fmt(r['diff'], 12)} output:[{out}]")


def _rejected(call, cache, names) -> bool:
    """True when `call` raises one of the status names and leaves the cache's
    lengths, storage pointers and storage bytes as they were."""
    before = _state(cache)
    try:
        call()
    except K.KvcError as e:
        return any(e.name.startswith(n) for n in names) and _state(cache) == before
    return False


def _error_evidence(device) -> dict:
    params = _params(device)
    layer = _layer(params)
    single = _tensor(trace_inputs()[0].reshape(1, 1, WIDTH), device)
    res = {}
    c = K.kvc_cache_create(layer, 1, 2)
    K.kvc_append_and_attend(layer, c, single)
    two = _tensor(trace_inputs()[:2].reshape(1, 2, WIDTH), device)
    res["two_tokens"] = _rejected(lambda: K.kvc_append_and_attend(layer, c, two), c,
                                  ["KVC_ERR_SINGLE_TOKEN_REQUIRED"])
    c = K.kvc_cache_create(layer, 1, 1)
    K.kvc_append_and_attend(layer, c, single)
    res["full_cache"] = _rejected(lambda: K.kvc_append_and_attend(layer, c, single), c, ["KVC_ERR_FULL"])
    wider = _layer(_params(device, width=2 * WIDTH))
    c = K.kvc_cache_create(wider, 1, POSITIONS)
    res["model_mismatch"] = _rejected(lambda: K.kvc_append_and_attend(layer, c, single), c,
                                      ["KVC_ERR_CACHE_MODEL_WIDTH_MISMATCH"])
    one_head = _layer(_params(device), heads=1)
    c = K.kvc_cache_create(one_head, 1, POSITIONS)
    res["head_mismatch"] = _rejected(lambda: K.kvc_append_and_attend(layer, c, single), c,
                                     ["KVC_ERR_CACHE_HEAD_COUNT_MISMATCH"])
    rebuilt = _layer(_params(device))
    c = K.kvc_cache_create(rebuilt, 1, POSITIONS)
    res["layer_mismatch"] = _rejected(lambda: K.kvc_append_and_attend(layer, c, single), c,
                                      ["KVC_ERR_CACHE_LAYER_MISMATCH"])
    c = K.kvc_cache_create(layer, 1, POSITIONS)
    K.kvc_append_and_attend(layer, c, single)
    doubled = _layer(params, base=2 * ROPE_BASE)
    res["rope_mismatch"] = _rejected(lambda: K.kvc_append_and_attend(doubled, c, single), c,
                                     ["KVC_ERR_CACHE_ROPE_MISMATCH"])
    more = _layer(params, positions=POSITIONS + 1)
    res["rope_positions_mismatch"] = _rejected(lambda: K.kvc_append_and_attend(more, c, single), c,
                                               ["KVC_ERR_CACHE_ROPE_MISMATCH"])
    c = K.kvc_cache_create(layer, 1, POSITIONS)
    K.kvc_append_and_attend(layer, c, single)
    big = _tensor(np.full((1, 1, WIDTH), np.finfo(np.float64).max), device)
    res["nonfinite_projection"] = _rejected(lambda: K.kvc_append_and_attend(layer, c, big), c,
                                            ["KVC_ERR_NONFINITE_"])
    # every case's check already includes "state unchanged"; unchanged summarises them
    res["unchanged"] = all(res.values())
    return res


def chapter_report(device: str = "cuda:0") -> str:
    """The Chapter 37 evidence report of this library, one line per fact group."""
    x = trace_inputs()
    layer = _layer(_params(device))
    cache = K.kvc_cache_create(layer, 1, POSITIONS)
    records = _steps(layer, cache, x, device)
    lines = [_step_line(r) for r in records]
    full = sum(r["work"]["full_prefix_rows_per_projection"] for r in records)
    incr = sum(r["work"]["incremental_rows_per_projection"] for r in records)
    reused = sum(r["work"]["reused_key_value_rows"] for r in records)
    lines.append(f"work=full_rows_per_projection:{full} incremental_rows_per_projection:{incr} "
                 f"reused_rows_per_kv_projection:{reused} avoided_rows_across_kv:{2 * reused}")
    before = int(K.kvc_lengths(cache)[0][0])
    ptrs = K.kvc_storage_pointers(cache)
    storage = K.kvc_copy_storage(cache)
    K.kvc_reset(cache)
    after = int(K.kvc_lengths(cache)[0][0])
    reused_alloc = K.kvc_storage_pointers(cache) == ptrs
    unchanged = all(a.tobytes() == b.tobytes() for a, b in zip(K.kvc_copy_storage(cache), storage))
    replay = _steps(layer, cache, x, device)
    identical = all(
        a["before"] == b["before"] and a["after"] == b["after"] and a["shape"] == b["shape"]
        and a["output"].tobytes() == b["output"].tobytes() and a["diff"] == b["diff"]
        for a, b in zip(records, replay))
    lines.append(f"reset=before:{before} after:{after} allocation_reused:{_flag(reused_alloc)} "
                 f"storage_unchanged:{_flag(unchanged)} replay_identical:{_flag(identical)}")
    errors = _error_evidence(device)
    lines.append("errors=" + " ".join(f"{k}:{_flag(v)}" for k, v in errors.items()))
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    print(chapter_report(), end="")
