"""Run the oracle over many (batch, head) slices in a process pool — test infrastructure.

Used to time the oracle as a CPU baseline.  Each worker evaluates whole heads with
``attention.attention_forward`` / ``attention_backward`` and one BLAS thread, so the
pool size is the number of cores the oracle uses.  The pool is created with the
``fork`` start method; callers create it before any GPU work in the process.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time

from . import attention

_SHARED = {}


def _init(arrays, scale, causal, window, lengths):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    _SHARED.update(arrays=arrays, scale=scale, causal=causal, window=window, lengths=lengths)


def _one_head(task):
    kind, b, h, keep = task
    res = _eval_head(kind, b, h)
    if keep:
        return res
    # timing only: hand back a checksum instead of the arrays (keeps the pipe traffic out
    # of the measurement)
    return (b, h, float(sum(float(x.sum()) for x in res[2:])))


def _eval_head(kind, b, h):
    a = _SHARED["arrays"]
    s, c, w = _SHARED["scale"], _SHARED["causal"], _SHARED["window"]
    # a padded batch: the sample's own rows (oracle.padded), the rest is zeros
    L = _SHARED["lengths"][b] if _SHARED["lengths"] is not None else a["q"].shape[2]
    o, lse = attention.attention_forward(a["q"][b, h, :L], a["k"][b, h, :L], a["v"][b, h, :L],
                                         s, c, w)
    if kind == "fwd":
        return (b, h, o, lse)
    dq, dk, dv = attention.attention_backward(a["q"][b, h, :L], a["k"][b, h, :L],
                                              a["v"][b, h, :L], a["do"][b, h, :L], s, c, w)
    return (b, h, o, lse, dq, dk, dv)


def blas_info() -> str:
    """The BLAS library numpy calls (vendor and version), as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = libs[0]
            return f"{i.get('internal_api', '?')} {i.get('version') or ''}".strip()
    except Exception:
        pass
    return "unknown BLAS"


def available_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def run_heads(arrays, heads, scale, causal, window, backward=False, workers=None, keep=True,
              lengths=None):
    """Evaluate the listed (b, h) heads; returns (results, seconds, workers_used).

    ``arrays`` maps "q", "k", "v" (and "do" when ``backward``) to float64 [B, H, N, d];
    ``lengths`` (per batch, already clamped to [1, N]) makes them a padded batch, each head
    evaluated on its sample's rows only.  Results then cover those rows only.
    The timed interval covers the pool's work only, not its start-up.  With ``keep`` False
    each result is (b, h, checksum) instead of the output arrays.
    """
    workers = max(1, min(workers or available_cores(), len(heads)))
    kind = "fwdbwd" if backward else "fwd"
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_init,
                  initargs=(arrays, scale, causal, window, lengths)) as pool:
        pool.map(_noop, range(workers))           # start every worker before timing
        t0 = time.perf_counter()
        res = pool.map(_one_head, [(kind, b, h, keep) for b, h in heads], chunksize=1)
        dt = time.perf_counter() - t0
    return res, dt, workers


def _noop(_):
    return None
