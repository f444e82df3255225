"""Runs an oracle function on every (batch, head) pair in a process pool.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: used by ``tests/``
and by the ``cpu_baseline`` leg of ``bench.py``, never by the product path.

Every (batch, head) pair of linear attention has its own state and no pair
reads another's tokens (the pages state the method per head and leave
batching and heads out, "Efficient attention variants" sec. 10), so the
oracle can run the pairs in separate processes without changing a single
operation: each worker calls the same plain function on one pair's arrays,
and the results are stacked back in (batch, head) order.

The pool forks its workers.  ``start`` must run before the calling process
initialises a GPU, so that no worker inherits GPU state; the workers only
run NumPy.  Without a started pool ``map_heads`` runs the pairs one after
another in the calling process.
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

__all__ = ["start", "stop", "processes", "map_heads", "host_cpus"]

_POOL = None
_NPROC = 0


def host_cpus(cap=16):
    """Cores this process may run on (its affinity mask), at most ``cap``."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(n, cap))


def _init_worker():
    # one BLAS thread per worker: the pool itself supplies the parallelism
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass


def start(n=None):
    """Start the worker pool (``n`` processes, default ``host_cpus()``).
    Returns the number of workers."""
    global _POOL, _NPROC
    if _POOL is None:
        _NPROC = int(n or host_cpus())
        if _NPROC > 1:
            _POOL = mp.get_context("fork").Pool(_NPROC, initializer=_init_worker)
        else:
            _NPROC = 1
    return _NPROC


def stop():
    global _POOL, _NPROC
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
    _POOL = None
    _NPROC = 0


def processes():
    """Workers of the running pool (1 when none runs)."""
    return _NPROC if _POOL is not None else 1


def _call(job):
    fn, args, kw = job
    return fn(*args, **kw)


def map_heads(fn, *arrays, head_kw=None, **kw):
    """Call ``fn(a_0[b, h], a_1[b, h], ..., **kw, **head_kw(b, h))`` for every
    (b, h) of the leading [B, H] dimensions of ``arrays`` (``None`` entries
    are passed through as ``None``) and stack each returned array back to
    [B, H, ...].  ``fn`` must be a module-level function.  Returns what
    ``fn`` returns, stacked (a tuple if ``fn`` returns a tuple)."""
    ref = next(a for a in arrays if a is not None)
    B, H = ref.shape[:2]
    jobs = []
    for b in range(B):
        for h in range(H):
            args = tuple(None if a is None else np.ascontiguousarray(a[b, h]) for a in arrays)
            extra = dict(kw)
            if head_kw is not None:
                extra.update(head_kw(b, h))
            jobs.append((fn, args, extra))
    if _POOL is not None:
        results = _POOL.map(_call, jobs, chunksize=1)
    else:
        results = [_call(j) for j in jobs]
    if isinstance(results[0], tuple):
        return tuple(np.stack([r[i] for r in results]).reshape((B, H) + np.shape(results[0][i]))
                     for i in range(len(results[0])))
    return np.stack(results).reshape((B, H) + np.shape(results[0]))
