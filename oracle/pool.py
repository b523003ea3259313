"""The oracle over whole tensors, on every host core: `attention` of
oracle/attention.py evaluated per (batch row, query head, block of query
rows) in a pool of worker processes.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: the tests and the
benchmark's CPU-baseline leg use it to compare or time the definition at full
workload sizes. Nothing is reorganised: each task calls the same `attention`
on the rows it owns, which materialises their whole score rows in fp64 as the
definition reads; rows are independent of one another, so splitting the rows
between processes changes no value.

Workers are started fresh (spawned, not forked from the caller, which may hold
a GPU context), limit their BLAS library to one thread each, and read the
inputs from memory-mapped .npy files in a temporary directory, so the inputs
are not copied once per task.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import tempfile
import time

import numpy as np

from .attention import attention, attention_backward, kv_head_of

__all__ = ["attention_parallel", "attention_backward_slices", "default_workers"]

_ARRAYS: dict = {}
_BARRIER = None


def default_workers(limit: int = 16) -> int:
    """Worker count: the cores this process may run on, at most `limit`."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, limit))


def _init(path: str, barrier) -> None:
    global _BARRIER
    _BARRIER = barrier
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass
    for name in os.listdir(path):
        if name.endswith(".npy"):
            _ARRAYS[name[:-4]] = np.load(os.path.join(path, name), mmap_mode="r")


def _sync() -> int:
    _BARRIER.wait(timeout=600)
    return os.getpid()


def _start(ctx, workers: int, path: str):
    """A pool whose workers have all started and loaded their inputs. The
    executor starts a worker per task while none is idle, and each of these
    tasks holds its worker at a barrier until all have arrived, so times taken
    afterwards exclude starting the workers."""
    ex = cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=_init,
                                initargs=(path, ctx.Barrier(workers)))
    pids = {f.result() for f in [ex.submit(_sync) for _ in range(workers)]}
    assert len(pids) == workers
    return ex


def _task(b: int, h: int, r0: int, r1: int, scale: float, kw: dict):
    """O and LSE of rows [r0, r1) of query head h, batch row b."""
    q, k, v = _ARRAYS["q"], _ARRAYS["k"], _ARRAYS["v"]
    H, Hkv = q.shape[1], k.shape[1]
    kh = kv_head_of(h, H, Hkv)
    extra = dict(kw)
    if "doc_ids" in _ARRAYS:
        extra["doc_ids"] = _ARRAYS["doc_ids"][b:b + 1]
    # one query head against its own key/value head (slopes and bias tables
    # indexed by the head's position in the call, so they are sliced too)
    if "alibi_slopes" in _ARRAYS:
        extra["alibi_slopes"] = _ARRAYS["alibi_slopes"][h:h + 1]
    if "rel_bias" in _ARRAYS:
        extra["rel_bias"] = _ARRAYS["rel_bias"][h:h + 1]
    O, L = attention(q[b:b + 1, h:h + 1], k[b:b + 1, kh:kh + 1], v[b:b + 1, kh:kh + 1], scale,
                     rows=np.arange(r0, r1), **extra)
    return b, h, r0, r1, O[0, 0], L[0, 0]


def attention_parallel(q, k, v, scale: float, *, workers: int | None = None, rows_per_task: int = 1024,
                       heads=None, batches=None, doc_ids=None, alibi_slopes=None, rel_bias=None,
                       stats: dict | None = None, **kw):
    """`attention(q, k, v, scale, **kw)` with the rows of every (batch row,
    query head) split into blocks of `rows_per_task` and evaluated in
    `workers` processes. Returns (O, LSE) as `attention` does; heads outside
    `heads` and batch rows outside `batches` are left as NaN. `stats`, if
    given, receives the wall time of the evaluation (started workers, inputs
    loaded) and the worker count."""
    q = np.asarray(q)
    B, H, Sq, D = q.shape
    workers = workers or default_workers()
    heads = list(range(H)) if heads is None else list(heads)
    batches = list(range(B)) if batches is None else list(batches)
    tmp = tempfile.mkdtemp(prefix="oracle_pool_")
    try:
        arrays = dict(q=q, k=k, v=v, doc_ids=doc_ids, alibi_slopes=alibi_slopes, rel_bias=rel_bias)
        for name, a in arrays.items():
            if a is not None:
                a = np.asarray(a)
                if a.dtype.kind == "f" and name in ("q", "k", "v"):
                    # exact for the bf16 and fp32 values the callers pass
                    a32 = a.astype(np.float32)
                    a = a32 if np.array_equal(a32, a) else a.astype(np.float64)
                np.save(os.path.join(tmp, name + ".npy"), a)
        O = np.full((B, H, Sq, D), np.nan)
        L = np.full((B, H, Sq), np.nan)
        tasks = [(b, h, r0, min(Sq, r0 + rows_per_task)) for b in batches for h in heads
                 for r0 in range(0, Sq, rows_per_task)]
        with _start(mp.get_context("spawn"), workers, tmp) as ex:
            t0 = time.perf_counter()
            futs = [ex.submit(_task, b, h, r0, r1, float(scale), kw) for b, h, r0, r1 in tasks]
            for f in cf.as_completed(futs):
                b, h, r0, r1, o, lse = f.result()
                O[b, h, r0:r1] = o
                L[b, h, r0:r1] = lse
        if stats is not None:
            stats.update(seconds=time.perf_counter() - t0, workers=workers, tasks=len(tasks))
        return O, L
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _bwd_task(b: int, h: int, scale: float, kw: dict):
    """Gradients of one (batch row, query head) slice: the oracle's backward
    on that head's query rows against its key/value head (its share of the
    group's dK and dV)."""
    q, k, v, g = _ARRAYS["q"], _ARRAYS["k"], _ARRAYS["v"], _ARRAYS["dout"]
    kh = kv_head_of(h, q.shape[1], k.shape[1])
    extra = dict(kw)
    if "doc_ids" in _ARRAYS:
        extra["doc_ids"] = _ARRAYS["doc_ids"][b:b + 1]
    if "alibi_slopes" in _ARRAYS:
        extra["alibi_slopes"] = _ARRAYS["alibi_slopes"][h:h + 1]
    if "rel_bias" in _ARRAYS:
        extra["rel_bias"] = _ARRAYS["rel_bias"][h:h + 1]
    dq, dk, dv = attention_backward(q[b:b + 1, h:h + 1], k[b:b + 1, kh:kh + 1], v[b:b + 1, kh:kh + 1],
                                    g[b:b + 1, h:h + 1], scale, **extra)
    return b, h, dq[0, 0], dk[0, 0], dv[0, 0]


def attention_backward_slices(q, k, v, dout, scale: float, slices, *, workers: int | None = None,
                              doc_ids=None, alibi_slopes=None, rel_bias=None, stats: dict | None = None,
                              **kw):
    """The oracle's gradients per (batch row, query head) slice in `slices`,
    in `workers` processes: {(b, h): (dQ, dK share, dV share)}. The dK and dV
    of a key/value head are the sums of its query heads' shares."""
    workers = workers or default_workers()
    tmp = tempfile.mkdtemp(prefix="oracle_pool_")
    try:
        for name, a in dict(q=q, k=k, v=v, dout=dout, doc_ids=doc_ids, alibi_slopes=alibi_slopes,
                            rel_bias=rel_bias).items():
            if a is not None:
                np.save(os.path.join(tmp, name + ".npy"), np.asarray(a))
        out = {}
        with _start(mp.get_context("spawn"), workers, tmp) as ex:
            t0 = time.perf_counter()
            futs = [ex.submit(_bwd_task, b, h, float(scale), kw) for b, h in slices]
            for f in cf.as_completed(futs):
                b, h, dq, dk, dv = f.result()
                out[(b, h)] = (dq, dk, dv)
        if stats is not None:
            stats.update(seconds=time.perf_counter() - t0, workers=workers, tasks=len(slices))
        return out
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
