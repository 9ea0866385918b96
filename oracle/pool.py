"""Run the fp64 oracle's per-rank attention with its heads spread over
worker processes.

TEST INFRASTRUCTURE, like the rest of this package: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it. It adds no arithmetic: every worker calls ``cp_oracle.rank_attention``
(or ``causal_attention``) unchanged on the query heads of one or more KV
heads, and the parent places the results. Each query head's rows depend only
on that head and its KV head, so the assembled result is the single-process
one (up to the BLAS library's own summation order, ~1e-16 relative).

Process workers are started with the "spawn" method (fresh interpreters
that never touch a GPU) and read the inputs from memory-mapped files (under
/dev/shm when it has room), so nothing large is pickled. Thread workers share this process's
arrays. Either way BLAS is limited to one thread per worker; the worker
count is the parallelism.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile
import time
from typing import Optional, Sequence

import numpy as np

from . import cp_oracle

__all__ = ["default_workers", "rank_attention_pooled", "rank_attention_backward_pooled"]

_W = {}  # per worker: the memory-mapped inputs and the BLAS limiter


def default_workers(cap: int = 16) -> int:
    """Cores this process may run on (its affinity mask), at most ``cap``."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def _init(folder: str, barrier) -> None:
    _W["barrier"] = barrier
    try:
        from threadpoolctl import threadpool_limits

        _W["limit"] = threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass
    for name in ("q", "k", "v"):
        _W[name] = np.load(os.path.join(folder, name + ".npy"), mmap_mode="r")


def _task(job):
    return _compute(_W, job)


def _compute(inputs, job):
    """One rank_attention call: the query heads ``heads`` of KV head ``kvh``
    on the local rows ``rows``."""
    heads, kvh, n_img, cu, P, r, rows, split, literal = job
    t0 = time.perf_counter()
    q = np.asarray(inputs["q"][:, heads], dtype=np.float64)
    k = np.asarray(inputs["k"][:, [kvh]], dtype=np.float64)
    v = np.asarray(inputs["v"][:, [kvh]], dtype=np.float64)
    out, lse = cp_oracle.rank_attention(q, k, v, n_img, cu, P, r, local_rows=rows, literal=literal,
                                        split=split)
    return out, lse, time.perf_counter() - t0


def rank_attention_pooled(q, k, v, n_img, cu_seqlens, cp_size: int, cp_rank: int,
                          local_rows: Optional[Sequence[int]] = None, split: str = "head_tail",
                          literal: bool = False, heads: Optional[Sequence[int]] = None,
                          workers: Optional[int] = None, stats: Optional[dict] = None,
                          timeout_s: float = 900.0, row_chunk: Optional[int] = None,
                          executor: str = "process"):
    """``cp_oracle.rank_attention`` over the query heads ``heads`` (all if
    None), each KV group's heads in a worker process.

    q [T, H, D], k and v [T, Hkv, D]: numpy arrays or CPU torch tensors
    (torch bf16 and fp32 values are written exactly as float32; numpy
    float32 and float64 arrays keep their dtype).
    Returns out [R', len(heads), D] and lse [len(heads), R'] for the rows
    ``local_rows`` (all rank rows if None), in the order of ``heads``.
    ``executor``: "process" (spawned workers, as above) or "thread" (threads
    of this process over the same tasks: numpy releases the interpreter
    lock in its array loops, and nothing is started outside this process,
    which suits a caller that already holds a GPU context).
    ``row_chunk`` also splits the rows into tasks of at most that many rows
    (each task is still one ``rank_attention`` call on its rows).
    ``stats``, if given, receives the worker count and the wall time of the
    parallel part (inputs already written). Raises TimeoutError if the
    workers have not finished after ``timeout_s`` seconds (a worker that
    died would otherwise leave the pool waiting for ever). The calling
    program's main module must be import-safe (``if __name__ ==
    "__main__"``), as for any spawned pool.
    """
    q, k, v = (_as_array(x) for x in (q, k, v))
    T, H, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    heads = list(range(H)) if heads is None else [int(h) for h in heads]
    groups = {}
    for pos, h in enumerate(heads):
        groups.setdefault(h // G, []).append((pos, h))
    jobs, places = [], []
    n_img = None if n_img is None else np.asarray(n_img)
    cu = None if cu_seqlens is None else np.asarray(cu_seqlens)
    if local_rows is None:
        index, _ = cp_oracle.partition_index(T, n_img, cu, cp_size, cp_rank, split)
        local_rows = np.arange(len(index))
    rows = np.asarray(local_rows, dtype=np.int64)
    R = len(rows)
    step = R if not row_chunk else max(1, int(row_chunk))
    for g, members in sorted(groups.items()):
        for r0 in range(0, max(R, 1), step):
            sel = rows[r0:r0 + step]
            jobs.append(([h for _, h in members], g, n_img, cu, int(cp_size), int(cp_rank), sel, split,
                         literal))
            places.append(([pos for pos, _ in members], r0, len(sel)))
    n_workers = min(workers or default_workers(), len(jobs))
    if executor == "thread":
        results, wall = _run_threads(q, k, v, jobs, n_workers, timeout_s)
    elif executor == "process":
        results, wall = _run_processes(q, k, v, jobs, n_workers, timeout_s)
    else:
        raise ValueError(f"executor must be 'process' or 'thread', not {executor!r}")
    out = np.zeros((R, len(heads), D))
    lse = np.full((len(heads), R), -np.inf)
    for (o, l_, _), (pos, r0, n) in zip(results, places):
        out[r0:r0 + n, pos] = o
        lse[pos, r0:r0 + n] = l_
    if stats is not None:
        stats.update({"workers": n_workers, "executor": executor, "wall_s": wall,
                      "worker_s": float(sum(x[2] for x in results))})
    return out, lse


def _run_threads(q, k, v, jobs, n_workers, timeout_s):
    from concurrent.futures import ThreadPoolExecutor

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    inputs = {"q": q, "k": k, "v": v}
    limit = threadpool_limits(1) if threadpool_limits else None
    try:
        with ThreadPoolExecutor(n_workers) as ex:
            t0 = time.perf_counter()
            futs = [ex.submit(_compute, inputs, job) for job in jobs]
            results = [f.result(timeout=timeout_s) for f in futs]
            wall = time.perf_counter() - t0
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return results, wall


def _scratch_dir(nbytes: int) -> Optional[str]:
    """/dev/shm (memory) when it has room for the inputs twice over, else
    the default temporary directory."""
    try:
        if os.path.isdir("/dev/shm") and shutil.disk_usage("/dev/shm").free > 2 * nbytes:
            return "/dev/shm"
    except OSError:  # pragma: no cover
        pass
    return None


def _run_processes(q, k, v, jobs, n_workers, timeout_s):
    folder = tempfile.mkdtemp(prefix="cp_oracle_", dir=_scratch_dir(q.nbytes + k.nbytes + v.nbytes))
    try:
        for name, arr in (("q", q), ("k", k), ("v", v)):
            np.save(os.path.join(folder, name + ".npy"), arr)
        ctx = mp.get_context("spawn")
        barrier = ctx.Barrier(n_workers)
        with ctx.Pool(n_workers, initializer=_init, initargs=(folder, barrier)) as pool:
            # every worker is up (inputs mapped) before the clock starts: each
            # of these tasks waits until all workers hold one
            pool.map_async(_ready, range(n_workers), chunksize=1).get(timeout_s)
            t0 = time.perf_counter()
            results = pool.map_async(_task, jobs, chunksize=1).get(timeout_s)
            wall = time.perf_counter() - t0
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    return results, wall


def _ready(_):
    _W["barrier"].wait()
    return os.getpid()


def _as_array(x) -> np.ndarray:
    """torch bf16/fp32 tensors as float32 (exact); numpy float64 stays float64."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    return np.ascontiguousarray(a if a.dtype in (np.float32, np.float64) else a.astype(np.float64))


def _backward_task(inputs, job):
    """One rank_attention_backward call: the query heads ``heads`` of KV head
    ``kvh``, the terms of the local rows ``rows``."""
    heads, kvh, n_img, cu, P, r, rows, split = job
    q = np.asarray(inputs["q"][:, heads], dtype=np.float64)
    k = np.asarray(inputs["k"][:, [kvh]], dtype=np.float64)
    v = np.asarray(inputs["v"][:, [kvh]], dtype=np.float64)
    do = np.asarray(inputs["dout"][:, heads], dtype=np.float64)
    dq, dk, dv = cp_oracle.rank_attention_backward(q, k, v, do, n_img, cu, P, r, split=split,
                                                   local_rows=rows)
    return dq[rows], dk[:, 0], dv[:, 0]


def rank_attention_backward_pooled(q, k, v, dout, n_img, cu_seqlens, cp_size: int, cp_rank: int,
                                   split: str = "head_tail", workers: Optional[int] = None,
                                   row_chunk: int = 256, timeout_s: float = 900.0):
    """``cp_oracle.rank_attention_backward`` over (KV head, row chunk) tasks
    in threads of this process (see ``rank_attention_pooled``). Each task
    calls it unchanged on one KV head's query heads and a chunk of the
    rank's rows; the parent places the chunks' dq rows and adds up their
    dk, dv (the row terms are independent; see its docstring). Returns
    dq [R, H, D], dk and dv [T, Hkv, D]."""
    from concurrent.futures import ThreadPoolExecutor

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    q, k, v, dout = (_as_array(x) for x in (q, k, v, dout))
    T, H, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    n_img = None if n_img is None else np.asarray(n_img)
    cu = None if cu_seqlens is None else np.asarray(cu_seqlens)
    index, _ = cp_oracle.partition_index(T, n_img, cu, cp_size, cp_rank, split)
    R = len(index)
    jobs = [(list(range(g * G, (g + 1) * G)), g, n_img, cu, int(cp_size), int(cp_rank),
             np.arange(r0, min(R, r0 + row_chunk)), split)
            for g in range(Hkv) for r0 in range(0, R, row_chunk)]
    dq = np.zeros((R, H, D))
    dk = np.zeros((T, Hkv, D))
    dv = np.zeros((T, Hkv, D))
    inputs = {"q": q, "k": k, "v": v, "dout": dout}
    limit = threadpool_limits(1) if threadpool_limits else None
    try:
        with ThreadPoolExecutor(min(workers or default_workers(), max(len(jobs), 1))) as ex:
            futs = [ex.submit(_backward_task, inputs, job) for job in jobs]
            for job, f in zip(jobs, futs):
                heads, g, rows = job[0], job[1], job[6]
                gq, gk, gv = f.result(timeout=timeout_s)
                dq[rows[0]:rows[-1] + 1, heads[0]:heads[-1] + 1] = gq
                dk[:, g] += gk
                dv[:, g] += gv
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return dq, dk, dv
