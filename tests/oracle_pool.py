"""Run the oracle over many query rows in worker processes (test harness).

The oracle itself is unchanged; rows are split over forked workers that
inherit the input arrays.
"""
from __future__ import annotations

import os
import sys
from multiprocessing import get_context

import numpy as np

import oracle
import seeded_inputs as si

_STATE = {}


def _one_blas_thread():
    """Worker initializer: one BLAS / OpenMP thread per worker process (the
    pool already runs one process per core)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _widen(bits):
    return si.bf16_bits_to_f32(bits).astype(np.float64)


_WIDE = {}


def _head_qkv(h):
    """Head h's Q, K and V widened to float64, kept for the worker's next
    task (tasks come in head order, so a worker mostly stays on one head)."""
    if _WIDE.get("h") != h:
        _WIDE.clear()
        _WIDE.update(h=h, Q=_widen(_STATE["Q"][h]), K=_widen(_STATE["K"][h]),
                     V=_widen(_STATE["V"][h]))
    return _WIDE["Q"], _WIDE["K"], _WIDE["V"]


def _work(args):
    h, rows = args
    Q, K, V = _head_qkv(h)
    return oracle.attention_rows(Q, K, V, _STATE["masks"][h], rows)


def oracle_rows(w: si.Workload, Q, K, V, masks, rows: np.ndarray, jobs: int = 0,
                block: int = 256) -> np.ndarray:
    """float64 [H, len(rows), d] for original-order query ``rows``."""
    if jobs <= 0:
        jobs = max(1, min(16, len(os.sched_getaffinity(0))))
    _STATE.update(w=w, Q=Q, K=K, V=V, masks=masks)
    _WIDE.clear()
    tasks = [(h, rows[i:i + block]) for h in range(w.num_heads)
             for i in range(0, len(rows), block)]
    if jobs == 1 or len(tasks) == 1:
        parts = [_work(t) for t in tasks]
    else:
        with get_context("fork").Pool(min(jobs, len(tasks)), _one_blas_thread) as pool:
            parts = pool.map(_work, tasks)
    out = np.zeros((w.num_heads, len(rows), w.head_dim))
    k = 0
    for h in range(w.num_heads):
        for i in range(0, len(rows), block):
            out[h, i:i + block] = parts[k]
            k += 1
    return out


def _compare_work(args):
    h, rows = args
    Q, K, V = _head_qkv(h)
    ref = oracle.attention_rows(Q, K, V, _STATE["masks"][h], rows)
    O = _STATE["O"]
    got = O[h, rows].astype(np.float64)
    d = got - ref
    return (float(np.abs(d).max()), float(np.abs(d).sum()), float((d * d).sum()),
            float((ref * ref).sum()), d.size, bool(np.isfinite(got).all()))


def compare_all_rows(w: si.Workload, Q, K, V, masks, O: np.ndarray, jobs: int = 0,
                     block: int = 128) -> dict:
    """The oracle over every query row of every head, compared in the workers
    with ``O`` (float32 [H, N, d], original order): max and mean absolute
    error, relative L2 error, and whether every output is finite. Only these
    statistics leave the workers, so the full float64 output never has to be
    held at once."""
    if jobs <= 0:
        jobs = max(1, min(16, len(os.sched_getaffinity(0))))
    _STATE.update(w=w, Q=Q, K=K, V=V, masks=masks, O=O)
    _WIDE.clear()
    rows = np.arange(w.seq_len)
    tasks = [(h, rows[i:i + block]) for h in range(w.num_heads)
             for i in range(0, len(rows), block)]
    parts = []
    try:
        with get_context("fork").Pool(min(jobs, len(tasks)), _one_blas_thread) as pool:
            # progress to stderr about every tenth of the work, so that a
            # long comparison shows it is alive
            step = max(1, len(tasks) // 10)
            for i, r in enumerate(pool.imap(_compare_work, tasks, chunksize=4)):
                parts.append(r)
                if (i + 1) % step == 0:
                    print(f"    oracle rows: {i + 1}/{len(tasks)} blocks", file=sys.stderr,
                          flush=True)
    finally:
        _STATE.pop("O", None)
    n = sum(p[4] for p in parts)
    return {"max_abs": max(p[0] for p in parts), "mean_abs": sum(p[1] for p in parts) / n,
            "rel_l2": float(np.sqrt(sum(p[2] for p in parts) / max(sum(p[3] for p in parts),
                                                                    1e-300))),
            "finite": all(p[5] for p in parts), "elements": n}
