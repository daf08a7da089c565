"""Run the oracle over many query rows in worker processes (test harness).

The oracle itself is unchanged; rows are split over forked workers that
inherit the input arrays.
"""
from __future__ import annotations

import os
from multiprocessing import get_context

import numpy as np

import oracle
import seeded_inputs as si

_STATE = {}


def _widen(bits):
    return si.bf16_bits_to_f32(bits).astype(np.float64)


def _work(args):
    h, rows = args
    w, Q, K, V, masks = (_STATE[k] for k in ("w", "Q", "K", "V", "masks"))
    q = _widen(Q[h])
    return oracle.attention_rows(q, _widen(K[h]), _widen(V[h]), masks[h], rows)


def oracle_rows(w: si.Workload, Q, K, V, masks, rows: np.ndarray, jobs: int = 0,
                block: int = 256) -> np.ndarray:
    """float64 [H, len(rows), d] for original-order query ``rows``."""
    if jobs <= 0:
        jobs = max(1, min(16, len(os.sched_getaffinity(0))))
    _STATE.update(w=w, Q=Q, K=K, V=V, masks=masks)
    tasks = [(h, rows[i:i + block]) for h in range(w.num_heads)
             for i in range(0, len(rows), block)]
    if jobs == 1 or len(tasks) == 1:
        parts = [_work(t) for t in tasks]
    else:
        with get_context("fork").Pool(min(jobs, len(tasks))) as pool:
            parts = pool.map(_work, tasks)
    out = np.zeros((w.num_heads, len(rows), w.head_dim))
    k = 0
    for h in range(w.num_heads):
        for i in range(0, len(rows), block):
            out[h, i:i + block] = parts[k]
            k += 1
    return out
