"""Glue between seeded workloads and the oracle (test-side only)."""
from __future__ import annotations

from functools import lru_cache

import numpy as np

import oracle
import seeded_inputs as si


def params_of(w: si.Workload) -> oracle.MaskParams:
    return oracle.MaskParams(w.frames, w.grid_h, w.grid_w, w.frame_window,
                             w.band, w.sink)


def masks_of(w: si.Workload):
    p = params_of(w)
    return [oracle.HeadMask(p, k, w.tile_aligned, w.tile_q, w.tile_k)
            for k in w.head_kinds]


@lru_cache(maxsize=64)
def oracle_kind_map(w: si.Workload, kind: str):
    """Oracle class map, schedule and stats of one head kind (cached)."""
    p = params_of(w)
    m = oracle.HeadMask(p, kind, w.tile_aligned, w.tile_q, w.tile_k)
    counts = oracle.tile_counts(m, w.tile_q, w.tile_k)
    cls = oracle.tile_classes(counts, p.N, w.tile_q, w.tile_k)
    sched = oracle.head_schedule(m, cls, w.tile_q, w.tile_k)
    stats = oracle.head_stats(m, counts, cls, sched, w.tile_q, w.tile_k)
    return counts, cls, sched, stats


def widen(bits: np.ndarray) -> np.ndarray:
    return si.bf16_bits_to_f32(bits).astype(np.float64)
