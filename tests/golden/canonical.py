"""Canonical byte form and digests of a tile map (no method arithmetic).

The oracle side (``make_tilemap_golden.py``) and the GPU tests both serialise
a head's class map and schedule this way, so maps too large to store can be
compared through a SHA-256 digest.

  classes:  uint8 [nQ][nK], row-major (0 = SKIP, 1 = FULL, 2 = BOUNDARY)
  schedule: for each Q tile, int32 little-endian
            [n_full, n_boundary, sink_a, sink_b, full ids..., boundary ids...]
"""
from __future__ import annotations

import hashlib
from typing import Sequence

import numpy as np


def class_digest(classes: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(classes, dtype=np.uint8).tobytes()).hexdigest()


def schedule_digest(full: Sequence[np.ndarray], boundary: Sequence[np.ndarray],
                    sink_a: Sequence[int], sink_b: Sequence[int]) -> str:
    h = hashlib.sha256()
    for qt in range(len(full)):
        f = np.asarray(full[qt], dtype="<i4")
        b = np.asarray(boundary[qt], dtype="<i4")
        h.update(np.array([len(f), len(b), sink_a[qt], sink_b[qt]], dtype="<i4").tobytes())
        h.update(f.tobytes())
        h.update(b.tobytes())
    return h.hexdigest()


def golden_key(workload_name: str, tile_q: int, tile_k: int) -> str:
    return f"{workload_name}@{tile_q}x{tile_k}"
