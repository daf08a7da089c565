"""Tile class map and execution schedule, by explicit counting.

TEST INFRASTRUCTURE (see the package header).

The class of a tile follows the tile-aware masking of the pages ("Google Speeds
Up Video Diffusion on TPUs with Optimized Sparse Attention", "Efficient Kernel
Implementation"; Newsbite "Summary"): a tile whose pairs are all retained is
FULL and runs mask-free, a tile that mixes retained and dropped pairs is
BOUNDARY and is masked element by element, and a tile with no retained pair is
SKIP. Counting runs over the tile's existing elements only: the last row and
column tiles are ragged when N is not a multiple of BQ or BK.

Schedule (which KV tiles a Q tile executes), reading taken:
  * spatial and dense heads execute every non-SKIP tile;
  * temporal heads: the frame-0 sink sits at every F-th column of the
    re-ordered layout, so every KV tile holds retained pairs. Executing the
    literal map would visit every tile, which the pages rule out (the naive
    kernel already skipped more than half the tiles, Newsbite "Interesting
    facts"). The exact decomposition used instead: the Q tile executes the
    hull of KV tiles that hold any band pair, each with its literal class,
    and the frame-0 keys outside that hull -- raster indices [0, a) and
    [b, S) -- as mask-free sink keys. Outside the hull no band pair exists, so
    every retained pair is covered exactly once.
  * order: FULL tiles ascending, then BOUNDARY tiles ascending, then the sink
    keys.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

from .masks import (DENSE, SPATIAL, TEMPORAL, HeadMask, MaskParams,
                    kernel_coords, keep_contiguous_part)

SKIP, FULL, BOUNDARY = 0, 1, 2


def _tiles(n: int, b: int):
    return [(i, min(n, i + b)) for i in range(0, n, b)]


def _q_tiles(N: int, tile_q: int, qtiles: Optional[Sequence[int]]):
    qts = _tiles(N, tile_q)
    ids = range(len(qts)) if qtiles is None else list(qtiles)
    return [(i, qts[i]) for i in ids]


def tile_counts(mask: HeadMask, tile_q: int, tile_k: int,
                qtiles: Optional[Sequence[int]] = None) -> np.ndarray:
    """Retained pairs in every (Q tile, KV tile), int64 [nQ, nK].

    With ``qtiles``, only those Q tiles (rows of the result, in that order).
    """
    N = mask.p.N
    col_starts = np.arange(0, N, tile_k)
    cols = np.arange(N)
    sel = _q_tiles(N, tile_q, qtiles)
    out = np.zeros((len(sel), len(col_starts)), dtype=np.int64)
    for i, (_, (r0, r1)) in enumerate(sel):
        blk = mask.kernel_block(np.arange(r0, r1), cols)
        out[i] = np.add.reduceat(np.count_nonzero(blk, axis=0).astype(np.int64),
                                 col_starts)
    return out


def tile_classes(counts: np.ndarray, N: int, tile_q: int, tile_k: int,
                 qtiles: Optional[Sequence[int]] = None) -> np.ndarray:
    """SKIP / FULL / BOUNDARY from retained-pair counts, uint8 [nQ, nK]."""
    rows = np.array([b - a for _, (a, b) in _q_tiles(N, tile_q, qtiles)],
                    dtype=np.int64)
    cols = np.array([b - a for a, b in _tiles(N, tile_k)], dtype=np.int64)
    area = rows[:, None] * cols[None, :]
    cls = np.full(counts.shape, BOUNDARY, dtype=np.uint8)
    cls[counts == 0] = SKIP
    cls[counts == area] = FULL
    return cls


@dataclass
class TileSchedule:
    """Per Q tile: KV tiles to run and the frame-0 sink keys outside them."""

    full: List[np.ndarray]       # ascending KV tile ids, mask-free
    boundary: List[np.ndarray]   # ascending KV tile ids, masked
    sink_a: np.ndarray           # sink raster indices [0, a) ...
    sink_b: np.ndarray           # ... and [b, S), mask-free


def _band_tiles(p: MaskParams, tile_q: int, tile_k: int,
                qtiles: Optional[Sequence[int]] = None) -> np.ndarray:
    """bool [nQ, nK]: the tile holds at least one band pair (temporal head)."""
    N = p.N
    cols = np.arange(N)
    fk, sk = kernel_coords(p, TEMPORAL, cols)
    starts = np.arange(0, N, tile_k)
    out = []
    for _, (r0, r1) in _q_tiles(N, tile_q, qtiles):
        fq, sq = kernel_coords(p, TEMPORAL, np.arange(r0, r1))
        blk = keep_contiguous_part(p, TEMPORAL, fq[:, None], sq[:, None],
                                   fk[None, :], sk[None, :])
        out.append(np.add.reduceat(blk.any(axis=0).astype(np.int64), starts) > 0)
    return np.array(out)


def head_schedule(mask: HeadMask, classes: np.ndarray, tile_q: int,
                  tile_k: int, qtiles: Optional[Sequence[int]] = None) -> TileSchedule:
    """Schedule of every Q tile, or of ``qtiles`` when ``classes`` holds only
    those rows (as returned by ``tile_counts(..., qtiles)``)."""
    p, kind = mask.p, mask.kind
    nq, nk = classes.shape
    full, bnd = [], []
    sink_a = np.zeros(nq, dtype=np.int64)
    sink_b = np.full(nq, p.S, dtype=np.int64)
    band = _band_tiles(p, tile_q, tile_k, qtiles) if kind == TEMPORAL else None
    for qt in range(nq):
        run = np.ones(nk, dtype=bool)
        if kind == TEMPORAL:
            hit = np.flatnonzero(band[qt])
            lo, hi = hit[0], hit[-1]           # every Q tile has a band pair
            run[:] = False
            run[lo:hi + 1] = True
            if p.sink:
                # frame-0 keys are the positions s'*F; split them by the hull
                sink_cols = np.arange(p.S) * p.frames
                below = sink_cols < lo * tile_k
                above = sink_cols >= min(p.N, (hi + 1) * tile_k)
                sink_a[qt] = int(below.sum())
                sink_b[qt] = p.S - int(above.sum())
                assert np.all(below[:sink_a[qt]]) and np.all(above[sink_b[qt]:])
        ids = np.arange(nk)
        full.append(ids[run & (classes[qt] == FULL)])
        bnd.append(ids[run & (classes[qt] == BOUNDARY)])
    return TileSchedule(full, bnd, sink_a, sink_b)


def head_stats(mask: HeadMask, counts: np.ndarray, classes: np.ndarray,
               sched: TileSchedule, tile_q: int, tile_k: int) -> Dict[str, int]:
    """Logical class counts, executed work and retained pairs of one head.

    ``exec_sink`` counts the sink keys of each Q tile in groups of BK
    (ceil(a/BK) + ceil((S-b)/BK)). ``covered_pairs`` is the retained pairs that
    the schedule executes; it must equal ``retained_pairs``.
    """
    p = mask.p
    rows = np.array([b - a for a, b in _tiles(p.N, tile_q)], dtype=np.int64)
    n_sink = sched.sink_a + (p.S - sched.sink_b)
    covered = 0
    for qt in range(classes.shape[0]):
        covered += int(counts[qt, sched.full[qt]].sum())
        covered += int(counts[qt, sched.boundary[qt]].sum())
        covered += int(rows[qt] * n_sink[qt])
    return {
        "tiles": int(classes.size),
        "skip": int((classes == SKIP).sum()),
        "full": int((classes == FULL).sum()),
        "boundary": int((classes == BOUNDARY).sum()),
        "exec_full": int(sum(len(x) for x in sched.full)),
        "exec_boundary": int(sum(len(x) for x in sched.boundary)),
        "exec_sink": int((-(-sched.sink_a // tile_k)).sum()
                         + (-(-(p.S - sched.sink_b) // tile_k)).sum()),
        "retained_pairs": int(counts.sum()),
        "covered_pairs": covered,
    }
