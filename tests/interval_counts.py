"""Closed forms and interval arithmetic that pin the oracle.

Nothing here calls the oracle or the HIP path. Pair and tile counts are
derived from the mask definitions by counting integer intervals, a different
route from the oracle's explicit boolean blocks, so a dropped term, a wrong
index or a transposed layout in either shows up as a mismatch.
"""
from __future__ import annotations

import numpy as np


def closed_form_pairs(F: int, S: int, kind: str, W_f: int, W_s: int,
                      sink: bool = True) -> int:
    """Retained (query, key) pairs of one head, in closed form.

    spatial:  S^2 * sum_f |[max(0, f-W_f), min(F-1, f+W_f)] u {0}|
    temporal: F^2 * B + F * (S^2 - B), B = #{(s, s'): |s - s'| <= W_s}
    dense:    (F*S)^2
    """
    if kind == "dense":
        return (F * S) ** 2
    if kind == "spatial":
        total = 0
        for f in range(F):
            lo, hi = max(0, f - W_f), min(F - 1, f + W_f)
            n = hi - lo + 1
            if sink and lo > 0:
                n += 1
            total += n
        return S * S * total
    if kind == "temporal":
        W = min(W_s, S - 1)
        B = S * (2 * W + 1) - W * (W + 1)
        if not sink:
            return F * F * B
        return F * F * B + F * (S * S - B)
    raise ValueError(kind)


def _len(a, b):
    return np.maximum(0, b - a)


def _mult(a, b, F):
    """Multiples of F in [a, b) (elementwise, b >= a or empty)."""
    ca = -((-a) // F)
    cb = -((-b) // F)
    return np.where(b > a, cb - ca, 0)


def _row_counts(F, S, kind, W_f, W_s, sink, rows, c0, c1):
    """counts[i, j]: retained keys of kernel-layout row rows[i] in [c0[j], c1[j])."""
    r = rows[:, None]
    c0 = c0[None, :]
    c1 = c1[None, :]
    if kind == "dense":
        return np.broadcast_to(c1 - c0, (len(rows), c0.shape[1])).astype(np.int64)
    if kind == "spatial":
        f = r // S
        a = np.maximum(0, f - W_f) * S
        b = np.minimum(F, f + W_f + 1) * S
        win = _len(np.maximum(a, c0), np.minimum(b, c1))
        if not sink:
            return win
        zs = _len(np.maximum(0, c0), np.minimum(S, c1))
        both = _len(np.maximum(np.maximum(a, 0), c0), np.minimum(np.minimum(b, S), c1))
        return win + zs - both
    if kind == "temporal":
        s = r // F
        a = np.maximum(0, s - W_s) * F
        b = np.minimum(S, s + W_s + 1) * F
        lo, hi = np.maximum(a, c0), np.minimum(b, c1)
        band = _len(lo, hi)
        if not sink:
            return band
        return band + _mult(c0, c1, F) - _mult(lo, np.maximum(lo, hi), F)
    raise ValueError(kind)


def _band_row_counts(F, S, W_s, rows, c0, c1):
    r = rows[:, None]
    s = r // F
    a = np.maximum(0, s - W_s) * F
    b = np.minimum(S, s + W_s + 1) * F
    return _len(np.maximum(a, c0[None, :]), np.minimum(b, c1[None, :]))


def interval_tile_counts(F, S, kind, W_f, W_s, sink, BQ, BK,
                         tile_aligned=False, row_chunk=8192) -> np.ndarray:
    """Retained pairs per (Q tile, KV tile), int64 [nQ, nK]."""
    N = F * S
    c0 = np.arange(0, N, BK, dtype=np.int64)
    c1 = np.minimum(N, c0 + BK)
    nq = -(-N // BQ)
    out = np.zeros((nq, len(c0)), dtype=np.int64)
    band_tiles = np.zeros((nq, len(c0)), dtype=np.int64)
    step = max(BQ, (row_chunk // BQ) * BQ)
    for r0 in range(0, N, step):
        rows = np.arange(r0, min(N, r0 + step), dtype=np.int64)
        qt = rows // BQ
        cnt = _row_counts(F, S, kind, W_f, W_s, sink, rows, c0, c1)
        np.add.at(out, qt, cnt)
        if kind == "temporal" and tile_aligned:
            np.add.at(band_tiles, qt, _band_row_counts(F, S, W_s, rows, c0, c1))
    if not tile_aligned or kind == "dense":
        return out
    rows_per = np.minimum(N, np.arange(nq) * BQ + BQ) - np.arange(nq) * BQ
    area = rows_per[:, None] * (c1 - c0)[None, :]
    if kind == "spatial":
        return np.where(out > 0, area, 0)
    sinkcols = _mult(c0, c1, F) if sink else np.zeros_like(c0)
    return np.where(band_tiles > 0, area, rows_per[:, None] * sinkcols[None, :])


def interval_classes(counts: np.ndarray, N: int, BQ: int, BK: int) -> np.ndarray:
    nq, nk = counts.shape
    rows = np.minimum(N, np.arange(nq) * BQ + BQ) - np.arange(nq) * BQ
    cols = np.minimum(N, np.arange(nk) * BK + BK) - np.arange(nk) * BK
    area = rows[:, None] * cols[None, :]
    cls = np.full(counts.shape, 2, dtype=np.uint8)
    cls[counts == 0] = 0
    cls[counts == area] = 1
    return cls


def temporal_hull(F, S, W_s, BQ, BK, sink=True):
    """Closed-form band hull [t_lo, t_hi] and sink split (a, b) per Q tile.

    Rows of Q tile qt span raster indices s0 = first_row // F to
    s1 = last_row // F; band keys span raster indices [s0 - W_s, s1 + W_s]
    clipped to [0, S-1], i.e. kernel positions
    [max(0, s0-W_s)*F, (min(S-1, s1+W_s)+1)*F - 1].
    """
    N = F * S
    nq = -(-N // BQ)
    first = np.arange(nq) * BQ
    last = np.minimum(N, first + BQ) - 1
    s0, s1 = first // F, last // F
    t_lo = (np.maximum(0, s0 - W_s) * F) // BK
    t_hi = ((np.minimum(S - 1, s1 + W_s) + 1) * F - 1) // BK
    if not sink:
        return t_lo, t_hi, np.zeros(nq, np.int64), np.full(nq, S, np.int64)
    a = -((-(t_lo * BK)) // F)
    b = -((-np.minimum(N, (t_hi + 1) * BK)) // F)
    return t_lo, t_hi, a, b
