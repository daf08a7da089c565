"""Token layouts and head masks, written out as explicit boolean blocks.

TEST INFRASTRUCTURE (see the package header): float64/bool numpy only.

Notation. A latent video has F frames of Hh x Ww tokens; S = Hh*Ww tokens per
frame and N = F*S tokens in all. A token is (f, s): frame f, raster index
s = y*Ww + x. Its original, frame-major position is t = f*S + s.

Head kinds ("Google Speeds Up Video Diffusion on TPUs with Optimized Sparse
Attention", "Sparse Attention Patterns"; Newsbite "Interesting facts"):
  * spatial:  keep (q, k) when |f_q - f_k| <= W_f, or when f_k = 0 (sink);
  * temporal: keep (q, k) when |s_q - s_k| <= W_s, or when f_k = 0 (sink);
  * dense:    keep every pair (the dense baseline of Newsbite "Summary").

Readings taken (the pages give no formulas):
  * The window and the band are symmetric and non-causal; nothing on the pages
    mentions causality.
  * The temporal band is measured on the raster index s, not on the position
    in the re-ordered sequence.
  * The sink is on the key side only: every query sees all S keys of frame 0.
  * Kernel layout ("different token-ordering" per head kind, Newsbite
    "Interesting facts"): spatial and dense heads keep the original order
    p = t; temporal heads are re-ordered spatial-major, p = s*F + f, so a
    narrow spatial band becomes a contiguous run of positions.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

SPATIAL = "spatial"
TEMPORAL = "temporal"
DENSE = "dense"
KINDS = (SPATIAL, TEMPORAL, DENSE)


@dataclass(frozen=True)
class MaskParams:
    frames: int          # F
    grid_h: int          # Hh
    grid_w: int          # Ww
    frame_window: int    # W_f
    band: int            # W_s
    sink: bool           # keep all keys of frame 0

    @property
    def S(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def N(self) -> int:
        return self.frames * self.S


def original_coords(p: MaskParams, t: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(frame, raster index) of original-order positions t = f*S + s."""
    t = np.asarray(t, dtype=np.int64)
    return (t // p.S).astype(np.int32), (t % p.S).astype(np.int32)


def kernel_coords(p: MaskParams, kind: str, pos: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(frame, raster index) of positions in the head's kernel layout."""
    pos = np.asarray(pos, dtype=np.int64)
    if kind == TEMPORAL:
        f, s = pos % p.frames, pos // p.frames          # p = s*F + f
    else:
        f, s = pos // p.S, pos % p.S                    # p = f*S + s
    return f.astype(np.int32), s.astype(np.int32)


def kernel_position(p: MaskParams, kind: str, t: np.ndarray) -> np.ndarray:
    """Kernel-layout position of original-order token t."""
    f, s = original_coords(p, t)
    f, s = f.astype(np.int64), s.astype(np.int64)
    if kind == TEMPORAL:
        return s * p.frames + f
    return f * p.S + s


def to_kernel_layout(p: MaskParams, kind: str, x: np.ndarray) -> np.ndarray:
    """Re-order rows (axis 0, original order) into the head's kernel layout."""
    out = np.empty_like(x)
    out[kernel_position(p, kind, np.arange(p.N))] = x
    return out


def to_original_layout(p: MaskParams, kind: str, y: np.ndarray) -> np.ndarray:
    """Inverse of ``to_kernel_layout``."""
    return y[kernel_position(p, kind, np.arange(p.N))]


def keep_pairs(p: MaskParams, kind: str, fq, sq, fk, sk) -> np.ndarray:
    """The head mask on broadcastable (frame, raster) coordinates."""
    fq, sq, fk, sk = (np.asarray(a, dtype=np.int32) for a in (fq, sq, fk, sk))
    shape = np.broadcast_shapes(fq.shape, sq.shape, fk.shape, sk.shape)
    if kind == DENSE:
        return np.ones(shape, dtype=bool)
    if kind == SPATIAL:
        m = np.abs(fq - fk) <= p.frame_window
    elif kind == TEMPORAL:
        m = np.abs(sq - sk) <= p.band
    else:
        raise ValueError(f"unknown head kind {kind!r}")
    if p.sink:
        m = m | (fk == 0)
    return np.broadcast_to(m, shape)


def keep_contiguous_part(p: MaskParams, kind: str, fq, sq, fk, sk) -> np.ndarray:
    """The part of the mask that is a contiguous run of kernel positions.

    Spatial heads: the whole mask (window and sink are both runs of whole
    frames in natural order). Temporal heads: the band only; the frame-0 sink
    sits at every F-th position in the re-ordered layout. Dense: everything.
    """
    if kind == TEMPORAL:
        sq, sk = np.asarray(sq, dtype=np.int32), np.asarray(sk, dtype=np.int32)
        return np.abs(sq - sk) <= p.band
    return keep_pairs(p, kind, fq, sq, fk, sk)


def strided_sink(p: MaskParams, kind: str, fk) -> np.ndarray:
    """Temporal heads' frame-0 keys (the non-contiguous part), else nothing."""
    fk = np.asarray(fk, dtype=np.int32)
    if kind == TEMPORAL and p.sink:
        return fk == 0
    return np.zeros(fk.shape, dtype=bool)


class HeadMask:
    """Explicit mask of one head, exact or tile-aligned.

    ``kernel_block(rows, cols)`` takes kernel-layout positions,
    ``original_block(rows, cols)`` takes original-order positions; both return
    a bool array of shape (len(rows), len(cols)).

    Tile-aligned reading (the pages give neither the rounding rule nor the
    tile sizes; StreamingMeme lead, Newsbite "Summary"): the contiguous part
    of the mask is dilated outward to whole (BQ x BK) tiles of the kernel
    layout -- a pair is kept when its tile holds any pair of the contiguous
    part -- and the temporal frame-0 sink is kept exactly (rounding it would
    make every tile of a temporal head full). The result is a superset of the
    exact mask.
    """

    def __init__(self, p: MaskParams, kind: str, tile_aligned: bool = False,
                 tile_q: Optional[int] = None, tile_k: Optional[int] = None):
        if kind not in KINDS:
            raise ValueError(f"unknown head kind {kind!r}")
        if tile_aligned and (not tile_q or not tile_k):
            raise ValueError("tile-aligned mask needs tile sizes")
        self.p, self.kind, self.tile_aligned = p, kind, tile_aligned
        self.tile_q, self.tile_k = tile_q, tile_k
        self._any_rows = {}

    def _contiguous_tile_any(self, qt: int) -> np.ndarray:
        """any[kt] for Q tile qt: tile (qt, kt) holds a contiguous-part pair."""
        if qt not in self._any_rows:
            p, BQ, BK = self.p, self.tile_q, self.tile_k
            cols = np.arange(p.N)
            fk, sk = kernel_coords(p, self.kind, cols)
            fq, sq = kernel_coords(p, self.kind,
                                   np.arange(qt * BQ, min(p.N, (qt + 1) * BQ)))
            blk = keep_contiguous_part(p, self.kind, fq[:, None], sq[:, None],
                                       fk[None, :], sk[None, :])
            starts = np.arange(0, p.N, BK)
            self._any_rows[qt] = np.add.reduceat(
                blk.any(axis=0).astype(np.int64), starts) > 0
        return self._any_rows[qt]

    def kernel_block(self, rows, cols) -> np.ndarray:
        p = self.p
        rows = np.asarray(rows, dtype=np.int64)
        cols = np.asarray(cols, dtype=np.int64)
        fq, sq = kernel_coords(p, self.kind, rows)
        fk, sk = kernel_coords(p, self.kind, cols)
        if not self.tile_aligned:
            return np.array(keep_pairs(p, self.kind, fq[:, None], sq[:, None],
                                       fk[None, :], sk[None, :]))
        qts = rows // self.tile_q
        table = {int(q): self._contiguous_tile_any(int(q)) for q in np.unique(qts)}
        dil = np.stack([table[int(q)] for q in qts])[:, cols // self.tile_k]
        return dil | strided_sink(p, self.kind, fk)[None, :]

    def original_block(self, rows, cols) -> np.ndarray:
        return self.kernel_block(kernel_position(self.p, self.kind, rows),
                                 kernel_position(self.p, self.kind, cols))
