"""Explicit-mask scaled-dot-product attention in float64.

TEST INFRASTRUCTURE (see the package header).

For every head and every query row, in the original token order:
    S = scale * q K^T,  S[~M] = -inf,  P = softmax(S),  o = P V,
with scale = 1/sqrt(d). A row with no retained key gives o = 0 (cannot happen
with the masks here: every query keeps its own frame / raster index).

This is the plain definition of what the pages' kernels compute: the
full/boundary split changes how the work is traversed, not the result (the
exact variant keeps the intended query-key budget, Newsbite "What changed").
The attention itself is the self-attention of the video diffusion model
("Google Speeds Up Video Diffusion on TPUs with Optimized Sparse Attention",
"The Challenge: Attention at Scale"). Inputs are the bf16 values the GPU reads,
widened to float64, so both sides consume identical numbers.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .masks import HeadMask


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                   mask: HeadMask, rows: np.ndarray,
                   scale: Optional[float] = None, block: int = 256) -> np.ndarray:
    """o for the given original-order query rows of one head.

    q, k, v: float64 [N, d] in original order. Returns float64 [len(rows), d].
    """
    N, d = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(N)
    out = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    for i in range(0, len(rows), block):
        r = rows[i:i + block]
        s = scale * (q[r] @ k.T)
        keep = mask.original_block(r, cols)
        s = np.where(keep, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        has = np.isfinite(m[:, 0])
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - m)
        e = np.where(keep, e, 0.0)
        den = e.sum(axis=1, keepdims=True)
        o = (e @ v) / np.where(den > 0, den, 1.0)
        out[i:i + block] = np.where(has[:, None], o, 0.0)
    return out


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
              masks: Sequence[HeadMask], rows: Optional[np.ndarray] = None,
              scale: Optional[float] = None) -> np.ndarray:
    """o for every head: Q, K, V float64 [H, N, d] in original order."""
    H, N, _ = Q.shape
    if rows is None:
        rows = np.arange(N)
    return np.stack([attention_rows(Q[h], K[h], V[h], masks[h], rows, scale)
                     for h in range(H)])
