"""Online head routing by sampling, in float64.

TEST INFRASTRUCTURE (see the package header).

What the pages fix: a head of a video diffusion transformer is routed to the
spatial or to the temporal mask, and the routing is decided from a sample
("Google Speeds Up Video Diffusion on TPUs with Optimized Sparse Attention",
section "Sparse Attention Patterns"); Sparse VideoGen profiles the heads while
the model runs and routes each to one of the two masks ("Accelerating
Spatio-Temporal Attention for Video Diffusion on TPUs", Newsbite, summary).

Reading taken (the pages give no procedure, no sample size and no error
measure): the caller draws the sample, a set of query rows in the original
token order. For one head, attention on those rows is computed three times,
with every key, under the spatial mask and under the temporal mask, each
exactly as ``attention_rows`` defines it. The error of a mask is the mean
squared difference between its output and the dense output, over the sampled
rows and all d output columns. The head goes to the mask with the smaller
error; a tie goes to the spatial mask. Parity: pinned by
``tests/test_oracle_routing.py`` (brute force with the masks written out
again from their definitions, a closed form for Q = 0 with V the frame-0
indicator, masks that keep every pair, planted spatial and temporal heads).
"""
from __future__ import annotations

from typing import List, NamedTuple, Optional

import numpy as np

from .attention import attention_rows
from .masks import DENSE, SPATIAL, TEMPORAL, HeadMask, MaskParams


class Route(NamedTuple):
    err_spatial: float    # mean squared error of the spatial mask's output
    err_temporal: float   # mean squared error of the temporal mask's output
    kind: str             # SPATIAL or TEMPORAL


def route_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, p: MaskParams,
               rows: np.ndarray, scale: Optional[float] = None) -> Route:
    """q, k, v: float64 [N, d] of one head in original order; rows: sampled
    original-order query indices."""
    dense = attention_rows(q, k, v, HeadMask(p, DENSE), rows, scale)
    spatial = attention_rows(q, k, v, HeadMask(p, SPATIAL), rows, scale)
    temporal = attention_rows(q, k, v, HeadMask(p, TEMPORAL), rows, scale)
    es = float(np.mean((spatial - dense) ** 2))
    et = float(np.mean((temporal - dense) ** 2))
    return Route(es, et, SPATIAL if es <= et else TEMPORAL)


def route_heads(Q: np.ndarray, K: np.ndarray, V: np.ndarray, p: MaskParams,
                rows: np.ndarray, scale: Optional[float] = None) -> List[Route]:
    """route_head for every head of float64 [H, N, d] inputs."""
    return [route_head(Q[h], K[h], V[h], p, rows, scale) for h in range(Q.shape[0])]
