"""CPU oracle for structured-sparse (Sparse VideoGen) video attention.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
float64 statement of what the forward pass computes. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It shares no code with the HIP path (no kernels, headers, tables or
helpers) and imports nothing from it; the two meet only through the seeded
inputs of ``seeded_inputs``.

What the pages fix, and where:
  * Attention heads of video diffusion transformers specialise into spatial
    heads (same or nearby frames) and temporal heads (a narrow spatial region
    across many frames); each head is routed to a spatial or a temporal mask
    ("Google Speeds Up Video Diffusion on TPUs with Optimized Sparse
    Attention", section "Sparse Attention Patterns").
  * The two head kinds need different token orders and mask patterns, and
    both masks keep full attention to the first frame as an attention sink
    ("Accelerating Spatio-Temporal Attention for Video Diffusion on TPUs",
    Newsbite, section "Interesting facts").
  * Visited tiles are either "full" (every pair retained) or "boundary"
    (retained and dropped pairs mixed); full tiles take a mask-free path
    (marsel.app page, section "Efficient Kernel Implementation", tile-aware
    masking; Newsbite "Summary").
  * Each head is routed to the spatial or the temporal mask from a sample of
    its attention (same sections; routing.py gives the reading taken).
  * A tile-aligned variant rounds mask edges to the physical tiles so that few
    tiles need masking (StreamingMeme lead paragraph; Newsbite "Summary",
    "What changed").

Readings taken where the pages are silent are listed in each module.

Parity status: every function here is pinned by tests under ``tests/``
(closed-form pair counts, interval-arithmetic tile counts, brute force on tiny
inputs, agreement with dense SDPA for all-true masks and per-frame SDPA for a
frame-diagonal mask, softmax row sums, permutation invariance).
"""
from .masks import (DENSE, SPATIAL, TEMPORAL, MaskParams, HeadMask,
                    kernel_coords, original_coords, kernel_position,
                    to_kernel_layout, to_original_layout)
from .tilemap import (SKIP, FULL, BOUNDARY, TileSchedule, tile_counts,
                      tile_classes, head_schedule, head_stats)
from .attention import attention_rows, attention
from .routing import Route, route_head, route_heads

__all__ = [
    "DENSE", "SPATIAL", "TEMPORAL", "MaskParams", "HeadMask",
    "kernel_coords", "original_coords", "kernel_position",
    "to_kernel_layout", "to_original_layout",
    "SKIP", "FULL", "BOUNDARY", "TileSchedule", "tile_counts",
    "tile_classes", "head_schedule", "head_stats",
    "attention_rows", "attention", "Route", "route_head", "route_heads",
]
