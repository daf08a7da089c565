"""Seeded synthetic workloads shared by the oracle side and the HIP side.

This module only describes workload shapes and draws random inputs. It holds
none of the attention method's arithmetic: no mask, no layout map, no tile
logic, no softmax. Both the CPU oracle (``oracle/``) and the GPU harness
(tests, ``bench.py``) take their inputs from here, so the two sides consume the
very same bf16 values.

Workloads follow the kernel benchmark described on the pages: synthetic bf16
inputs of 75,600 tokens x 10 heads x head dim 128 ("Accelerating
Spatio-Temporal Attention for Video Diffusion on TPUs", Newsbite summary and
TL;DR), a latent video of 21 frames of 45x80 tokens, split into spatial and
temporal heads ("Google Speeds Up Video Diffusion on TPUs with Optimized Sparse
Attention", section "Sparse Attention Patterns"). No dataset is involved.

Draw recipe (fixed here because the pages give none):
  * one independent stream per tensor and head:
    ``numpy.random.default_rng([seed, tensor, head])`` with tensor 0, 1, 2
    for Q, K, V, drawing ``standard_normal((N, d), float32)`` in the original
    frame-major token order t = f*S + s (the streams are filled in parallel
    threads, which keeps the 302,400-token workload quick to generate);
  * each value rounded to bf16 with round-to-nearest-even;
  * an optional query subset comes from its own stream,
    ``default_rng([seed, 3])``: distinct tokens, sorted.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "SWEEP_TILES",
    "workload",
    "draw_qkv",
    "draw_query_subset",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


@dataclass(frozen=True)
class Workload:
    """Shape and mask parameters of one synthetic workload (plain numbers)."""

    name: str
    frames: int            # F, latent frames
    grid_h: int            # Hh, latent rows per frame
    grid_w: int            # Ww, latent columns per frame
    head_kinds: Tuple[str, ...]  # "spatial" | "temporal" | "dense", one per head
    head_dim: int          # d
    frame_window: int      # W_f, spatial heads keep |f - f'| <= W_f
    band: int              # W_s, temporal heads keep |s - s'| <= W_s
    sink: bool             # keep every key of latent frame 0
    tile_q: int            # BQ
    tile_k: int            # BK
    tile_aligned: bool     # round mask edges outward to whole tiles
    seed: int
    query_subset: Optional[int] = None  # compare only this many query tokens

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def seq_len(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def num_heads(self) -> int:
        return len(self.head_kinds)

    def with_tiles(self, tile_q: int, tile_k: int) -> "Workload":
        return replace(self, tile_q=tile_q, tile_k=tile_k,
                       name=f"{self.name}-{tile_q}x{tile_k}")


_SP5_TP5 = ("spatial",) * 5 + ("temporal",) * 5

WORKLOADS: Dict[str, Workload] = {
    # 4 frames of 8x8 latents, one spatial and one temporal head, d=64.
    "tiny": Workload("tiny", 4, 8, 8, ("spatial", "temporal"), 64, 1, 8, True,
                     32, 32, False, seed=1),
    # 6x8 frames: frame edges (48 tokens) do not fall on 32-token tile edges,
    # so the spatial head also gets boundary tiles.
    "tiny-misaligned": Workload("tiny-misaligned", 4, 6, 8,
                                ("spatial", "temporal"), 64, 1, 8, True,
                                32, 32, False, seed=11),
    # The pages' kernel benchmark shape: 21 x 45 x 80 = 75,600 tokens.
    "main": Workload("main", 21, 45, 80, _SP5_TP5, 128, 4, 700, True,
                     256, 128, False, seed=2),
    # All-true mask through the same kernel: the on-chip dense baseline.
    "dense": Workload("dense", 21, 45, 80, ("dense",) * 10, 128, 4, 700, True,
                      256, 128, False, seed=3),
    # Main shape with mask edges rounded outward to whole tiles.
    "tile-aligned": Workload("tile-aligned", 21, 45, 80, _SP5_TP5, 128, 4, 700,
                             True, 256, 128, True, seed=4),
    # 4x the tokens: 21 x 90 x 160 = 302,400.
    "1440p": Workload("1440p", 21, 90, 160, _SP5_TP5, 128, 4, 2800, True,
                      256, 128, False, seed=5, query_subset=2048),
}

# Tile sizes swept for the tile-aligned workload.
SWEEP_TILES: List[Tuple[int, int]] = [(bq, bk) for bq in (128, 256, 512)
                                      for bk in (64, 128, 256)]


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. Inputs are finite normal draws, so
    no NaN handling is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_head(seed: int, tensor: int, head: int, n: int, d: int) -> np.ndarray:
    x = np.empty((n, d), dtype=np.float32)
    np.random.default_rng([seed, tensor, head]).standard_normal(out=x, dtype=np.float32)
    return f32_to_bf16_bits(x)


def draw_qkv(w: Workload, seed: Optional[int] = None):
    """Draw Q, K, V as bf16 bit patterns, shape (H, N, d), original order."""
    seed = w.seed if seed is None else seed
    H, N, d = w.num_heads, w.seq_len, w.head_dim
    out = [np.empty((H, N, d), dtype=np.uint16) for _ in range(3)]

    def fill(job):
        t, h = job
        out[t][h] = _draw_head(seed, t, h, N, d)

    jobs = [(t, h) for t in range(3) for h in range(H)]
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(jobs)))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, jobs))
    return out[0], out[1], out[2]


def draw_query_subset(w: Workload, count: int, seed: Optional[int] = None) -> np.ndarray:
    """Sorted distinct original-order query tokens from their own stream."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng([seed, 3])
    idx = rng.choice(w.seq_len, size=min(count, w.seq_len), replace=False)
    return np.sort(idx).astype(np.int64)
