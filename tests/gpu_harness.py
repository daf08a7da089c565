"""GPU-side helpers for the parity tests: move seeded inputs to the device and
run the library's calls. No attention arithmetic happens here."""
from __future__ import annotations

import sys

import numpy as np
import torch

import seeded_inputs as si
import structured_sparse_attention_amd as svg


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> CUDA bfloat16 tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def from_device(t: torch.Tensor) -> np.ndarray:
    """CUDA bfloat16 tensor -> float32 numpy (exact widening)."""
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return si.bf16_bits_to_f32(bits)


def build_map(w: si.Workload, stream=None) -> svg.TileMap:
    return svg.svg_build_tile_map(
        w.frames, w.grid_h, w.grid_w, w.head_kinds, w.frame_window, w.band, w.sink,
        svg.ROUND_TILE if w.tile_aligned else svg.ROUND_EXACT, w.tile_q, w.tile_k, stream)


def to_kernel_layout(w: si.Workload, x: torch.Tensor) -> torch.Tensor:
    y = torch.empty_like(x)
    svg.svg_permute_tokens(x, y, w.frames, w.tokens_per_frame, w.head_kinds,
                           svg.TO_KERNEL_LAYOUT)
    return y


def to_original_layout(w: si.Workload, y: torch.Tensor) -> torch.Tensor:
    x = torch.empty_like(y)
    svg.svg_permute_tokens(y, x, w.frames, w.tokens_per_frame, w.head_kinds,
                           svg.TO_ORIGINAL_LAYOUT)
    return x


def run_attention(w: si.Workload, Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                  flags: int = 0, tile_map: svg.TileMap = None) -> np.ndarray:
    """Original-order bf16 bits in -> original-order float32 O (from bf16)."""
    q, k, v = (to_kernel_layout(w, to_device(x)) for x in (Q, K, V))
    o = torch.empty_like(q)
    m = tile_map if tile_map is not None else build_map(w)
    svg.svg_attn_fwd(q, k, v, o, w.head_kinds, m, flags=flags)
    out = to_original_layout(w, o)
    torch.cuda.synchronize()
    res = from_device(out)
    if tile_map is None:
        m.destroy()
    return res


def gpu_head_schedule(tm: svg.TileMap, h: int):
    """Per-Q-tile (full ids, boundary ids, a, b) of head h from the device map."""
    row_ptr, n_full, sink_ab, entries = tm.schedule()
    nq = tm.info.num_q_tiles
    full, bnd, a, b = [], [], [], []
    for qt in range(nq):
        r = h * nq + qt
        s, e = int(row_ptr[r]), int(row_ptr[r + 1])
        full.append(entries[s:s + int(n_full[r])])
        bnd.append(entries[s + int(n_full[r]):e])
        a.append(int(sink_ab[r, 0]))
        b.append(int(sink_ab[r, 1]))
    return full, bnd, np.array(a), np.array(b)
