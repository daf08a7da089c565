"""Tile-size search (svg_autotune_tiles) on the GPU: every candidate is timed,
the fastest is returned, and the attention the search ran, as well as a run
with the chosen tiles, match the oracle to the attention gate."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import structured_sparse_attention_amd as svg
from gpu_harness import from_device, run_attention, say, to_device, to_kernel_layout, \
    to_original_layout
from oracle_cases import masks_of, widen
from test_gpu_attention import check
from test_oracle_pins import RAGGED

pytestmark = pytest.mark.gpu

CANDIDATES = [(32, 32), (64, 64), (128, 96), (256, 64), (256, 128), (512, 64), (512, 256)]


def test_autotune_picks_the_fastest_and_keeps_parity():
    w = RAGGED
    say(f"[autotune] {w.name} N={w.seq_len} H={w.num_heads} d={w.head_dim}: "
        f"{len(CANDIDATES)} candidates")
    Q, K, V = si.draw_qkv(w)
    q, k, v = (to_kernel_layout(w, to_device(x)) for x in (Q, K, V))
    o = torch.empty_like(q)
    best, ms = svg.svg_autotune_tiles(q, k, v, o, w.frames, w.grid_h, w.grid_w, w.head_kinds,
                                      w.frame_window, w.band, CANDIDATES, sink_first_frame=w.sink,
                                      reps=3)
    say(f"  ms per candidate: {[round(x, 4) for x in ms]}, best {CANDIDATES[best]}")
    assert len(ms) == len(CANDIDATES)
    assert all(np.isfinite(x) and x > 0 for x in ms)
    assert best == int(np.argmin(ms))
    ref = oracle.attention(widen(Q), widen(K), widen(V), masks_of(w))
    # o holds the last candidate's attention
    last = from_device(to_original_layout(w, o))
    check(last, ref, f"search output at {CANDIDATES[-1]}")
    bq, bk = CANDIDATES[best]
    check(run_attention(w.with_tiles(bq, bk), Q, K, V), ref, f"chosen tiles {bq}x{bk}")


def test_autotune_rejects_unsupported_candidates_before_running():
    w = RAGGED
    Q, K, V = si.draw_qkv(w)
    q, k, v = (to_device(x) for x in (Q, K, V))
    o = torch.zeros_like(q)
    with pytest.raises(svg.SvgError) as e:
        svg.svg_autotune_tiles(q, k, v, o, w.frames, w.grid_h, w.grid_w, w.head_kinds,
                               w.frame_window, w.band, [(256, 128), (192, 128)])
    assert e.value.status == svg.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert not bool(o.view(torch.int16).any())  # nothing ran
