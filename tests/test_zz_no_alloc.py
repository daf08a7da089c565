"""svg_route_heads_noalloc (no allocation, the library's static scratch)
against svg_route_heads on the GPU, through the C ABI: two calls in a row,
the second on a smaller input, each compared with the allocating call and
with the routing oracle to the routing tests' bar."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import structured_sparse_attention_amd as svg
from gpu_harness import say, to_device
from oracle_cases import widen
from test_oracle_pins import RAGGED

pytestmark = pytest.mark.gpu

REL, FLOOR = 5e-3, 1e-4


def _route(w, Q, K, V, rows, no_alloc):
    q, k, v = (to_device(x) for x in (Q, K, V))
    return svg.svg_route_heads(q, k, v, w.frames, w.grid_h, w.grid_w, w.frame_window, w.band,
                               rows, sink_first_frame=w.sink, no_alloc=no_alloc)


def _check(w, Q, K, V, rows, what):
    k_ref, e_ref = _route(w, Q, K, V, rows, no_alloc=False)
    k_na, e_na = _route(w, Q, K, V, rows, no_alloc=True)
    p = oracle.MaskParams(w.frames, w.grid_h, w.grid_w, w.frame_window, w.band, w.sink)
    Qd, Kd, Vd = widen(Q), widen(K), widen(V)
    for h in range(Q.shape[0]):
        ref = oracle.route_head(Qd[h], Kd[h], Vd[h], p, rows)
        dense = oracle.attention_rows(Qd[h], Kd[h], Vd[h], oracle.HeadMask(p, oracle.DENSE), rows)
        floor = FLOOR * float(np.mean(dense ** 2))
        bars = []
        for m, want in enumerate((ref.err_spatial, ref.err_temporal)):
            bar = REL * want + floor
            say(f"  {what} head {h} mask {m}: no-alloc {e_na[h, m]:.6e} allocating "
                f"{e_ref[h, m]:.6e} oracle {want:.6e}")
            assert np.isfinite(e_na[h, m])
            assert abs(e_na[h, m] - want) <= bar
            assert abs(e_na[h, m] - e_ref[h, m]) <= 2 * bar
            bars.append(bar)
        if abs(ref.err_spatial - ref.err_temporal) > sum(bars):
            assert k_na[h] == k_ref[h] == ref.kind, (what, h, k_na[h], k_ref[h], ref.kind)


def test_no_alloc_routing_matches_allocating_routing_twice():
    # first call: the main workload's shape (75,600 tokens, 10 heads, d 128)
    w = si.workload("main")
    say(f"[route-noalloc] {w.name} N={w.seq_len} H={w.num_heads}: 96 rows")
    Q, K, V = si.draw_qkv(w)
    _check(w, Q, K, V, si.draw_query_subset(w, 96, seed=78), "main")
    # second call, smaller: fewer tokens, heads and rows (the array keeps the
    # first call's contents)
    w2 = RAGGED
    Q2, K2, V2 = si.draw_qkv(w2)
    rows2 = si.draw_query_subset(w2, 40, seed=9)
    say(f"[route-noalloc] {w2.name} N={w2.seq_len} H={w2.num_heads}: {len(rows2)} rows")
    _check(w2, Q2, K2, V2, rows2, "ragged")


def test_no_alloc_routing_rejects_work_beyond_its_scratch():
    # 1440p: one head's V^T alone is larger than the static array
    w = si.workload("1440p")
    H, N, d = 1, w.seq_len, w.head_dim
    import torch
    q = torch.zeros((H, N, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(svg.SvgError) as e:
        svg.svg_route_heads(q, q, q, w.frames, w.grid_h, w.grid_w, w.frame_window, w.band,
                            np.arange(8), no_alloc=True)
    assert e.value.status == svg.ERR_UNSUPPORTED
    assert "without allocation" in str(e.value)
