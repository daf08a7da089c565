"""Sampled head routing (svg_route_heads) on the GPU against the oracle.

Errors: the GPU rounds P to bf16 for the PV product (fp32 accumulation), the
oracle is float64. A rounding error of at most 2^-9 per weight averages over
the kept keys of a row, so an output moves by well under 2^-9 of its size;
the measured deviation of a mask error from the oracle's is at most 4.1e-4
of its value over the cases below (the worst on 1-3 rows of a 450-token
sequence). The bar is 5e-3 of the oracle's value plus a floor of 1e-4 times
the mean squared dense output, for errors near zero (a mask that keeps
nearly every weight), where two independent rounding errors dominate. A
routing decision is compared where the oracle's two errors differ by more
than both bars; closer than that, either kind is a correct result and only
its validity is checked.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import structured_sparse_attention_amd as svg
from gpu_harness import say, to_device
from oracle_cases import widen
from test_oracle_pins import RAGGED, RAGGED_NOSINK

pytestmark = pytest.mark.gpu

REL, FLOOR = 5e-3, 1e-4


def _params(w):
    return oracle.MaskParams(w.frames, w.grid_h, w.grid_w, w.frame_window, w.band, w.sink)


def _compare(w, Q, K, V, rows, what, expect=None):
    q, k, v = (to_device(x) for x in (Q, K, V))
    kinds, err = svg.svg_route_heads(q, k, v, w.frames, w.grid_h, w.grid_w, w.frame_window,
                                     w.band, rows, sink_first_frame=w.sink)
    p = _params(w)
    Qd, Kd, Vd = widen(Q), widen(K), widen(V)
    decided = 0
    for h in range(Q.shape[0]):
        ref = oracle.route_head(Qd[h], Kd[h], Vd[h], p, rows)
        dense = oracle.attention_rows(Qd[h], Kd[h], Vd[h], oracle.HeadMask(p, oracle.DENSE), rows)
        floor = FLOOR * float(np.mean(dense ** 2))
        bars = []
        for got, want in ((err[h, 0], ref.err_spatial), (err[h, 1], ref.err_temporal)):
            bar = REL * want + floor
            say(f"  {what} head {h}: gpu {got:.6e} oracle {want:.6e} (bar {bar:.1e})")
            assert np.isfinite(got) and abs(got - want) <= bar, (what, h, got, want)
            bars.append(bar)
        assert kinds[h] in ("spatial", "temporal")
        if abs(ref.err_spatial - ref.err_temporal) > sum(bars):
            assert kinds[h] == ref.kind, (what, h, kinds[h], ref)
            decided += 1
        if expect is not None:
            assert kinds[h] == expect[h], (what, h, kinds[h], expect[h])
    return kinds, decided


CASES = [si.workload("tiny"), si.workload("tiny-misaligned"), RAGGED, RAGGED_NOSINK,
         si.Workload("one-frame", 1, 7, 9, ("spatial", "temporal", "dense"), 64, 0, 3, True,
                     32, 32, False, seed=31),
         si.Workload("d128-multi-tile", 6, 12, 16, ("spatial", "temporal"), 128, 1, 40, True,
                     256, 128, False, seed=36),
         # frames shorter than a 32-key step (keys of 3+ frames per step)
         si.Workload("short-frames", 9, 3, 5, ("spatial", "temporal"), 64, 1, 2, True, 32, 32,
                     False, seed=42),
         si.Workload("short-frames-nosink", 9, 3, 5, ("spatial", "temporal"), 128, 2, 1, False,
                     32, 32, False, seed=43),
         # one token; one token per frame (every step spans 32 frames)
         si.Workload("one-token", 1, 1, 1, ("spatial", "temporal"), 64, 0, 0, True, 32, 32,
                     False, seed=44),
         si.Workload("token-frames", 70, 1, 1, ("spatial", "temporal"), 128, 3, 0, True, 32, 32,
                     False, seed=45)]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_routing_errors_match_oracle_small(w):
    say(f"[route] {w.name} N={w.seq_len} H={w.num_heads} d={w.head_dim}")
    Q, K, V = si.draw_qkv(w)
    rows = np.arange(w.seq_len) if w.seq_len <= 512 else si.draw_query_subset(w, 300)
    _compare(w, Q, K, V, rows, w.name)


def _planted(w, seed):
    """Head 0: scores 30 inside a query's own frame, else 0; head 1: inside its
    own raster index; V random. bf16-exact values."""
    N, S, d = w.seq_len, w.tokens_per_frame, w.head_dim
    t = np.arange(N)
    alpha = 30.0 * math.sqrt(d)
    Q = np.zeros((2, N, d), np.float32)
    K = np.zeros((2, N, d), np.float32)
    K[0, t, t // S] = 1.0
    K[1, t, t % S] = 1.0
    Q[:] = alpha * K
    V = np.random.default_rng(seed).standard_normal((2, N, d)).astype(np.float32)
    return tuple(si.f32_to_bf16_bits(x) for x in (Q, K, V))


def test_planted_heads_route_to_their_masks():
    w = si.Workload("planted", 6, 6, 8, ("spatial", "temporal"), 64, 1, 2, True, 32, 32,
                    False, seed=41)
    say(f"[route-planted] N={w.seq_len} S={w.tokens_per_frame}")
    Q, K, V = _planted(w, 41)
    rows = np.arange(0, w.seq_len, 5)
    kinds, decided = _compare(w, Q, K, V, rows, "planted", expect=["spatial", "temporal"])
    assert decided == 2


def _far_maximum(w, j_star, seed):
    """Every query scores 100 (natural log units) on key j_star and 0 on every
    other key; V random. bf16-exact values."""
    N, d = w.seq_len, w.head_dim
    Q = np.zeros((1, N, d), np.float32)
    K = np.zeros((1, N, d), np.float32)
    Q[0, :, 0] = 100.0 * math.sqrt(d)
    K[0, j_star, 0] = 1.0
    V = np.random.default_rng(seed).standard_normal((1, N, d)).astype(np.float32)
    return tuple(si.f32_to_bf16_bits(x) for x in (Q, K, V))


@pytest.mark.parametrize("case", ["outside-both", "inside-temporal"])
def test_far_maximum_outside_a_mask(case):
    # The dense maximum (key j* = frame 5, raster index 40) lies 144 log2
    # units above every other score. Rows in frames 0-3 never keep j* under
    # the spatial mask (W_f = 1): that mask's weights, measured against the
    # dense maximum, fall below fp32's normal range, and its output must be
    # the plain average of its kept V rows all the same. Rows at raster
    # indices 38-42 keep j* under the temporal mask (W_s = 2); rows at 0-30
    # keep it under neither.
    w = si.Workload("far-max", 6, 6, 8, ("spatial",), 64, 1, 2, True, 32, 32, False, seed=46)
    S = w.tokens_per_frame
    Q, K, V = _far_maximum(w, 5 * S + 40, 46)
    cols = (38, 39, 40, 41, 42) if case == "inside-temporal" else (0, 7, 15, 22, 30)
    rows = np.array([f * S + c for f in range(4) for c in cols])
    say(f"[route-far-max] {case}: {len(rows)} rows")
    kinds, decided = _compare(w, Q, K, V, rows, case,
                              expect=["temporal"] if case == "inside-temporal" else None)


def test_single_repeated_and_edge_rows():
    w = RAGGED
    Q, K, V = si.draw_qkv(w)
    for rows in (np.array([0]), np.array([w.seq_len - 1] * 3 + [0, 0]),
                 np.array([w.tokens_per_frame - 1, w.tokens_per_frame])):
        say(f"[route-rows] {rows.tolist()}")
        _compare(w, Q, K, V, rows, f"rows {rows.tolist()}")


@pytest.mark.timeout(600)
def test_routing_main_workload_sampled_rows():
    w = si.workload("main")
    say(f"[route-main] N={w.seq_len} H={w.num_heads}: 64 sampled rows")
    Q, K, V = si.draw_qkv(w)
    rows = si.draw_query_subset(w, 64, seed=77)
    kinds, decided = _compare(w, Q, K, V, rows, "main")
    say(f"  kinds {kinds}, {decided} decided beyond the error bars")


@pytest.mark.timeout(900)
def test_routing_main_workload_one_percent_of_rows():
    """The bench's larger routing case: 1% of the tokens (756 rows), six
    128-row blocks per head, the last ragged, over a few long key splits."""
    w = si.workload("main")
    n = w.seq_len // 100
    say(f"[route-main-1pct] N={w.seq_len} H={w.num_heads}: {n} sampled rows")
    Q, K, V = si.draw_qkv(w)
    rows = si.draw_query_subset(w, n, seed=77)
    kinds, decided = _compare(w, Q, K, V, rows, "main-1pct")
    say(f"  kinds {kinds}, {decided} decided beyond the error bars")


def test_routing_rejects_bad_rows():
    w = si.workload("tiny")
    Q, K, V = si.draw_qkv(w)
    q, k, v = (to_device(x) for x in (Q, K, V))
    for rows in (np.array([w.seq_len]), np.array([-1]), np.zeros(0, np.int32)):
        with pytest.raises(svg.SvgError) as e:
            svg.svg_route_heads(q, k, v, w.frames, w.grid_h, w.grid_w, w.frame_window, w.band,
                                rows)
        assert e.value.status == svg.ERR_INVALID_ARG


def test_windows_beyond_the_sequence_match_whole_sequence_windows():
    # A band or window as wide as int32 allows keeps every pair of its kind,
    # like one as wide as the sequence: the call clamps both before the
    # kernels' interval arithmetic, which would otherwise overflow.
    w = RAGGED
    Q, K, V = si.draw_qkv(w)
    rows = si.draw_query_subset(w, 64, seed=5)
    q, k, v = (to_device(x) for x in (Q, K, V))
    big = 2 ** 31 - 1
    say(f"[route-wide] N={w.seq_len}: W_f = W_s = {big}")
    k1, e1 = svg.svg_route_heads(q, k, v, w.frames, w.grid_h, w.grid_w, big, big, rows,
                                 sink_first_frame=w.sink)
    k2, e2 = svg.svg_route_heads(q, k, v, w.frames, w.grid_h, w.grid_w, w.frames - 1,
                                 w.tokens_per_frame - 1, rows, sink_first_frame=w.sink)
    np.testing.assert_array_equal(e1, e2)
    assert k1 == k2
    wide = si.Workload(w.name + "-wide", w.frames, w.grid_h, w.grid_w, w.head_kinds,
                       w.head_dim, big, big, w.sink, w.tile_q, w.tile_k, False, w.seed)
    _compare(wide, Q, K, V, rows, "int32-wide windows")
