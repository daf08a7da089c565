"""Pins of the CPU oracle against facts that do not come from the oracle.

Each check would fail for a plausible mistake in the oracle:
  * closed-form pair counts  -> a wrong window/band bound, a missing sink term;
  * interval-arithmetic tile counts and classes -> wrong layout map, ragged
    tiles counted past N, transposed rows/cols;
  * brute-force scalar attention -> a dropped scale, a wrong softmax axis;
  * dense SDPA agreement, per-frame SDPA -> the mask or softmax itself;
  * row sums, Q=0 count probe -> dropped or double-counted keys;
  * permutation invariance -> the layout maps and their inverses.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from interval_counts import (closed_form_pairs, interval_classes,
                             interval_tile_counts, temporal_hull)
from oracle_cases import masks_of, oracle_kind_map, params_of, widen

TINY = ["tiny", "tiny-misaligned"]

# A small workload that spans several tiles with ragged last tiles in both
# directions (N = 5*9*10 = 450; 450 mod 64 = 2, 450 mod 32 = 2).
RAGGED = si.Workload("ragged", 5, 9, 10, ("spatial", "temporal", "dense"), 64,
                     1, 13, True, 64, 32, False, seed=21)
RAGGED_NOSINK = si.Workload("ragged-nosink", 5, 9, 10, ("spatial", "temporal"),
                            64, 1, 13, False, 64, 32, False, seed=22)


# ---------------------------------------------------------------- pair counts
@pytest.mark.parametrize("name", TINY)
def test_closed_form_pairs_tiny(name):
    w = si.workload(name)
    for kind in w.head_kinds:
        _, _, _, st = oracle_kind_map(w, kind)
        assert st["retained_pairs"] == closed_form_pairs(
            w.frames, w.tokens_per_frame, kind, w.frame_window, w.band, w.sink)


def test_closed_form_pairs_literal_values():
    # Values of the closed forms at the workload shapes (interval arithmetic
    # on the mask definitions, evaluated by hand-checkable formulas).
    assert closed_form_pairs(4, 64, "spatial", 1, 8) == 49_152
    assert closed_form_pairs(4, 64, "temporal", 1, 8) == 28_576
    assert closed_form_pairs(4, 48, "spatial", 1, 8) == 27_648
    assert closed_form_pairs(4, 48, "temporal", 1, 8) == 18_144
    assert closed_form_pairs(21, 3600, "spatial", 4, 700) == 2_397_600_000
    assert closed_form_pairs(21, 3600, "temporal", 4, 700) == 2_184_378_000
    assert closed_form_pairs(21, 14400, "spatial", 4, 2800) == 38_361_600_000
    assert closed_form_pairs(21, 14400, "temporal", 4, 2800) == 34_935_432_000


@pytest.mark.parametrize("w", [RAGGED, RAGGED_NOSINK], ids=lambda w: w.name)
def test_closed_form_pairs_ragged(w):
    for kind in w.head_kinds:
        _, _, _, st = oracle_kind_map(w, kind)
        assert st["retained_pairs"] == closed_form_pairs(
            w.frames, w.tokens_per_frame, kind, w.frame_window, w.band, w.sink)


def test_closed_form_matches_brute_force_pairs():
    # the closed form itself against a brute-force double loop on a tiny grid
    F, Hh, Ww, Wf, Ws = 3, 2, 3, 1, 2
    S = Hh * Ww
    for sink in (True, False):
        sp = tp = 0
        for t in range(F * S):
            for u in range(F * S):
                fq, sq, fk, sk = t // S, t % S, u // S, u % S
                sp += (abs(fq - fk) <= Wf) or (sink and fk == 0)
                tp += (abs(sq - sk) <= Ws) or (sink and fk == 0)
        assert sp == closed_form_pairs(F, S, "spatial", Wf, Ws, sink)
        assert tp == closed_form_pairs(F, S, "temporal", Wf, Ws, sink)


# ---------------------------------------------------------------- tile maps
@pytest.mark.parametrize("w", [si.workload("tiny"), si.workload("tiny-misaligned"),
                               RAGGED, RAGGED_NOSINK], ids=lambda w: w.name)
def test_tile_counts_match_interval_arithmetic(w):
    for kind in set(w.head_kinds):
        counts, cls, _, _ = oracle_kind_map(w, kind)
        ic = interval_tile_counts(w.frames, w.tokens_per_frame, kind,
                                  w.frame_window, w.band, w.sink, w.tile_q, w.tile_k)
        np.testing.assert_array_equal(counts, ic)
        np.testing.assert_array_equal(cls, interval_classes(ic, w.seq_len, w.tile_q, w.tile_k))


def test_tiny_class_and_schedule_counts():
    w = si.workload("tiny")
    sp = oracle_kind_map(w, "spatial")[3]
    tp = oracle_kind_map(w, "temporal")[3]
    assert (sp["skip"], sp["full"], sp["boundary"]) == (16, 48, 0)
    assert (tp["skip"], tp["full"], tp["boundary"]) == (0, 8, 56)
    assert (tp["exec_full"], tp["exec_boundary"], tp["exec_sink"]) == (8, 14, 16)
    w = si.workload("tiny-misaligned")
    sp = oracle_kind_map(w, "spatial")[3]
    tp = oracle_kind_map(w, "temporal")[3]
    assert (sp["skip"], sp["full"], sp["boundary"]) == (6, 24, 6)
    assert (tp["skip"], tp["full"], tp["boundary"]) == (0, 6, 30)
    assert (tp["exec_full"], tp["exec_boundary"], tp["exec_sink"]) == (6, 10, 8)


@pytest.mark.parametrize("w", [si.workload("tiny"), si.workload("tiny-misaligned"),
                               RAGGED, RAGGED_NOSINK], ids=lambda w: w.name)
def test_schedule_matches_closed_form_hull_and_covers_mask(w):
    for kind in set(w.head_kinds):
        counts, cls, sched, st = oracle_kind_map(w, kind)
        assert st["covered_pairs"] == st["retained_pairs"]
        if kind != "temporal":
            assert np.all(sched.sink_a == 0) and np.all(sched.sink_b == w.tokens_per_frame)
            for qt in range(cls.shape[0]):
                np.testing.assert_array_equal(sched.full[qt], np.flatnonzero(cls[qt] == 1))
                np.testing.assert_array_equal(sched.boundary[qt], np.flatnonzero(cls[qt] == 2))
            continue
        lo, hi, a, b = temporal_hull(w.frames, w.tokens_per_frame, w.band,
                                     w.tile_q, w.tile_k, w.sink)
        np.testing.assert_array_equal(sched.sink_a, a)
        np.testing.assert_array_equal(sched.sink_b, b)
        for qt in range(cls.shape[0]):
            ids = np.arange(lo[qt], hi[qt] + 1)
            np.testing.assert_array_equal(sched.full[qt], ids[cls[qt, ids] == 1])
            np.testing.assert_array_equal(sched.boundary[qt], ids[cls[qt, ids] == 2])


def test_main_shape_sampled_tiles_match_interval_arithmetic():
    w = si.workload("main")
    p = params_of(w)
    qt = [0, 1, 13, 148, 200, 294, 295]          # includes the ragged last tile
    for kind in ("spatial", "temporal"):
        m = oracle.HeadMask(p, kind)
        c = oracle.tile_counts(m, w.tile_q, w.tile_k, qtiles=qt)
        ic = interval_tile_counts(w.frames, w.tokens_per_frame, kind,
                                  w.frame_window, w.band, w.sink, w.tile_q, w.tile_k)
        np.testing.assert_array_equal(c, ic[qt])
        cls = oracle.tile_classes(c, p.N, w.tile_q, w.tile_k, qtiles=qt)
        sched = oracle.head_schedule(m, cls, w.tile_q, w.tile_k, qtiles=qt)
        if kind == "temporal":
            lo, hi, a, b = temporal_hull(w.frames, w.tokens_per_frame, w.band,
                                         w.tile_q, w.tile_k)
            np.testing.assert_array_equal(sched.sink_a, a[qt])
            np.testing.assert_array_equal(sched.sink_b, b[qt])


def test_main_shape_interval_totals():
    # Whole-map class counts at 75,600 tokens, BQ=256, BK=128, by interval
    # arithmetic: the numbers the GPU tile map must reproduce.
    w = si.workload("main")
    sp = interval_classes(interval_tile_counts(21, 3600, "spatial", 4, 700, True, 256, 128),
                          w.seq_len, 256, 128)
    tc = interval_tile_counts(21, 3600, "temporal", 4, 700, True, 256, 128)
    tp = interval_classes(tc, w.seq_len, 256, 128)
    assert [(sp == k).sum() for k in (0, 1, 2)] == [100_842, 72_687, 1_407]
    assert [(tp == k).sum() for k in (0, 1, 2)] == [0, 60_515, 114_421]
    lo, hi, a, b = temporal_hull(21, 3600, 700, 256, 128)
    full = sum(int((tp[q, lo[q]:hi[q] + 1] == 1).sum()) for q in range(tp.shape[0]))
    bnd = sum(int((tp[q, lo[q]:hi[q] + 1] == 2).sum()) for q in range(tp.shape[0]))
    sink = int((-(-a // 128)).sum() + (-(-(3600 - b) // 128)).sum())
    assert (full, bnd, sink) == (60_515, 1_371, 5_612)


# ---------------------------------------------------------------- rounded mask
@pytest.mark.parametrize("name", TINY)
def test_tile_aligned_mask_is_superset_with_no_masked_hull_tiles(name):
    w = si.workload(name)
    wa = si.Workload(w.name + "-ta", w.frames, w.grid_h, w.grid_w, w.head_kinds,
                     w.head_dim, w.frame_window, w.band, w.sink, w.tile_q,
                     w.tile_k, True, w.seed)
    p = params_of(w)
    cols = np.arange(p.N)
    for kind in set(w.head_kinds):
        exact = oracle.HeadMask(p, kind)
        rnd = oracle.HeadMask(p, kind, True, w.tile_q, w.tile_k)
        E = exact.kernel_block(cols, cols)
        R = rnd.kernel_block(cols, cols)
        assert np.all(R[E])                      # superset
        counts, cls, sched, st = oracle_kind_map(wa, kind)
        assert st["exec_boundary"] == 0          # no predicate tiles run
        assert st["covered_pairs"] == st["retained_pairs"] == int(R.sum())
        ic = interval_tile_counts(w.frames, w.tokens_per_frame, kind,
                                  w.frame_window, w.band, w.sink, w.tile_q,
                                  w.tile_k, tile_aligned=True)
        np.testing.assert_array_equal(counts, ic)
    # tiny temporal: 33,280 pairs after rounding (drift +16.46%)
    if name == "tiny":
        assert oracle_kind_map(wa, "temporal")[3]["retained_pairs"] == 33_280


def test_tile_aligned_main_totals_by_interval_arithmetic():
    sp = interval_tile_counts(21, 3600, "spatial", 4, 700, True, 256, 128, tile_aligned=True)
    tp = interval_tile_counts(21, 3600, "temporal", 4, 700, True, 256, 128, tile_aligned=True)
    assert int(sp.sum()) == 2_423_218_432
    assert int(tp.sum()) == 2_200_303_616


# ---------------------------------------------------------------- attention
def _sdpa(q, k, v, attn_mask=None):
    q, k, v = (torch.from_numpy(x)[None] for x in (q, k, v))
    m = None if attn_mask is None else torch.from_numpy(attn_mask)[None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m)[0].numpy()


def _brute(q, k, v, keep):
    N, d = k.shape
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((q.shape[0], v.shape[1]))
    for i in range(q.shape[0]):
        s = [scale * sum(float(q[i, c]) * float(k[j, c]) for c in range(d))
             if keep[i, j] else None for j in range(N)]
        m = max(x for x in s if x is not None)
        e = [math.exp(x - m) if x is not None else 0.0 for x in s]
        z = sum(e)
        for c in range(v.shape[1]):
            out[i, c] = sum(e[j] * float(v[j, c]) for j in range(N)) / z
    return out


def test_brute_force_scalar_attention_tiny():
    w = si.workload("tiny-misaligned")
    Q, K, V = (widen(x) for x in si.draw_qkv(w))
    rows = np.array([0, 5, 47, 48, 100, 150, 191])
    S = w.tokens_per_frame

    def scalar_keep(kind, t, u):
        fq, sq, fk, sk = t // S, t % S, u // S, u % S
        if kind == "spatial":
            return abs(fq - fk) <= w.frame_window or fk == 0
        return abs(sq - sk) <= w.band or fk == 0

    for h, m in enumerate(masks_of(w)):
        o = oracle.attention_rows(Q[h], K[h], V[h], m, rows)
        keep = np.array([[scalar_keep(w.head_kinds[h], int(t), u)
                          for u in range(w.seq_len)] for t in rows])
        ref = _brute(Q[h][rows], K[h], V[h][:, :8], keep)
        np.testing.assert_allclose(o[:, :8], ref, atol=1e-12, rtol=0)


def test_dense_matches_sdpa():
    w = RAGGED
    Q, K, V = (widen(x) for x in si.draw_qkv(w))
    m = oracle.HeadMask(params_of(w), "dense")
    o = oracle.attention_rows(Q[2], K[2], V[2], m, np.arange(w.seq_len))
    np.testing.assert_allclose(o, _sdpa(Q[2], K[2], V[2]), atol=1e-12, rtol=0)


def test_wide_window_and_band_reduce_to_dense():
    w = RAGGED
    Q, K, V = (widen(x) for x in si.draw_qkv(w))
    ref = _sdpa(Q[0], K[0], V[0])
    for kind, Wf, Ws in (("spatial", w.frames - 1, 0), ("temporal", 0, w.tokens_per_frame - 1)):
        p = oracle.MaskParams(w.frames, w.grid_h, w.grid_w, Wf, Ws, False)
        o = oracle.attention_rows(Q[0], K[0], V[0], oracle.HeadMask(p, kind),
                                  np.arange(w.seq_len))
        np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_frame_diagonal_mask_is_per_frame_sdpa():
    w = RAGGED
    Q, K, V = (widen(x) for x in si.draw_qkv(w))
    p = oracle.MaskParams(w.frames, w.grid_h, w.grid_w, 0, 0, False)
    o = oracle.attention_rows(Q[0], K[0], V[0], oracle.HeadMask(p, "spatial"),
                              np.arange(w.seq_len))
    S = w.tokens_per_frame
    for f in range(w.frames):
        sl = slice(f * S, (f + 1) * S)
        np.testing.assert_allclose(o[sl], _sdpa(Q[0][sl], K[0][sl], V[0][sl]),
                                   atol=1e-12, rtol=0)


def test_explicit_mask_matches_sdpa_with_bool_mask():
    # A library routine with the oracle's mask as an input: checks the softmax
    # and masking step independently of the mask construction.
    w = RAGGED
    Q, K, V = (widen(x) for x in si.draw_qkv(w))
    for h, m in enumerate(masks_of(w)):
        keep = m.original_block(np.arange(w.seq_len), np.arange(w.seq_len))
        o = oracle.attention_rows(Q[h], K[h], V[h], m, np.arange(w.seq_len))
        np.testing.assert_allclose(o, _sdpa(Q[h], K[h], V[h], keep), atol=1e-12, rtol=0)


def test_softmax_rows_sum_to_one():
    w = RAGGED
    Q, K, _ = (widen(x) for x in si.draw_qkv(w))
    ones = np.ones((w.seq_len, 3))
    for h, m in enumerate(masks_of(w)):
        o = oracle.attention_rows(Q[h], K[h], ones, m, np.arange(w.seq_len))
        np.testing.assert_allclose(o, 1.0, atol=1e-12, rtol=0)


def test_zero_query_count_probe_closed_form():
    # Q = 0: every retained key gets weight 1/n_row. With V[:,0] = 1 and
    # V[:,1] = [key in frame 0], o[:,1] = (frame-0 keys kept) / n_row, which
    # has a closed form per row.
    w = si.workload("tiny-misaligned")
    p = params_of(w)
    S, F, N = w.tokens_per_frame, w.frames, w.seq_len
    t = np.arange(N)
    f, s = t // S, t % S
    V = np.stack([np.ones(N), (f == 0).astype(float)], axis=1)
    Q0 = np.zeros((N, 4))
    K = np.random.default_rng(0).standard_normal((N, 4))
    for kind in ("spatial", "temporal"):
        o = oracle.attention_rows(Q0, K, V, oracle.HeadMask(p, kind), t)
        if kind == "spatial":
            nf = np.array([min(F - 1, x + 1) - max(0, x - 1) + 1 + (x - 1 > 0) for x in f])
            n_row = nf * S
            n_sink = np.full(N, S)
        else:
            band = np.minimum(S - 1, s + w.band) - np.maximum(0, s - w.band) + 1
            n_row = band * F + (S - band)
            n_sink = np.full(N, S)
        np.testing.assert_allclose(o[:, 0], 1.0, atol=1e-12)
        np.testing.assert_allclose(o[:, 1], n_sink / n_row, atol=1e-12)


def test_permuting_tokens_and_mask_permutes_output():
    w = RAGGED
    Q, K, V = (widen(x) for x in si.draw_qkv(w))
    perm = np.random.default_rng(5).permutation(w.seq_len)
    allr = np.arange(w.seq_len)

    class Permuted:
        def __init__(self, base):
            self.base = base

        def original_block(self, r, c):
            return self.base.original_block(perm[r], perm[c])

    for h, m in enumerate(masks_of(w)):
        o = oracle.attention_rows(Q[h], K[h], V[h], m, allr)
        op = oracle.attention_rows(Q[h][perm], K[h][perm], V[h][perm], Permuted(m), allr)
        np.testing.assert_allclose(op, o[perm], atol=1e-12, rtol=0)


def test_kernel_layout_round_trip_and_coordinates():
    w = RAGGED
    p = params_of(w)
    x = np.arange(p.N * 2).reshape(p.N, 2)
    t = np.arange(p.N)
    for kind in ("spatial", "temporal", "dense"):
        y = oracle.to_kernel_layout(p, kind, x)
        np.testing.assert_array_equal(oracle.to_original_layout(p, kind, y), x)
        pos = oracle.kernel_position(p, kind, t)
        assert sorted(pos.tolist()) == t.tolist()
        f0, s0 = oracle.original_coords(p, t)
        f1, s1 = oracle.kernel_coords(p, kind, pos)
        np.testing.assert_array_equal(f0, f1)
        np.testing.assert_array_equal(s0, s1)
    # temporal order is spatial-major: consecutive positions step the frame
    f, s = oracle.kernel_coords(p, "temporal", np.arange(2 * p.frames))
    assert f.tolist() == list(range(p.frames)) * 2
    assert s.tolist() == [0] * p.frames + [1] * p.frames


# Executed tiles per head of the exact main masks at every swept tile pair,
# (spatial, temporal), and the BOUNDARY tiles among them: the table computed
# from the mask definitions alone. The golden digests the GPU maps are
# compared with must carry the same figures.
EXACT_SWEEP_EXECUTED = {
    (128, 64): (294_320, 268_327), (128, 128): (147_597, 134_405),
    (128, 256): (74_305, 67_730), (256, 64): (147_751, 134_755),
    (256, 128): (74_094, 67_498), (256, 256): (37_301, 34_126),
    (512, 64): (74_213, 67_830), (512, 128): (37_215, 33_975),
    (512, 256): (18_734, 17_176),
}


@pytest.mark.slow
@pytest.mark.parametrize("bq,bk", si.SWEEP_TILES)
def test_exact_main_sweep_executed_tiles(bq, bk):
    import json
    import os
    F, S, Wf, Ws = 21, 3600, 4, 700
    N = F * S
    sp = interval_classes(interval_tile_counts(F, S, "spatial", Wf, Ws, True, bq, bk), N, bq, bk)
    tp = interval_classes(interval_tile_counts(F, S, "temporal", Wf, Ws, True, bq, bk), N, bq, bk)
    lo, hi, a, b = temporal_hull(F, S, Ws, bq, bk)
    t_full = sum(int((tp[q, lo[q]:hi[q] + 1] == 1).sum()) for q in range(tp.shape[0]))
    t_bnd = sum(int((tp[q, lo[q]:hi[q] + 1] == 2).sum()) for q in range(tp.shape[0]))
    t_sink = int((-(-a // bk)).sum() + (-(-(S - b) // bk)).sum())
    s_full, s_bnd = int((sp == 1).sum()), int((sp == 2).sum())
    assert (s_full + s_bnd, t_full + t_bnd + t_sink) == EXACT_SWEEP_EXECUTED[(bq, bk)]
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", "tilemaps.json")) as f:
        g = json.load(f)
    key = "main@256x128" if (bq, bk) == (256, 128) else f"main-{bq}x{bk}@{bq}x{bk}"
    gs, gt = g[key]["kinds"]["spatial"]["stats"], g[key]["kinds"]["temporal"]["stats"]
    assert (gs["exec_full"], gs["exec_boundary"], gs["exec_sink"]) == (s_full, s_bnd, 0)
    assert (gt["exec_full"], gt["exec_boundary"], gt["exec_sink"]) == (t_full, t_bnd, t_sink)
