"""HIP tile map vs the oracle, bit-exact: class map, schedule and statistics.

Small workloads are compared with the oracle run live; the large ones with
digests the oracle wrote (tests/golden/make_tilemap_golden.py).
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest

import seeded_inputs as si

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
from canonical import class_digest, golden_key, schedule_digest  # noqa: E402

with open(os.path.join(HERE, "golden", "tilemaps.json")) as _f:
    GOLDEN = json.load(_f)

STAT_KEYS = ("tiles", "skip", "full", "boundary", "exec_full", "exec_boundary",
             "exec_sink", "retained_pairs")


def _small_workloads():
    from test_oracle_pins import RAGGED, RAGGED_NOSINK
    base = [si.workload("tiny"), si.workload("tiny-misaligned"), RAGGED, RAGGED_NOSINK]
    out = list(base)
    for w in base:
        out.append(si.Workload(w.name + "-ta", w.frames, w.grid_h, w.grid_w, w.head_kinds,
                               w.head_dim, w.frame_window, w.band, w.sink, w.tile_q,
                               w.tile_k, True, w.seed))
    # ragged tiles of other sizes, single ragged tile, degenerate shapes
    out.append(RAGGED.with_tiles(128, 64))
    out.append(RAGGED.with_tiles(512, 256))
    out.append(si.Workload("one-frame", 1, 7, 9, ("spatial", "temporal", "dense"), 64,
                           0, 3, True, 32, 32, False, seed=31))
    out.append(si.Workload("one-token", 1, 1, 1, ("spatial", "temporal"), 64, 0, 0, True,
                           32, 32, False, seed=32))
    out.append(si.Workload("wide", 3, 5, 7, ("spatial", "temporal"), 64, 9, 999, True,
                           64, 96, False, seed=33))
    out.append(si.Workload("narrow", 6, 4, 5, ("spatial", "temporal"), 64, 0, 0, False,
                           32, 64, False, seed=34))
    # the same degenerate shapes with the tile-aligned mask
    for w in list(out[-4:]):
        out.append(si.Workload(w.name + "-ta", w.frames, w.grid_h, w.grid_w, w.head_kinds,
                               w.head_dim, w.frame_window, w.band, w.sink, w.tile_q,
                               w.tile_k, True, w.seed))
    return out


@pytest.mark.parametrize("w", _small_workloads(), ids=lambda w: w.name)
def test_tile_map_matches_live_oracle(w):
    from gpu_harness import build_map, gpu_head_schedule, say
    from oracle_cases import oracle_kind_map
    say(f"[tilemap] {w.name} BQ={w.tile_q} BK={w.tile_k} aligned={w.tile_aligned}")
    tm = build_map(w)
    cls = tm.classes()
    stats = tm.stats()
    for h, kind in enumerate(w.head_kinds):
        counts, ocls, osched, ost = oracle_kind_map(w, kind)
        np.testing.assert_array_equal(cls[h], ocls, err_msg=f"classes head {h} ({kind})")
        full, bnd, a, b = gpu_head_schedule(tm, h)
        for qt in range(ocls.shape[0]):
            np.testing.assert_array_equal(full[qt], osched.full[qt], err_msg=f"full h{h} qt{qt}")
            np.testing.assert_array_equal(bnd[qt], osched.boundary[qt], err_msg=f"bnd h{h} qt{qt}")
        np.testing.assert_array_equal(a, osched.sink_a)
        np.testing.assert_array_equal(b, osched.sink_b)
        for k in STAT_KEYS:
            assert stats[h][k] == ost[k], (h, k, stats[h][k], ost[k])
    tm.destroy()


def _golden_workloads():
    out = [si.workload("main"), si.workload("dense"), si.workload("1440p")]
    ta = si.workload("tile-aligned")
    out += [ta.with_tiles(bq, bk) for bq, bk in si.SWEEP_TILES]
    main = si.workload("main")
    out += [main.with_tiles(bq, bk) for bq, bk in si.SWEEP_TILES
            if (bq, bk) != (main.tile_q, main.tile_k)]
    return out


@pytest.mark.parametrize("w", _golden_workloads(), ids=lambda w: f"{w.name}@{w.tile_q}x{w.tile_k}")
def test_tile_map_matches_oracle_digest(w):
    from gpu_harness import build_map, gpu_head_schedule, say
    say(f"[tilemap-digest] {w.name} BQ={w.tile_q} BK={w.tile_k}")
    g = GOLDEN[golden_key(w.name, w.tile_q, w.tile_k)]
    tm = build_map(w)
    cls = tm.classes()
    stats = tm.stats()
    for h, kind in enumerate(w.head_kinds):
        ref = g["kinds"][kind]
        assert cls.shape[1:] == (ref["nq"], ref["nk"])
        for k in STAT_KEYS:
            assert stats[h][k] == ref["stats"][k], (h, kind, k, stats[h][k], ref["stats"][k])
        assert class_digest(cls[h]) == ref["classes_sha256"], f"classes head {h}"
        full, bnd, a, b = gpu_head_schedule(tm, h)
        assert schedule_digest(full, bnd, a, b) == ref["schedule_sha256"], f"schedule head {h}"
    tm.destroy()


def test_main_map_totals_match_interval_arithmetic():
    # the device map's totals against the closed-form / interval figures
    from gpu_harness import build_map
    tm = build_map(si.workload("main"))
    st = tm.stats()
    for h in range(5):
        assert (st[h]["skip"], st[h]["full"], st[h]["boundary"]) == (100_842, 72_687, 1_407)
        assert st[h]["retained_pairs"] == 2_397_600_000
    for h in range(5, 10):
        assert (st[h]["skip"], st[h]["full"], st[h]["boundary"]) == (0, 60_515, 114_421)
        assert (st[h]["exec_full"], st[h]["exec_boundary"], st[h]["exec_sink"]) == (60_515, 1_371, 5_612)
        assert st[h]["retained_pairs"] == 2_184_378_000
    tm.destroy()


def test_rebuild_in_place_is_identical():
    from gpu_harness import build_map
    tm = build_map(si.workload("main"))
    c1, s1 = tm.classes(), tm.schedule()
    tm.rebuild()
    c2, s2 = tm.classes(), tm.schedule()
    np.testing.assert_array_equal(c1, c2)
    for x, y in zip(s1, s2):
        np.testing.assert_array_equal(x, y)
    tm.destroy()
