"""Write tests/golden/tilemaps.json: oracle tile maps of every workload.

Calls only ``oracle/`` (and ``seeded_inputs`` for the workload shapes). For
each workload and tile size, and each head kind, it stores the SHA-256 of the
oracle's class map and schedule (canonical form in ``canonical.py``) and the
per-head statistics. The GPU tests compare the HIP tile map with these.

Usage:  python tests/golden/make_tilemap_golden.py [--jobs 8] [--only NAME]
Q tiles are spread over worker processes; the oracle itself is unchanged.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from multiprocessing import get_context

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import seeded_inputs as si  # noqa: E402
from canonical import class_digest, golden_key, schedule_digest  # noqa: E402

OUT = os.path.join(HERE, "tilemaps.json")


def cases():
    out = []
    for name in ("tiny", "tiny-misaligned", "main", "dense", "1440p"):
        out.append(si.workload(name))
    ta = si.workload("tile-aligned")
    for bq, bk in si.SWEEP_TILES:
        out.append(ta.with_tiles(bq, bk))
    # the exact masks of the main workload at every swept tile pair (the
    # pair the tile search picks is the one a caller runs)
    main = si.workload("main")
    for bq, bk in si.SWEEP_TILES:
        if (bq, bk) != (main.tile_q, main.tile_k):
            out.append(main.with_tiles(bq, bk))
    return out


def _params(w):
    return oracle.MaskParams(w.frames, w.grid_h, w.grid_w, w.frame_window,
                             w.band, w.sink)


def _chunk(args):
    w, kind, qts = args
    m = oracle.HeadMask(_params(w), kind, w.tile_aligned, w.tile_q, w.tile_k)
    counts = oracle.tile_counts(m, w.tile_q, w.tile_k, qtiles=qts)
    cls = oracle.tile_classes(counts, m.p.N, w.tile_q, w.tile_k, qtiles=qts)
    sched = oracle.head_schedule(m, cls, w.tile_q, w.tile_k, qtiles=qts)
    return qts, counts, cls, sched


def kind_map(w, kind, pool, jobs):
    N = w.seq_len
    nq = -(-N // w.tile_q)
    per = max(1, -(-nq // (jobs * 4)))
    chunks = [list(range(i, min(nq, i + per))) for i in range(0, nq, per)]
    parts = pool.map(_chunk, [(w, kind, c) for c in chunks])
    counts = np.concatenate([p[1] for p in parts])
    cls = np.concatenate([p[2] for p in parts])
    sched = oracle.TileSchedule(
        full=[x for p in parts for x in p[3].full],
        boundary=[x for p in parts for x in p[3].boundary],
        sink_a=np.concatenate([p[3].sink_a for p in parts]),
        sink_b=np.concatenate([p[3].sink_b for p in parts]))
    m = oracle.HeadMask(_params(w), kind, w.tile_aligned, w.tile_q, w.tile_k)
    stats = oracle.head_stats(m, counts, cls, sched, w.tile_q, w.tile_k)
    return {
        "classes_sha256": class_digest(cls),
        "schedule_sha256": schedule_digest(sched.full, sched.boundary,
                                           sched.sink_a, sched.sink_b),
        "stats": stats,
        "nq": int(cls.shape[0]),
        "nk": int(cls.shape[1]),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--only", default=None)
    a = ap.parse_args()
    db = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            db = json.load(f)
    with get_context("fork").Pool(a.jobs) as pool:
        for w in cases():
            key = golden_key(w.name, w.tile_q, w.tile_k)
            if a.only and a.only not in key:
                continue
            t0 = time.time()
            entry = {"workload": w.name, "tile_q": w.tile_q, "tile_k": w.tile_k,
                     "tile_aligned": w.tile_aligned, "kinds": {}}
            for kind in sorted(set(w.head_kinds)):
                entry["kinds"][kind] = kind_map(w, kind, pool, a.jobs)
            db[key] = entry
            with open(OUT, "w") as f:
                json.dump(db, f, indent=1, sort_keys=True)
            print(f"{key}: {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    main()
