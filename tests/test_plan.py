"""The persistent attention launch's work plan (host code, no GPU).

The planner is compiled with the host compiler beside a small driver and fed
step counts: every step of every unit must be executed exactly once, in
contiguous parts from step 0, the last part running to the end of the row;
split units must own consecutive partial-result slots listed in a combine
entry; the workgroups must end level on realistic row lengths.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structured_sparse_attention_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "native", "plan_driver.cpp")
TO_END = 0x7FFFFFFF


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_driver")
    subprocess.run([gxx, "-O2", "-std=c++17", "-I", CSRC, DRIVER, os.path.join(CSRC, "plan.cpp"),
                    "-o", exe], check=True)

    def run(steps, n_wg=256, n_xcd=8, overhead=4, min_part=32, block=16, weights=None, tail=0.0):
        steps = [int(s) for s in steps]
        inp = (f"{len(steps)} {n_wg} {n_xcd} {block} {overhead} {min_part} "
               f"{0 if weights is None else 1} {tail!r}\n" + " ".join(map(str, steps)))
        if weights is not None:
            inp += "\n" + " ".join(f"{float(x):.6f}" for x in weights)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        lines = out.splitlines()
        P, n_slots, max_load, total_load, n_items, n_comb = map(int, lines[0].split())
        item_ptr = list(map(int, lines[1].split()))
        items = [tuple(map(int, l.split())) for l in lines[2:2 + n_items]]
        comb = [tuple(map(int, l.split())) for l in lines[2 + n_items:2 + n_items + n_comb]]
        k = 2 + n_items + n_comb
        queue_ptr = list(map(int, lines[k].split()))
        queue = [tuple(map(int, l.split())) for l in lines[k + 1:k + 1 + n_items]]
        return dict(P=P, n_slots=n_slots, max_load=max_load, total_load=total_load,
                    item_ptr=item_ptr, items=items, combine=comb, queue_ptr=queue_ptr,
                    queue=queue, n_xcd=n_xcd)
    return run


def check_plan(steps, plan, n_wg, overhead=4, weights=None):
    P = plan["P"]
    assert P == n_wg and len(plan["item_ptr"]) == P + 1 and plan["item_ptr"][0] == 0
    assert plan["item_ptr"][-1] == len(plan["items"])
    n_valid = sum(1 for s in steps if s >= 0)
    assert len(plan["items"]) <= n_valid + 5 * P
    assert plan["n_slots"] <= 5 * P
    parts = {}
    load = np.zeros(P)
    wt = [1.0] * len(steps) if weights is None else [float(np.float32(x)) for x in weights]
    for i in range(P):
        for unit, s0, s1, slot in plan["items"][plan["item_ptr"][i]:plan["item_ptr"][i + 1]]:
            parts.setdefault(unit, []).append((s0, s1, slot, i))
            end = steps[unit] if s1 == TO_END else s1
            load[i] += wt[unit] * (end - s0) + overhead
    assert sorted(parts) == [u for u, s in enumerate(steps) if s >= 0]
    X = min(plan["n_xcd"], P)
    qp = plan["queue_ptr"]
    tail_units = {it[0] for it in plan["queue"][qp[X]:qp[X + 1]]}
    comb = {u: (slot0, n) for u, slot0, n in plan["combine"]}
    assert len(comb) == len(plan["combine"])
    slots_seen = []
    for unit, ps in parts.items():
        ps.sort()
        assert ps[0][0] == 0 and ps[-1][1] == TO_END, (unit, ps)
        for (a0, a1, _, _), (b0, _, _, _) in zip(ps, ps[1:]):
            assert a1 == b0 and a0 < a1 <= steps[unit], (unit, ps)
        if len(ps) == 1:
            assert ps[0][2] == -1 and unit not in comb
        else:
            slot0, n = comb[unit]
            assert n == len(ps) and [p[2] for p in ps] == list(range(slot0, slot0 + n))
            if unit not in tail_units:
                assert len({p[3] for p in ps}) == n  # one part per workgroup
            slots_seen += [p[2] for p in ps]
    assert sorted(slots_seen) == list(range(plan["n_slots"]))
    assert abs(load.max() - plan["max_load"]) <= 1
    assert abs(load.sum() - plan["total_load"]) <= P
    # the per-XCD queues hold exactly the items of that XCD's workgroups
    # that are not in the shared tail (queue X); the queues hold every item
    assert len(qp) == X + 2 and qp[0] == 0 and qp[-1] == len(plan["items"])
    tail = plan["queue"][qp[X]:qp[X + 1]]
    assert sorted(plan["queue"]) == sorted(plan["items"])
    for x in range(X):
        mine = [it for i in range(x, P, X)
                for it in plan["items"][plan["item_ptr"][i]:plan["item_ptr"][i + 1]]
                if it[0] not in tail_units]
        assert sorted(plan["queue"][qp[x]:qp[x + 1]]) == sorted(mine), x
    # tail units are whole in the tail, and cut into parts of falling size
    assert not tail_units & {it[0] for it in plan["queue"][:qp[X]]}
    assert sum(1 for it in plan["queue"][qp[X]:qp[X + 1]] if it[3] >= 0) <= 3 * P
    return load


def main_like_steps():
    """Per-unit step counts of the main workload's 256x128 map (5 spatial,
    5 temporal heads), by interval arithmetic on the tile grid."""
    F, S, BQ, BK, CK, Wf, Ws = 21, 3600, 256, 128, 64, 4, 700
    N = F * S
    nq = -(-N // BQ)
    spatial, temporal = [], []
    for qt in range(nq):
        r0, r1 = qt * BQ, min(N, qt * BQ + BQ) - 1
        f0, f1 = r0 // S, r1 // S
        lo, hi = max(0, f0 - Wf) * S, min(F, f1 + Wf + 1) * S
        tiles = set(range(lo // BK, (hi - 1) // BK + 1)) | set(range(0, (S - 1) // BK + 1))
        spatial.append(2 * len(tiles))
        s0, s1 = r0 // F, r1 // F
        tlo = max(0, s0 - Ws) * F // BK
        thi = ((min(S - 1, s1 + Ws) + 1) * F - 1) // BK
        a = -(-(tlo * BK) // F)
        b = -(-min(N, (thi + 1) * BK) // F)
        temporal.append(2 * (thi - tlo + 1) + -(-a // CK) + -(-(S - b) // CK))
    return spatial * 5 + temporal * 5


@pytest.mark.parametrize("block,weighted,tail", [(16, False, 0.0), (0, False, 0.0),
                                                 (16, True, 0.0), (32, True, 0.05)])
def test_main_like_plan_is_exact_and_level(planner, block, weighted, tail):
    steps = main_like_steps()
    # spatial steps taking 3% longer than temporal ones
    weights = [1.03] * (len(steps) // 2) + [1.0] * (len(steps) // 2) if weighted else None
    plan = planner(steps, block=block, weights=weights, tail=tail)
    load = check_plan(steps, plan, 256, weights=weights)
    print(f"max/mean load {load.max() / load.mean():.4f}, {plan['n_slots']} partial slots, "
          f"{len(plan['combine'])} split units, {len(plan['items'])} items")
    # the busiest workgroup within 1% of the mean (whole-unit dealing: ~2.4%)
    assert load.max() / load.mean() < 1.01, load.max() / load.mean()
    assert plan["n_slots"] > 0


@pytest.mark.parametrize("seed", range(24))
def test_random_plans_cover_every_step_once(planner, seed):
    rng = np.random.default_rng(seed)
    n_wg = int(rng.choice([1, 3, 8, 13, 64, 256, 304]))
    n_xcd = int(rng.choice([1, 2, 8]))
    n = int(rng.choice([1, 2, 7, 40, 300, 2960]))
    steps = rng.integers(0, 700, size=n)
    steps[rng.random(n) < 0.05] = -1   # slices with no rows
    steps[rng.random(n) < 0.05] = 0
    overhead = int(rng.integers(0, 8))
    block = int(rng.choice([0, 1, 16]))
    weights = rng.uniform(0.5, 2.0, size=n) if seed % 2 else None
    plan = planner(steps, n_wg=n_wg, n_xcd=n_xcd, overhead=overhead,
                   min_part=int(rng.choice([1, 16, 32])), block=block, weights=weights,
                   tail=float(rng.choice([0.0, 0.05, 0.3, 1.0])))
    check_plan(list(steps), plan, n_wg, overhead=overhead, weights=weights)


def test_no_units_and_more_workgroups_than_steps(planner):
    plan = planner([-1, -1], n_wg=8)
    assert plan["items"] == [] and plan["n_slots"] == 0
    steps = [3]
    plan = planner(steps, n_wg=256, min_part=1)
    check_plan(steps, plan, 256)


def test_blocks_dealt_in_rounds_give_every_xcd_every_head(planner):
    steps = main_like_steps()
    plan = planner(steps, block=16)
    nq = len(steps) // 10
    for x in range(8):
        heads = set()
        for i in range(x, 256, 8):
            for unit, *_ in plan["items"][plan["item_ptr"][i]:plan["item_ptr"][i + 1]]:
                heads.add(unit // nq)
        assert heads == set(range(10)), (x, heads)


def test_shared_tail_parts_shrink_to_min_part(planner):
    """The main workload's plan with a 5% tail: the tail holds whole units
    only (no unit has parts both in an XCD queue and in the tail), its parts
    are queued longest first, and the last of them are about min_part steps
    long (raised a little to fit the slots): how level the workgroups end
    on the device."""
    steps = main_like_steps()
    plan = planner(steps, block=32, tail=0.05, min_part=32)
    check_plan(steps, plan, 256)
    qp = plan["queue_ptr"]
    tail = plan["queue"][qp[8]:qp[9]]
    lens = [(steps[u] if s1 == TO_END else s1) - s0 for u, s0, s1, _ in tail]
    work = sum(lens)
    assert 0.04 * sum(steps) < work <= 0.05 * sum(steps) + 4 * len(steps)
    assert 256 <= len(tail) <= 3 * 256
    assert lens == sorted(lens, reverse=True)
    assert all(32 <= n <= 48 for n in lens[-64:]), lens[-64:]
    assert max(lens[:32]) > 4 * max(lens[-64:])
    # without a tail every unit is in an XCD queue
    plan0 = planner(steps, block=32, tail=0.0)
    assert plan0["queue_ptr"][8] == plan0["queue_ptr"][9]


def test_tail_is_skipped_for_few_units(planner):
    steps = [100] * (4 * 16 - 1)
    plan = planner(steps, n_wg=16, n_xcd=2, tail=0.05)
    check_plan(steps, plan, 16)
    assert plan["queue_ptr"][2] == plan["queue_ptr"][3]
    steps = [100] * (4 * 16)
    plan = planner(steps, n_wg=16, n_xcd=2, tail=0.05)
    check_plan(steps, plan, 16)
    assert plan["queue_ptr"][3] > plan["queue_ptr"][2]


def test_tail_parts_fit_the_slots(planner):
    """A large tail share: min_part is raised until the parts fit the
    tail's 3 slots per workgroup, and the plan stays exact."""
    steps = main_like_steps()
    plan = planner(steps, block=32, tail=0.3, min_part=8)
    check_plan(steps, plan, 256)
    qp = plan["queue_ptr"]
    tail = plan["queue"][qp[8]:qp[9]]
    assert sum(1 for it in tail if it[3] >= 0) <= 3 * 256
