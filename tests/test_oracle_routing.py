"""Pins of the routing oracle (oracle/routing.py) to facts outside it.

* Brute force: pure-Python loops with both masks written out again from their
  definitions (|f - f'| <= W_f or f' = 0; |s - s'| <= W_s or f' = 0), softmax
  with math.exp, the squared error summed by hand.
* Closed form: with Q = 0 every kept key weighs the same, so with V equal to
  the frame-0 indicator each output is (kept frame-0 keys) / (kept keys).
* A mask that keeps every pair has error exactly 0.
* Planted heads: scores concentrated on a query's own frame route to the
  spatial mask, scores concentrated on its own raster index to the temporal
  mask (a swapped decision or a swapped pair of masks fails these).
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle import MaskParams, SPATIAL, TEMPORAL


def _brute_route(q, k, v, p: MaskParams, rows):
    S, N, d = p.S, p.N, q.shape[1]
    scale = 1.0 / math.sqrt(d)

    def out(t, keep):
        fq, sq = divmod(t, S)
        w, acc = [], [0.0] * d
        for u in range(N):
            fk, sk = divmod(u, S)
            if keep(fq, sq, fk, sk):
                sc = scale * sum(float(q[t, i]) * float(k[u, i]) for i in range(d))
                w.append((u, sc))
        mx = max(sc for _, sc in w)
        den = 0.0
        for u, sc in w:
            e = math.exp(sc - mx)
            den += e
            for i in range(d):
                acc[i] += e * float(v[u, i])
        return [a / den for a in acc]

    dense = lambda fq, sq, fk, sk: True
    spatial = lambda fq, sq, fk, sk: abs(fq - fk) <= p.frame_window or (p.sink and fk == 0)
    temporal = lambda fq, sq, fk, sk: abs(sq - sk) <= p.band or (p.sink and fk == 0)
    es = et = 0.0
    for t in rows:
        od, os_, ot = out(t, dense), out(t, spatial), out(t, temporal)
        es += sum((a - b) ** 2 for a, b in zip(os_, od))
        et += sum((a - b) ** 2 for a, b in zip(ot, od))
    n = len(rows) * d
    return es / n, et / n


@pytest.mark.parametrize("sink", [True, False])
@pytest.mark.parametrize("wf,ws", [(0, 1), (1, 0), (1, 2)])
def test_route_matches_brute_force(sink, wf, ws):
    p = MaskParams(4, 2, 3, wf, ws, sink)
    rng = np.random.default_rng(100 + 10 * wf + ws + (5 if sink else 0))
    q, k, v = (rng.standard_normal((p.N, 5)) for _ in range(3))
    rows = np.array([0, 3, 7, 11, 16, 23])
    r = oracle.route_head(q, k, v, p, rows)
    es, et = _brute_route(q, k, v, p, rows)
    assert r.err_spatial == pytest.approx(es, rel=1e-10, abs=1e-15)
    assert r.err_temporal == pytest.approx(et, rel=1e-10, abs=1e-15)
    assert r.kind == (SPATIAL if es <= et else TEMPORAL)


@pytest.mark.parametrize("sink", [True, False])
def test_route_zero_queries_closed_form(sink):
    F, Hh, Ww, d, wf, ws = 7, 3, 5, 4, 1, 2
    p = MaskParams(F, Hh, Ww, wf, ws, sink)
    S, N = p.S, p.N
    t = np.arange(N)
    v = np.repeat((t // S == 0).astype(float)[:, None], d, axis=1)
    q = np.zeros((N, d))
    k = np.random.default_rng(5).standard_normal((N, d))
    rows = np.arange(0, N, 4)
    r = oracle.route_head(q, k, v, p, rows)
    es = et = 0.0
    for x in rows:
        f, s = divmod(int(x), S)
        window = {g for g in range(F) if abs(g - f) <= wf}
        nb = sum(1 for u in range(S) if abs(u - s) <= ws)
        if sink:
            o_s = 1.0 / len(window | {0})
            o_t = S / (F * nb + (S - nb))
        else:
            o_s = (1.0 if 0 in window else 0.0) / len(window)
            o_t = 1.0 / F
        es += (o_s - 1.0 / F) ** 2
        et += (o_t - 1.0 / F) ** 2
    assert r.err_spatial == pytest.approx(es / len(rows), rel=1e-12, abs=1e-300)
    assert r.err_temporal == pytest.approx(et / len(rows), rel=1e-12, abs=1e-300)
    if not sink:
        assert r.err_temporal == pytest.approx(0.0, abs=1e-30)


def test_route_masks_that_keep_everything_have_zero_error():
    rng = np.random.default_rng(9)
    p = MaskParams(3, 2, 4, 2, 1, True)          # W_f >= F - 1: spatial keeps all
    q, k, v = (rng.standard_normal((p.N, 6)) for _ in range(3))
    r = oracle.route_head(q, k, v, p, np.arange(p.N))
    assert r.err_spatial == 0.0 and r.err_temporal > 0.0 and r.kind == SPATIAL
    p = MaskParams(3, 2, 4, 0, 7, False)         # W_s >= S - 1: temporal keeps all
    r = oracle.route_head(q, k, v, p, np.arange(p.N))
    assert r.err_temporal == 0.0 and r.err_spatial > 0.0 and r.kind == TEMPORAL


def _planted(p: MaskParams, code, d, alpha, seed):
    """Q, K whose scores are alpha * scale inside a code class, 0 outside."""
    t = np.arange(p.N)
    c = code(t)
    k = np.zeros((p.N, d))
    k[t, c] = 1.0
    q = alpha * k
    v = np.random.default_rng(seed).standard_normal((p.N, d))
    return q, k, v


def test_planted_heads_route_to_their_mask():
    p = MaskParams(6, 2, 3, 1, 0, True)          # S = 6, N = 36
    d = 8
    alpha = 30.0 * math.sqrt(d)                   # scores of 30 inside the class
    rows = np.arange(0, p.N, 3)
    q, k, v = _planted(p, lambda t: t // p.S, d, alpha, 1)   # same frame
    r = oracle.route_head(q, k, v, p, rows)
    assert r.kind == SPATIAL and r.err_spatial < 1e-9 < r.err_temporal
    q, k, v = _planted(p, lambda t: t % p.S, d, alpha, 2)    # same raster index
    r = oracle.route_head(q, k, v, p, rows)
    assert r.kind == TEMPORAL and r.err_temporal < 1e-9 < r.err_spatial
