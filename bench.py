"""Benchmark: structured-sparse video attention forward on one MI355X.

One step = one pass of the whole hot path over the main workload (75,600
tokens = 21 frames x 45x80 latents, 10 heads: 5 spatial + 5 temporal, d=128,
bf16, tiles 256x128, exact masks): rebuild the tile map in place (classify +
compact) and run the attention forward for all heads. Inputs are seeded
synthetic N(0,1) values already resident in HBM; temporal heads are put in
their kernel layout once, outside the timed region (the pages' kernel timings
exclude token permutation).

Prints one JSON line. `value` is effective TFLOP/s over retained pairs
(4 * d * retained pairs per step / step time). Alongside, under "extra": the
attention kernel alone (HIP events around each launch on the launch stream),
the tile-map build, the same-shape dense run through the same kernel, the
naive traversal (mask evaluated on every executed tile), the tile-aligned
variant, the 1440p workload (302,400 tokens), the token permutation of one
tensor (GB/s), a tile-size search (svg_autotune_tiles) over {128, 256, 512} x {64,
128, 256}, sampled head routing (svg_route_heads; not part of the step, as on
the pages) and a plain bf16 GEMM for reference; "cpu_baseline" times the float64
oracle on a bounded sample.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
                    [--no-extras] [--cpu-rows 12288] [--profile] [--copy-calibration]
                    [--routing-only] [--workload main|dense|tile-aligned|1440p]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense bf16 MFMA peak: 256 CU x 2.4 GHz x 4096 FLOP/clk (the published 2.5 PFLOP/s)
PEAK_BF16_TFLOPS = 2516.6
# the sources that decide the attention kernel's memory traffic: the kernel
# and the launch plan
TRAFFIC_SRC = [os.path.join(ROOT, "structured_sparse_attention_amd", "csrc", f)
               for f in ("attn_fwd.hip", "plan.cpp", "plan.hpp", "svg_internal.hpp", "svg_api.cpp")]
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_fwd_main_hbm_traffic.md")
METRIC = "sparse attn fwd ms + effective TFLOP/s (retained pairs) at 75,600 tok×10 heads×d128"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="main")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense, naive and tile-aligned runs")
    ap.add_argument("--cpu-rows", type=int, default=12288, help="oracle query rows per head")
    ap.add_argument("--profile", action="store_true",
                    help="the timed steps only, no extras and no CPU baseline (for rocprofv3)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--routing-only", action="store_true",
                    help="run only the sampled head routing on the main workload")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"copied {n} bytes x3")
    print(json.dumps({"copy_bytes": n, "copies": 3}))


def device_inputs(w):
    import torch
    import seeded_inputs as si
    from structured_sparse_attention_amd import svg_permute_tokens, TO_KERNEL_LAYOUT
    Q, K, V = si.draw_qkv(w)
    out = []
    for x in (Q, K, V):
        t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        y = torch.empty_like(t)
        svg_permute_tokens(t, y, w.frames, w.tokens_per_frame, w.head_kinds, TO_KERNEL_LAYOUT)
        out.append(y)
        del t
    torch.cuda.synchronize()
    return out, (Q, K, V)


def time_steps(w, q, k, v, o, steps, warmup, flags=0):
    """Time `steps` steps (map rebuild + attention) on the current stream.

    Returns (ms per step, attention-kernel ms list, map ms list, per-head
    stats, launch-plan statistics).
    """
    import torch
    import structured_sparse_attention_amd as svg
    tm = svg.svg_build_tile_map(
        w.frames, w.grid_h, w.grid_w, w.head_kinds, w.frame_window, w.band, w.sink,
        svg.ROUND_TILE if w.tile_aligned else svg.ROUND_EXACT, w.tile_q, w.tile_k)
    stats = tm.stats()
    plan = tm.plan_info()
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        tm.rebuild(stream)
        svg.svg_attn_fwd(q, k, v, o, w.head_kinds, tm, flags=flags, stream=stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        tm.rebuild(stream)
        ev[i][1].record(stream)
        svg.svg_attn_fwd(q, k, v, o, w.head_kinds, tm, flags=flags, stream=stream)
        ev[i][2].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    attn = [e[1].elapsed_time(e[2]) for e in ev]
    amap = [e[0].elapsed_time(e[1]) for e in ev]
    tm.destroy()
    return total / steps, attn, amap, stats, plan


# ------------------------------------------------------------------ CPU oracle

_POOL = {}


def _oracle_task(args):
    import oracle
    import seeded_inputs as si
    h, rows = args
    w, Q, K, V, masks = (_POOL[k] for k in ("w", "Q", "K", "V", "masks"))
    widen = lambda b: si.bf16_bits_to_f32(b).astype(np.float64)
    oracle.attention_rows(widen(Q[h]), widen(K[h]), widen(V[h]), masks[h], rows)
    return len(rows)


def cpu_baseline(w, Q, K, V, rows_per_head):
    """The oracle, as it stands, on a bounded sample of the same workload.

    Row blocks of 128 queries run in a process pool, one process per host core
    (capped at 16), each with single-threaded BLAS.
    """
    from multiprocessing import get_context
    import oracle
    params = oracle.MaskParams(w.frames, w.grid_h, w.grid_w, w.frame_window, w.band, w.sink)
    masks = [oracle.HeadMask(params, kd, w.tile_aligned, w.tile_q, w.tile_k)
             for kd in w.head_kinds]
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(w.seq_len, rows_per_head, replace=False))
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:
        limit = None
    _POOL.update(w=w, Q=Q, K=K, V=V, masks=masks)
    tasks = [(h, rows[i:i + 128]) for h in range(w.num_heads) for i in range(0, len(rows), 128)]
    pairs = sum(int(masks[h].original_block(rows, np.arange(w.seq_len)).sum())
                for h in range(w.num_heads))
    t = time.perf_counter()
    with get_context("fork").Pool(cores) as pool:
        done = sum(pool.map(_oracle_task, tasks))
    dt = time.perf_counter() - t
    assert done == rows_per_head * w.num_heads
    if limit is not None:
        limit.restore_original_limits()
    tflops = 4.0 * w.head_dim * pairs / dt / 1e12
    full_s = dt * w.seq_len / rows_per_head
    return {"value": tflops, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2),
            "full_workload_seconds_extrapolated": round(full_s, 1),
            "sample": f"a row sample, not the whole workload: {rows_per_head} of {w.seq_len} "
                      f"query rows per head x {w.num_heads} heads of the {w.name} workload, "
                      f"each against all {w.seq_len} keys (float64 explicit-mask attention, "
                      f"{pairs} retained pairs, {cores} processes with single-threaded BLAS); "
                      f"every row would take about {full_s:.0f} s at this rate"}


# ------------------------------------------------------------------ routing

def routing_times(w, host):
    """Wall time of svg_route_heads (synchronous: V^T, partial and combine
    kernels, copy-back; the untimed first call allocates the scratch that
    later calls reuse) on the original-order inputs, at 64 sampled rows and
    at 1% of the tokens."""
    import torch
    import seeded_inputs as si
    import structured_sparse_attention_amd as svg
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in host)
    out = {}
    for n in (64, w.seq_len // 100):
        rows = si.draw_query_subset(w, n, seed=77)
        call = lambda: svg.svg_route_heads(q, k, v, w.frames, w.grid_h, w.grid_w,
                                           w.frame_window, w.band, rows, sink_first_frame=w.sink)
        call()
        torch.cuda.synchronize()
        t = time.perf_counter()
        kinds, err = call()
        ms = (time.perf_counter() - t) * 1e3
        out[f"rows_{n}"] = {"ms": round(ms, 3), "kinds": kinds}
        log(f"[bench] routing {n} rows: {ms:.3f} ms, kinds {kinds}")
    del q, k, v
    return out


# ------------------------------------------------------------------ roofline

def gemm_reference(n=16384, reps=5):
    """TFLOP/s of a plain bf16 GEMM (torch.matmul, the vendor BLAS) on N(0,1)
    inputs: what the chip's MFMA pipes sustain on dense random data, at the
    clock it holds under that load. Context for `roofline.frac`, which is
    taken against the published peak at 2.4 GHz."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(11)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        c = a @ b
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return {"kind": f"torch.matmul bf16 {n}x{n}x{n}, N(0,1) inputs", "ms": round(ms, 4),
            "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)}


def heads_desc(w):
    """The workload's head kinds and mask parameters, for the config string."""
    n = {k: w.head_kinds.count(k) for k in ("spatial", "temporal", "dense")}
    parts = []
    if n["spatial"]:
        parts.append(f"{n['spatial']} spatial W_f={w.frame_window}")
    if n["temporal"]:
        parts.append(f"{n['temporal']} temporal W_s={w.band}")
    if n["dense"]:
        parts.append(f"{n['dense']} dense")
    return ", ".join(parts) + (", frame-0 sink" if w.sink and (n["spatial"] or n["temporal"])
                               else "")


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel and plan sources; else None."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    text = open(TRAFFIC_PROFILE).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9]+)", text)
    if not m or not b:
        return None
    h = hashlib.sha256()
    for f in TRAFFIC_SRC:
        h.update(open(f, "rb").read())
    return int(b.group(1)) if m.group(1) == h.hexdigest() else None


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): the path is measured "
              f"on one GPU's share at its real shape and has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        return copy_calibration()
    if a.routing_only:
        import seeded_inputs as si
        w = si.workload("main")
        print(json.dumps({"routing": routing_times(w, si.draw_qkv(w))}), flush=True)
        return
    import torch
    import seeded_inputs as si
    if a.profile:
        a.no_cpu_baseline, a.no_extras = True, True
    w = si.workload(a.workload)
    log(f"[bench] workload {w.name}: N={w.seq_len} H={w.num_heads} d={w.head_dim} "
        f"tiles {w.tile_q}x{w.tile_k}")
    (q, k, v), host = device_inputs(w)
    o = torch.empty_like(q)
    ms, attn, amap, stats, plan = time_steps(w, q, k, v, o, a.steps, a.warmup)
    pairs = sum(s["retained_pairs"] for s in stats)
    flop = 4.0 * w.head_dim * pairs
    value = flop / (ms * 1e-3) / 1e12
    attn_ms = float(np.mean(attn))
    achieved = flop / (attn_ms * 1e-3) / 1e12
    log(f"[bench] step {ms:.3f} ms (attention mean {attn_ms:.3f} / median "
        f"{np.median(attn):.3f} / min {min(attn):.3f} ms, map {np.mean(amap):.3f} ms), "
        f"{value:.1f} effective TFLOP/s")
    extra = {
        "attn_kernel_ms": {"mean": round(attn_ms, 4), "median": round(float(np.median(attn)), 4),
                           "min": round(min(attn), 4)},
        "launch_plan": dict(plan, busiest_over_mean=round(
            plan["max_load"] * plan["workgroups"] / max(1, plan["total_load"]), 4)),
        "tile_map_ms": round(float(np.mean(amap)), 4),
        "retained_pairs": pairs,
        "exec_tiles_full_boundary_sink": [sum(s["exec_full"] for s in stats),
                                          sum(s["exec_boundary"] for s in stats),
                                          sum(s["exec_sink"] for s in stats)],
        "logical_tiles_skip_full_boundary": [sum(s["skip"] for s in stats),
                                             sum(s["full"] for s in stats),
                                             sum(s["boundary"] for s in stats)],
    }
    if not a.no_extras and w.name == "main":
        import structured_sparse_attention_amd as svg
        n_extra = max(3, a.steps // 4)
        _, nattn, _, _, _ = time_steps(w, q, k, v, o, n_extra, 1, flags=svg.ATTN_MASK_ALL_TILES)
        extra["naive_mask_all_tiles_ms"] = round(float(np.mean(nattn)), 4)
        log(f"[bench] naive (mask every executed tile) {np.mean(nattn):.3f} ms")
        wt = si.workload("tile-aligned")
        _, tattn, _, tstats, _ = time_steps(wt, q, k, v, o, n_extra, 1)
        tpairs = sum(s["retained_pairs"] for s in tstats)
        extra["tile_aligned_ms"] = round(float(np.mean(tattn)), 4)
        extra["tile_aligned_pairs_drift"] = round(tpairs / pairs - 1.0, 5)
        extra["tile_aligned_tflops_rounded_mask"] = round(
            4.0 * w.head_dim * tpairs / (np.mean(tattn) * 1e-3) / 1e12, 1)
        extra["tile_aligned_tflops_exact_mask"] = round(
            4.0 * w.head_dim * pairs / (np.mean(tattn) * 1e-3) / 1e12, 1)
        log(f"[bench] tile-aligned {np.mean(tattn):.3f} ms (pairs {tpairs / pairs - 1:+.3%})")
        # token permutation (outside the step, as on the pages): all heads of
        # one tensor to the kernel layout; HBM-bound, bytes = 2 * H * N * d * 2
        stream = torch.cuda.current_stream()
        pev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        svg.svg_permute_tokens(q, o, w.frames, w.tokens_per_frame, w.head_kinds,
                               svg.TO_KERNEL_LAYOUT)
        pev[0].record(stream)
        for _ in range(10):
            svg.svg_permute_tokens(q, o, w.frames, w.tokens_per_frame, w.head_kinds,
                                   svg.TO_KERNEL_LAYOUT)
        pev[1].record(stream)
        torch.cuda.synchronize()
        pms = pev[0].elapsed_time(pev[1]) / 10
        pbytes = 2 * w.num_heads * w.seq_len * w.head_dim * 2
        extra["permute_tensor_ms"] = round(pms, 4)
        extra["permute_gbps"] = round(pbytes / (pms * 1e-3) / 1e9, 1)
        log(f"[bench] permute one tensor ({pbytes / 1e6:.0f} MB moved) {pms:.4f} ms, "
            f"{extra['permute_gbps']} GB/s")
        extra["routing"] = routing_times(w, host)
        cands = [(bq, bk) for bq in (128, 256, 512) for bk in (64, 128, 256)]
        best, cms = svg.svg_autotune_tiles(q, k, v, o, w.frames, w.grid_h, w.grid_w,
                                           w.head_kinds, w.frame_window, w.band, cands,
                                           sink_first_frame=w.sink, reps=3)
        extra["tile_search_exact"] = {"candidates": cands, "ms": [round(x, 4) for x in cms],
                                      "best": list(cands[best])}
        log(f"[bench] tile search: best {cands[best]} at {cms[best]:.3f} ms "
            f"({dict(zip(map(str, cands), [round(x, 3) for x in cms]))})")
        del q, k, v, o
        wd = si.workload("dense")
        (qd, kd, vd), _ = device_inputs(wd)
        od = torch.empty_like(qd)
        dms, dattn, _, dstats, _ = time_steps(wd, qd, kd, vd, od, n_extra, 1)
        dpairs = sum(s["retained_pairs"] for s in dstats)
        extra["dense_attn_kernel_ms"] = round(float(np.mean(dattn)), 4)
        extra["dense_tflops"] = round(4.0 * wd.head_dim * dpairs
                                      / (np.mean(dattn) * 1e-3) / 1e12, 1)
        extra["speedup_vs_dense"] = round(float(np.mean(dattn)) / attn_ms, 3)
        log(f"[bench] dense {np.mean(dattn):.3f} ms -> sparse speed-up "
            f"{np.mean(dattn) / attn_ms:.2f}x")
        del qd, kd, vd, od
        wl = si.workload("1440p")
        (ql, kl, vl), _ = device_inputs(wl)
        ol = torch.empty_like(ql)
        _, lattn, lmap, lstats, _ = time_steps(wl, ql, kl, vl, ol, 3, 1)
        lpairs = sum(s["retained_pairs"] for s in lstats)
        extra["1440p_attn_kernel_ms"] = round(float(np.mean(lattn)), 3)
        extra["1440p_tile_map_ms"] = round(float(np.mean(lmap)), 4)
        extra["1440p_tflops"] = round(4.0 * wl.head_dim * lpairs
                                      / (np.mean(lattn) * 1e-3) / 1e12, 1)
        log(f"[bench] 1440p (N={wl.seq_len}) {np.mean(lattn):.3f} ms, "
            f"{extra['1440p_tflops']} effective TFLOP/s")
        del ql, kl, vl, ol
        gref = gemm_reference()
        gref["attn_achieved_over_gemm"] = round(achieved / gref["tflops"], 3)
        extra["dense_gemm_reference"] = gref
        log(f"[bench] reference GEMM {gref}")
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: F={w.frames} {w.grid_h}x{w.grid_w} "
                               f"N={w.seq_len} H={w.num_heads} ({heads_desc(w)}) d={w.head_dim} "
                               f"tiles {w.tile_q}x{w.tile_k} "
                               f"{'tile-aligned' if w.tile_aligned else 'exact'}",
                   "global_batch": 1, "seq_len": w.seq_len, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic() if w.name == "main" else None},
        "extra": extra,
    }
    if not a.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(w, *host, a.cpu_rows)
        log(f"[bench] cpu baseline {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
