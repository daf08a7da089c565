// Host side of the C ABI: argument validation, tile-map lifecycle, kernel
// dispatch and error reporting. Every entry point validates its arguments
// before the first HIP call and reports failures as svg_status values with a
// thread-local message; nothing throws across the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <stdexcept>
#include <string>
#include <vector>

#include "plan.hpp"
#include "svg_internal.hpp"

namespace {

thread_local std::string g_last_error;

svg_status fail(svg_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

svg_status ok() {
  g_last_error.clear();
  return SVG_OK;
}

svg_status hip_fail(hipError_t e, const char* what) {
  return fail(SVG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool tile_q_ok(int32_t bq) {
  return bq == 32 || bq == 64 || bq == 128 || (bq >= 256 && bq <= (1 << 20) && bq % 256 == 0);
}
bool tile_k_ok(int32_t bk) { return bk >= 32 && bk <= 1024 && bk % 32 == 0; }

void free_buffers(svg::MapBuffers& b) {
  void* ptrs[] = {b.kinds, b.classes, b.rowinfo, b.entries, b.rowstats};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  b = svg::MapBuffers{};
}

void free_plan(svg_tile_map* m) {
  void* dev[] = {m->plan.dev, m->plan.counters, m->plan.part_o, m->plan.part_ml};
  for (void* p : dev)
    if (p) (void)hipFree(p);
  if (m->job.rowinfo_host) (void)hipHostFree(m->job.rowinfo_host);
  if (m->job.image_host) (void)hipHostFree(m->job.image_host);
  m->plan = svg::PlanBuffers{};
  m->job.rowinfo_host = m->job.image_host = nullptr;
}

// Everything a map owns; the caller has waited for its queued work.
void free_map(svg_tile_map* m) {
  if (m->built) (void)hipEventDestroy(m->built);
  if (m->used) (void)hipEventDestroy(m->used);
  free_plan(m);
  free_buffers(m->buf);
  delete m;
}

// Step count of every work unit (a workgroup's slice of a schedule row, -1
// for a slice past the end of the sequence) from the map's row info.
void unit_steps(const PlanJob& j, std::vector<int32_t>& steps) {
  const svg::MapGeometry& g = j.geom;
  const int64_t R = (int64_t)g.H * g.nQ;
  const int32_t ck = svg::kAttnStepKeys, cpt = (g.BK + ck - 1) / ck;
  steps.resize(R * j.nsub);
  for (int64_t r = 0; r < R; ++r) {
    const int32_t* ri = j.rowinfo_host + r * svg::kRowInfo;
    const int64_t n = (int64_t)(ri[0] + ri[1]) * cpt + (ri[2] + ck - 1) / ck +
                      (g.S - ri[3] + ck - 1) / ck;
    const int64_t q0 = (r % g.nQ) * (int64_t)g.BQ;
    for (int32_t sub = 0; sub < j.nsub; ++sub)
      steps[r * j.nsub + sub] = q0 + (int64_t)sub * j.wgq < g.N ? (int32_t)n : -1;
  }
}

// Host function queued on the build stream once the row info has reached
// the pinned staging: plans the persistent launch and writes the plan image
// that the stream copies to the device next. It makes no HIP call. Should
// planning fail (host memory), every unit becomes one whole item of
// workgroup (unit mod workgroups), written without allocating.
void plan_host_fn(void* user) {
  PlanJob& j = *static_cast<PlanJob*>(user);
  svg::PlanBuffers& pl = *j.plan;
  const svg::MapGeometry& g = j.geom;
  int32_t* im = j.image_host;
  int32_t* ptr = im + 4;
  svg::ItemDesc* items = reinterpret_cast<svg::ItemDesc*>(im + pl.items_off());
  int32_t* comb = im + pl.combine_off();
  // Each row's first schedule entry (row r's entries start at r * nK) into
  // the row info's unused field 6 (staging only; the device copy is not
  // touched). R * nK fits int32: the build checks the capacity.
  const int64_t R = (int64_t)g.H * g.nQ;
  for (int64_t r = 0; r < R; ++r) j.rowinfo_host[r * svg::kRowInfo + 6] = (int32_t)(r * g.nK);
  auto desc = [&](int32_t unit, int32_t s0, int32_t s1, int32_t slot) {
    const int32_t row = unit / j.nsub, sub = unit - row * j.nsub;
    const int32_t* ri = j.rowinfo_host + (int64_t)row * svg::kRowInfo;
    const int32_t h = row / g.nQ, qt = row - h * g.nQ;
    return svg::ItemDesc{unit,  s0,    s1, slot, ri[0], ri[0] + ri[1], ri[6], ri[2],
                         ri[3], h, qt * g.BQ + sub * j.wgq, j.kinds[h]};
  };
  try {
    std::vector<int32_t> steps;
    unit_steps(j, steps);
    std::vector<float> weight(steps.size());
    for (size_t u = 0; u < steps.size(); ++u)
      weight[u] = svg::kPlanStepWeight[j.kinds[(u / j.nsub) / g.nQ]];
    svg::PlanResult r;
    svg::plan_persistent(steps.data(), weight.data(), (int32_t)steps.size(), pl.n_wg, pl.n_xcd,
                         svg::kPlanBlockUnits, svg::kPlanItemOverhead, svg::kPlanMinPart,
                         svg::kPlanTail, r);
    // (the staging holds the bounds the plan keeps; a plan past them would
    // be a planner fault, and falls back to the plan below)
    if ((int64_t)r.queue_items.size() > pl.max_items || r.n_slots > pl.max_slots ||
        (int64_t)r.combine.size() > pl.max_combine ||
        (int64_t)r.queue_ptr.size() != pl.n_xcd + 2)
      throw std::length_error("launch plan past its bounds");
    im[0] = (int32_t)r.items.size();
    im[1] = (int32_t)r.combine.size();
    im[2] = r.n_slots;
    im[3] = 0;
    std::memcpy(ptr, r.queue_ptr.data(), r.queue_ptr.size() * sizeof(int32_t));
    for (size_t i = 0; i < r.queue_items.size(); ++i) {
      const svg::PlanItem& it = r.queue_items[i];
      items[i] = desc(it.unit, it.s0, it.s1, it.slot);
    }
    std::memcpy(comb, r.combine.data(), r.combine.size() * sizeof(svg::PlanCombine));
    j.items = (int64_t)r.items.size();
    j.split_units = (int64_t)r.combine.size();
    j.slots = r.n_slots;
    j.max_load = r.max_load;
    j.total_load = r.total_load;
  } catch (...) {
    // every unit whole, in order, XCD x taking units x, x + n_xcd, ...
    const int64_t n_units = R * j.nsub;
    int32_t n = 0;
    for (int32_t x = 0; x < pl.n_xcd; ++x) {
      ptr[x] = n;
      for (int64_t u = x; u < n_units; u += pl.n_xcd)
        if (((u / j.nsub) % g.nQ) * (int64_t)g.BQ + (u % j.nsub) * (int64_t)j.wgq < g.N)
          items[n++] = desc((int32_t)u, 0, svg::kPlanToEnd, -1);
    }
    ptr[pl.n_xcd] = ptr[pl.n_xcd + 1] = n;  // an empty shared tail
    im[0] = n;
    im[1] = im[2] = im[3] = 0;
    j.items = n;
    j.split_units = j.slots = j.max_load = j.total_load = 0;
  }
}

template <typename T>
hipError_t alloc(T** p, size_t count) {
  return hipMalloc(reinterpret_cast<void**>(p), count * sizeof(T) + 16);
}

svg_status wait_built(const svg_tile_map* m) {
  if (m->built) {
    const hipError_t e = hipEventSynchronize(m->built);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  }
  return SVG_OK;
}

// The map's buffers live on the device it was built on; its kernels must run
// there.
svg_status check_device(const svg_tile_map* m) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != m->device)
    return fail(SVG_ERR_INVALID_ARG, "the map was built on device %d, the current device is %d",
                m->device, dev);
  return SVG_OK;
}

// Uses of one map are ordered on the device, since they share its workspace
// (schedule, plan, partial results): on `st`, without blocking the host, wait
// for the map's last build and, unless `after_build_only`, its last attention
// launch. Under stream capture nothing is waited for (an event recorded
// outside a capture cannot be waited for inside it): the caller orders them.
hipError_t order_after(const svg_tile_map* m, hipStream_t st, bool after_build_only,
                       bool& capturing) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return e;
  capturing = cs != hipStreamCaptureStatusNone;
  if (capturing) return hipSuccess;
  if (!after_build_only && m->used_valid) e = hipStreamWaitEvent(st, m->used, 0);
  if (e == hipSuccess && m->built) e = hipStreamWaitEvent(st, m->built, 0);
  return e;
}

svg_status run_build(svg_tile_map* m, hipStream_t stream) {
  hipError_t e = svg::launch_build_tile_map(m->geom, m->buf, stream);
  if (e != hipSuccess) return hip_fail(e, "tile-map kernels");
  e = hipEventRecord(m->built, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  return ok();
}

// Arguments of a routing call after validation: N, S and the windows
// clamped to the sequence.
struct RouteArgs {
  int64_t N = 0;
  int32_t S = 0, W_f = 0, W_s = 0;
};

svg_status route_validate(const svg_mask_spec* spec, const void* q, const void* k, const void* v,
                          int32_t head_dim, float scale, const int32_t* rows, int32_t n_rows,
                          const int32_t* kinds, RouteArgs& out) {
  if (!spec) return fail(SVG_ERR_INVALID_ARG, "spec is NULL");
  if (!q || !k || !v) return fail(SVG_ERR_INVALID_ARG, "q, k and v must be non-NULL");
  if (!rows || !kinds) return fail(SVG_ERR_INVALID_ARG, "rows and kinds must be non-NULL");
  if (spec->frames < 1 || spec->grid_h < 1 || spec->grid_w < 1)
    return fail(SVG_ERR_INVALID_ARG, "frames, grid_h and grid_w must be >= 1");
  const int64_t S = (int64_t)spec->grid_h * spec->grid_w;
  const int64_t N = S * spec->frames;
  if (S > (1 << 30) || N > (1 << 30))
    return fail(SVG_ERR_INVALID_ARG, "sequence of %lld tokens exceeds 2^30", (long long)N);
  if (spec->num_heads < 1 || spec->num_heads > 4096)
    return fail(SVG_ERR_INVALID_ARG, "num_heads %d outside [1, 4096]", spec->num_heads);
  if (spec->frame_window < 0 || spec->temporal_band < 0)
    return fail(SVG_ERR_INVALID_ARG, "frame_window and temporal_band must be >= 0");
  if (n_rows < 1 || n_rows > 65536)
    return fail(SVG_ERR_INVALID_ARG, "n_rows %d outside [1, 65536]", n_rows);
  for (int32_t i = 0; i < n_rows; ++i)
    if (rows[i] < 0 || rows[i] >= N)
      return fail(SVG_ERR_INVALID_ARG, "rows[%d] = %d outside [0, %lld)", i, rows[i],
                  (long long)N);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(SVG_ERR_INVALID_ARG, "scale must be positive and finite");
  if (head_dim != 64 && head_dim != 128)
    return fail(SVG_ERR_UNSUPPORTED, "head_dim %d: supported are 64 and 128", head_dim);
  if (N * head_dim * 2 >= ((int64_t)1 << 31))
    return fail(SVG_ERR_UNSUPPORTED, "one head of %lld x %d bf16 values exceeds 2 GiB",
                (long long)N, head_dim);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(SVG_ERR_ALIGNMENT, "q, k and v must be 16-byte aligned");
  out.N = N;
  out.S = (int32_t)S;
  // Windows wider than the sequence behave like the sequence (as in
  // svg_build_tile_map); clamping keeps the kernels' interval arithmetic in
  // 32-bit range.
  out.W_f = spec->frame_window < spec->frames ? spec->frame_window : spec->frames;
  out.W_s = spec->temporal_band < S ? spec->temporal_band : (int32_t)S;
  return SVG_OK;
}

// The sampled rows in the order the routing kernels take them: by raster
// index (then by token), so that the 16 rows of a wave have neighbouring
// temporal bands. A row's result does not depend on its place; only the
// order of the float64 sum of row errors does.
void order_rows(const int32_t* rows, int32_t n, int32_t S, int32_t* out) {
  std::memcpy(out, rows, (size_t)n * 4);
  std::sort(out, out + n, [S](int32_t a, int32_t b) {
    const int32_t sa = a % S, sb = b % S;
    return sa != sb ? sa < sb : a < b;
  });
}

// Host staging of the ordered rows for svg_route_heads_noalloc; the lock
// also serialises that call's use of the device scratch within a process.
std::mutex g_noalloc_mu;
int32_t g_noalloc_rows[65536];

// svg_route_heads keeps its scratch between calls, per device (the largest
// so far): allocating and freeing a few hundred MB took about half of a
// call's time. The calls are synchronous and hold the lock throughout, so
// a scratch is never in use when it is replaced.
std::mutex g_route_mu;
struct RouteScratch {
  char* p = nullptr;
  int64_t bytes = 0;
};
std::vector<RouteScratch> g_route_scratch;  // by device

}  // namespace

extern "C" {

const char* svg_last_error(void) { return g_last_error.c_str(); }

int32_t svg_abi_version(void) { return SVG_ABI_VERSION; }

svg_status svg_build_tile_map(const svg_mask_spec* spec, int32_t tile_q, int32_t tile_k,
                              void* stream, svg_tile_map** out) {
  if (!spec) return fail(SVG_ERR_INVALID_ARG, "spec is NULL");
  if (!out) return fail(SVG_ERR_INVALID_ARG, "out is NULL");
  if (!spec->head_kind) return fail(SVG_ERR_INVALID_ARG, "spec->head_kind is NULL");
  if (spec->frames < 1 || spec->grid_h < 1 || spec->grid_w < 1)
    return fail(SVG_ERR_INVALID_ARG, "frames, grid_h and grid_w must be >= 1");
  const int64_t S = (int64_t)spec->grid_h * spec->grid_w;
  const int64_t N = S * spec->frames;
  if (S > (1 << 30) || N > (1 << 30))
    return fail(SVG_ERR_INVALID_ARG, "sequence of %lld tokens exceeds 2^30", (long long)N);
  if (spec->num_heads < 1 || spec->num_heads > 4096)
    return fail(SVG_ERR_INVALID_ARG, "num_heads %d outside [1, 4096]", spec->num_heads);
  if (spec->frame_window < 0 || spec->temporal_band < 0)
    return fail(SVG_ERR_INVALID_ARG, "frame_window and temporal_band must be >= 0");
  if (spec->round_mode != SVG_ROUND_EXACT && spec->round_mode != SVG_ROUND_TILE)
    return fail(SVG_ERR_INVALID_ARG, "round_mode %d is not an svg_round_mode", spec->round_mode);
  for (int32_t h = 0; h < spec->num_heads; ++h) {
    const int32_t k = spec->head_kind[h];
    if (k != SVG_HEAD_SPATIAL && k != SVG_HEAD_TEMPORAL && k != SVG_HEAD_DENSE)
      return fail(SVG_ERR_INVALID_ARG, "head_kind[%d] = %d is not an svg_head_kind", h, k);
  }
  if (!tile_q_ok(tile_q))
    return fail(SVG_ERR_UNSUPPORTED, "tile_q %d: supported are 32, 64, 128 and multiples of 256",
                tile_q);
  if (!tile_k_ok(tile_k))
    return fail(SVG_ERR_UNSUPPORTED, "tile_k %d: supported are multiples of 32 in [32, 1024]",
                tile_k);

  svg_tile_map* m = new (std::nothrow) svg_tile_map();
  if (!m) return fail(SVG_ERR_OOM, "host allocation of the map failed");
  svg::MapGeometry& g = m->geom;
  g.N = N;
  g.F = spec->frames;
  g.S = (int32_t)S;
  g.H = spec->num_heads;
  // Windows wider than the sequence behave like the sequence; clamping keeps
  // every product in range.
  g.W_f = spec->frame_window < spec->frames ? spec->frame_window : spec->frames;
  g.W_s = spec->temporal_band < g.S ? spec->temporal_band : g.S;
  g.sink = spec->sink_first_frame ? 1 : 0;
  g.round = spec->round_mode;
  g.BQ = tile_q;
  g.BK = tile_k;
  g.nQ = (int32_t)((N + tile_q - 1) / tile_q);
  g.nK = (int32_t)((N + tile_k - 1) / tile_k);
  m->kinds.assign(spec->head_kind, spec->head_kind + spec->num_heads);

  hipError_t e = hipGetDevice(&m->device);
  if (e != hipSuccess) {
    delete m;
    return hip_fail(e, "hipGetDevice");
  }
  const int64_t R = (int64_t)g.H * g.nQ;
  svg::MapBuffers& b = m->buf;
  b.capacity = R * g.nK;
  if (b.capacity > INT32_MAX) {
    delete m;
    return fail(SVG_ERR_UNSUPPORTED, "schedule of %lld entries exceeds int32 indexing",
                (long long)b.capacity);
  }
  // The persistent launch: one workgroup per compute unit, workgroup i on
  // XCD i mod (XCD count).
  svg::PlanBuffers& pl = m->plan;
  PlanJob& job = m->job;
  job.geom = g;
  job.kinds = m->kinds.data();
  job.wgq = svg::attn_waves(tile_q) * svg::kAttnQRowsPerWave;
  job.nsub = tile_q / job.wgq;
  job.plan = &pl;
  {
    int cus = 0, xcds = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, m->device);
    if (e == hipSuccess && hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs,
                                                 m->device) != hipSuccess)
      xcds = 1;
    if (e != hipSuccess || cus < 1) {
      delete m;
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidDevice, "compute unit count");
    }
    pl.n_wg = cus;
    pl.n_xcd = xcds >= 1 && xcds <= cus ? xcds : 1;
  }
  const int64_t n_units = R * job.nsub;
  if (svg::plan_max_items(n_units, pl.n_wg) > INT32_MAX / 4) {
    delete m;
    return fail(SVG_ERR_UNSUPPORTED, "%lld work units exceed the launch plan's indexing",
                (long long)n_units);
  }
  pl.max_items = svg::plan_max_items(n_units, pl.n_wg);
  pl.max_slots = svg::plan_max_slots(pl.n_wg);
  pl.max_combine = svg::plan_max_combine(pl.n_wg);
  const int64_t part_rows = pl.max_slots * job.wgq;
  hipError_t ea = hipSuccess;
  auto step = [&](hipError_t x) { if (ea == hipSuccess) ea = x; };
  step(alloc(&b.kinds, g.H));
  step(alloc(&b.classes, R * g.nK));
  step(alloc(&b.rowinfo, R * svg::kRowInfo));
  step(alloc(&b.entries, b.capacity));
  step(alloc(&b.rowstats, R * svg::kRowStats));
  step(alloc(&pl.dev, pl.dev_ints()));
  step(alloc(&pl.counters, (int64_t)svg::kQueueRing * (pl.n_xcd + 1)));
  step(alloc(&pl.part_o, part_rows * svg::kAttnMaxHeadDim));
  step(alloc(&pl.part_ml, part_rows * 2));
  if (ea == hipSuccess)
    ea = hipHostMalloc(reinterpret_cast<void**>(&job.rowinfo_host),
                       (size_t)R * svg::kRowInfo * sizeof(int32_t), hipHostMallocDefault);
  if (ea == hipSuccess)
    ea = hipHostMalloc(reinterpret_cast<void**>(&job.image_host),
                       (size_t)pl.dev_ints() * sizeof(int32_t), hipHostMallocDefault);
  if (ea != hipSuccess) {
    free_map(m);
    return fail(ea == hipErrorOutOfMemory ? SVG_ERR_OOM : SVG_ERR_HIP,
                "allocation for the tile map failed: %s", hipGetErrorString(ea));
  }
  // An all-zero image is a valid empty plan (no items, no combine entries).
  std::memset(job.image_host, 0, (size_t)pl.dev_ints() * sizeof(int32_t));
  if ((e = hipEventCreateWithFlags(&m->built, hipEventDisableTiming)) != hipSuccess) {
    m->built = nullptr;
    free_map(m);
    return hip_fail(e, "hipEventCreate");
  }
  if ((e = hipEventCreateWithFlags(&m->used, hipEventDisableTiming)) != hipSuccess) {
    m->used = nullptr;
    free_map(m);
    return hip_fail(e, "hipEventCreate");
  }
  // Queued on the caller's stream, nothing waited for: head kinds from
  // kernel arguments, the tile-map kernels, the row info to the pinned
  // staging, the planning host function, the plan image to the device.
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const char* what = "copy of head kinds";
  e = svg::launch_set_kinds(m->kinds.data(), g.H, b.kinds, st);
  if (e == hipSuccess) {
    what = "tile-map kernels";
    e = svg::launch_build_tile_map(g, b, st);
  }
  if (e == hipSuccess) {
    what = "copy of row info";
    e = hipMemcpyAsync(job.rowinfo_host, b.rowinfo, (size_t)R * svg::kRowInfo * sizeof(int32_t),
                       hipMemcpyDeviceToHost, st);
  }
  if (e == hipSuccess) {
    what = "launch planning";
    e = hipLaunchHostFunc(st, plan_host_fn, &job);
  }
  if (e == hipSuccess) {
    what = "copy of the launch plan";
    e = hipMemcpyAsync(pl.dev, job.image_host, (size_t)pl.dev_ints() * sizeof(int32_t),
                       hipMemcpyHostToDevice, st);
  }
  if (e == hipSuccess) {
    what = "hipEventRecord";
    e = hipEventRecord(m->built, st);
  }
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(st);
    free_map(m);
    return hip_fail(e, what);
  }
  *out = m;
  return ok();
}

svg_status svg_tile_map_rebuild(svg_tile_map* map, void* stream) {
  if (!map) return fail(SVG_ERR_INVALID_ARG, "map is NULL");
  const svg_status s = check_device(map);
  if (s != SVG_OK) return s;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(map->mu);
  hipError_t e = hipSuccess;
  if (map->used_valid) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(st, &cs);
    if (e == hipSuccess && cs == hipStreamCaptureStatusNone)
      e = hipStreamWaitEvent(st, map->used, 0);
  }
  if (e != hipSuccess) return hip_fail(e, "ordering after the map's last attention launch");
  return run_build(map, st);
}

svg_status svg_tile_map_info_get(const svg_tile_map* map, svg_tile_map_info* out) {
  if (!map || !out) return fail(SVG_ERR_INVALID_ARG, "map or out is NULL");
  const svg::MapGeometry& g = map->geom;
  out->seq_len = g.N;
  out->num_heads = g.H;
  out->tile_q = g.BQ;
  out->tile_k = g.BK;
  out->num_q_tiles = g.nQ;
  out->num_k_tiles = g.nK;
  out->frames = g.F;
  out->tokens_per_frame = g.S;
  out->entry_capacity = map->buf.capacity;
  return ok();
}

svg_status svg_tile_map_stats(const svg_tile_map* map, svg_head_stats* per_head,
                              int32_t num_heads) {
  if (!map || !per_head) return fail(SVG_ERR_INVALID_ARG, "map or per_head is NULL");
  if (num_heads != map->geom.H)
    return fail(SVG_ERR_SHAPE_MISMATCH, "num_heads %d, map has %d", num_heads, map->geom.H);
  svg_status s = wait_built(map);
  if (s != SVG_OK) return s;
  // the per-row statistics, summed per head here
  const svg::MapGeometry& g = map->geom;
  std::vector<int64_t> rows((size_t)num_heads * g.nQ * svg::kRowStats);
  const hipError_t e = hipMemcpy(rows.data(), map->buf.rowstats, rows.size() * sizeof(int64_t),
                                 hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "copy of tile-map stats");
  for (int32_t h = 0; h < num_heads; ++h) {
    int64_t a[svg::kRowStats] = {};
    for (int64_t qt = 0; qt < g.nQ; ++qt) {
      const int64_t* r = rows.data() + ((size_t)h * g.nQ + qt) * svg::kRowStats;
      for (int i = 0; i < svg::kRowStats; ++i) a[i] += r[i];
    }
    per_head[h] = svg_head_stats{a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7]};
  }
  return ok();
}

svg_status svg_tile_map_copy_classes(const svg_tile_map* map, uint8_t* host, size_t n) {
  if (!map || !host) return fail(SVG_ERR_INVALID_ARG, "map or host is NULL");
  const svg::MapGeometry& g = map->geom;
  const size_t want = (size_t)g.H * g.nQ * g.nK;
  if (n != want) return fail(SVG_ERR_SHAPE_MISMATCH, "n = %zu, class map has %zu bytes", n, want);
  svg_status s = wait_built(map);
  if (s != SVG_OK) return s;
  const hipError_t e = hipMemcpy(host, map->buf.classes, want, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "copy of class map");
  return ok();
}

svg_status svg_tile_map_copy_schedule(const svg_tile_map* map, int32_t* row_ptr,
                                      int32_t* n_full, int32_t* sink_ab, int32_t* entries,
                                      size_t n_entries) {
  if (!map) return fail(SVG_ERR_INVALID_ARG, "map is NULL");
  svg_status s = wait_built(map);
  if (s != SVG_OK) return s;
  const svg::MapGeometry& g = map->geom;
  const size_t R = (size_t)g.H * g.nQ;
  // row r's executed tiles are its FULL and BOUNDARY counts (row info 0, 1);
  // on the device its entries start at r * nK, packed here
  std::vector<int32_t> ri(R * svg::kRowInfo);
  hipError_t e = hipMemcpy(ri.data(), map->buf.rowinfo, ri.size() * sizeof(int32_t),
                           hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "copy of row info");
  std::vector<int32_t> rp(R + 1, 0);
  for (size_t r = 0; r < R; ++r)
    rp[r + 1] = rp[r] + ri[r * svg::kRowInfo + 0] + ri[r * svg::kRowInfo + 1];
  if (entries && n_entries < (size_t)rp[R])
    return fail(SVG_ERR_SHAPE_MISMATCH, "n_entries = %zu, schedule has %d entries", n_entries,
                rp[R]);
  if (row_ptr) std::memcpy(row_ptr, rp.data(), (R + 1) * sizeof(int32_t));
  for (size_t r = 0; r < R; ++r) {
    if (n_full) n_full[r] = ri[r * svg::kRowInfo + 0];
    if (sink_ab) {
      sink_ab[2 * r] = ri[r * svg::kRowInfo + 2];
      sink_ab[2 * r + 1] = ri[r * svg::kRowInfo + 3];
    }
  }
  if (entries && rp[R] > 0) {
    std::vector<int32_t> all(R * (size_t)g.nK);
    e = hipMemcpy(all.data(), map->buf.entries, all.size() * sizeof(int32_t),
                  hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "copy of schedule entries");
    for (size_t r = 0; r < R; ++r)
      std::memcpy(entries + rp[r], all.data() + r * g.nK, (size_t)(rp[r + 1] - rp[r]) * 4);
  }
  return ok();
}

svg_status svg_tile_map_plan_info(const svg_tile_map* map, svg_plan_info* out) {
  if (!map || !out) return fail(SVG_ERR_INVALID_ARG, "map or out is NULL");
  svg_status s = wait_built(map);
  if (s != SVG_OK) return s;
  out->workgroups = map->plan.n_wg;
  out->xcds = map->plan.n_xcd;
  out->work_items = map->job.items;
  out->split_rows = map->job.split_units;
  out->partial_slots = map->job.slots;
  out->max_load = map->job.max_load;
  out->total_load = map->job.total_load;
  return ok();
}

svg_status svg_tile_map_destroy(svg_tile_map* map) {
  if (!map) return ok();
  svg_status s = wait_built(map);
  if (s == SVG_OK && map->used_valid) {
    // the last attention launch that used the map, on whatever stream
    const hipError_t e = hipEventSynchronize(map->used);
    if (e != hipSuccess) s = hip_fail(e, "hipEventSynchronize");
  }
  free_map(map);
  return s == SVG_OK ? ok() : s;
}

svg_status svg_attn_fwd(const void* q, const void* k, const void* v, void* o, int64_t seq_len,
                        int32_t num_heads, int32_t head_dim, float scale,
                        const int32_t* head_kind, const svg_tile_map* map, uint32_t flags,
                        void* stream) {
  if (!q || !k || !v || !o) return fail(SVG_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (!map) return fail(SVG_ERR_INVALID_ARG, "map is NULL");
  if (!head_kind) return fail(SVG_ERR_INVALID_ARG, "head_kind is NULL");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(SVG_ERR_INVALID_ARG, "scale must be positive and finite");
  if (flags & ~(uint32_t)SVG_ATTN_MASK_ALL_TILES)
    return fail(SVG_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const svg::MapGeometry& g = map->geom;
  if (seq_len != g.N)
    return fail(SVG_ERR_SHAPE_MISMATCH, "seq_len %lld, map has %lld", (long long)seq_len,
                (long long)g.N);
  if (num_heads != g.H)
    return fail(SVG_ERR_SHAPE_MISMATCH, "num_heads %d, map has %d", num_heads, g.H);
  for (int32_t h = 0; h < num_heads; ++h)
    if (head_kind[h] != map->kinds[h])
      return fail(SVG_ERR_SHAPE_MISMATCH, "head_kind[%d] = %d, map was built with %d", h,
                  head_kind[h], map->kinds[h]);
  if (seq_len * head_dim * 2 >= ((int64_t)1 << 31))
    return fail(SVG_ERR_UNSUPPORTED, "one head of %lld x %d bf16 values exceeds 2 GiB",
                (long long)seq_len, head_dim);
  if (!svg::attn_supported(head_dim, g.BQ, g.BK))
    return fail(SVG_ERR_UNSUPPORTED, "head_dim %d with tiles %dx%d has no kernel", head_dim,
                g.BQ, g.BK);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SVG_ERR_ALIGNMENT, "q, k, v and o must be 16-byte aligned");
  const uintptr_t bytes = (uintptr_t)num_heads * (uintptr_t)seq_len * head_dim * 2;
  const uintptr_t ob = reinterpret_cast<uintptr_t>(o);
  for (const void* in : {q, k, v}) {
    const uintptr_t ib = reinterpret_cast<uintptr_t>(in);
    if (ob < ib + bytes && ib < ob + bytes)
      return fail(SVG_ERR_INVALID_ARG, "o overlaps an input");
  }
  const svg_status ds = check_device(map);
  if (ds != SVG_OK) return ds;
  svg::AttnArgs a{q, k, v, o, head_dim, scale, flags};
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(map->mu);
  bool capturing = false;
  hipError_t e = order_after(map, st, false, capturing);
  if (e != hipSuccess) return hip_fail(e, "ordering after the map's last use");
  const uint32_t ring = map->launches.fetch_add(1, std::memory_order_relaxed) % svg::kQueueRing;
  e = svg::launch_attn_fwd(g, map->buf, map->plan, ring, a, st);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  if (!capturing) {
    e = hipEventRecord(map->used, st);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    map->used_valid = true;
  }
  return ok();
}

svg_status svg_permute_tokens(const void* src, void* dst, int32_t frames,
                              int32_t tokens_per_frame, int32_t num_heads, int32_t head_dim,
                              const int32_t* head_kind, int32_t direction, void* stream) {
  if (!src || !dst || !head_kind) return fail(SVG_ERR_INVALID_ARG, "NULL pointer argument");
  if (frames < 1 || tokens_per_frame < 1 || num_heads < 1)
    return fail(SVG_ERR_INVALID_ARG, "frames, tokens_per_frame and num_heads must be >= 1");
  if ((int64_t)frames * tokens_per_frame > (1 << 30))
    return fail(SVG_ERR_INVALID_ARG, "sequence exceeds 2^30 tokens");
  if (head_dim < 8 || head_dim > 1024 || head_dim % 8)
    return fail(SVG_ERR_UNSUPPORTED, "head_dim %d: multiples of 8 up to 1024", head_dim);
  if ((int64_t)frames * tokens_per_frame * head_dim * 2 >= ((int64_t)1 << 31))
    return fail(SVG_ERR_UNSUPPORTED, "one head of %lld x %d bf16 values exceeds 2 GiB",
                (long long)frames * tokens_per_frame, head_dim);
  if (direction != SVG_TO_KERNEL_LAYOUT && direction != SVG_TO_ORIGINAL_LAYOUT)
    return fail(SVG_ERR_INVALID_ARG, "direction %d is not an svg_permute_dir", direction);
  for (int32_t h = 0; h < num_heads; ++h) {
    const int32_t kd = head_kind[h];
    if (kd != SVG_HEAD_SPATIAL && kd != SVG_HEAD_TEMPORAL && kd != SVG_HEAD_DENSE)
      return fail(SVG_ERR_INVALID_ARG, "head_kind[%d] = %d is not an svg_head_kind", h, kd);
  }
  if (!aligned16(src) || !aligned16(dst))
    return fail(SVG_ERR_ALIGNMENT, "src and dst must be 16-byte aligned");
  const uintptr_t bytes =
      (uintptr_t)num_heads * (uintptr_t)frames * tokens_per_frame * head_dim * 2;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return fail(SVG_ERR_INVALID_ARG, "src and dst overlap");
  const hipError_t e =
      svg::launch_permute_tokens(src, dst, frames, tokens_per_frame, num_heads, head_dim,
                                 head_kind, direction, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "permute kernel launch");
  return ok();
}

svg_status svg_autotune_tiles(const svg_mask_spec* spec, const void* q, const void* k,
                              const void* v, void* o, int32_t head_dim, float scale,
                              const int32_t* tile_q, const int32_t* tile_k, int32_t n_cand,
                              int32_t reps, void* stream, float* ms, int32_t* best) {
  if (!spec || !spec->head_kind) return fail(SVG_ERR_INVALID_ARG, "spec or its head_kind is NULL");
  if (!q || !k || !v || !o) return fail(SVG_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (!tile_q || !tile_k || !ms || !best)
    return fail(SVG_ERR_INVALID_ARG, "tile_q, tile_k, ms and best must be non-NULL");
  if (n_cand < 1 || n_cand > 256)
    return fail(SVG_ERR_INVALID_ARG, "n_cand %d outside [1, 256]", n_cand);
  if (reps < 1 || reps > 1000) return fail(SVG_ERR_INVALID_ARG, "reps %d outside [1, 1000]", reps);
  for (int32_t i = 0; i < n_cand; ++i)
    if (!tile_q_ok(tile_q[i]) || !tile_k_ok(tile_k[i]) ||
        !svg::attn_supported(head_dim, tile_q[i], tile_k[i]))
      return fail(SVG_ERR_UNSUPPORTED, "candidate %d: tiles %dx%d with head_dim %d have no kernel",
                  i, tile_q[i], tile_k[i], head_dim);
  const int64_t N = (int64_t)spec->frames * spec->grid_h * spec->grid_w;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t ev[2] = {nullptr, nullptr};
  for (hipEvent_t& e : ev) {
    const hipError_t he = hipEventCreate(&e);
    if (he != hipSuccess) {
      for (hipEvent_t x : ev)
        if (x) (void)hipEventDestroy(x);
      return hip_fail(he, "hipEventCreate");
    }
  }
  svg_status status = SVG_OK;
  int32_t arg = 0;
  for (int32_t i = 0; i < n_cand && status == SVG_OK; ++i) {
    svg_tile_map* map = nullptr;
    status = svg_build_tile_map(spec, tile_q[i], tile_k[i], stream, &map);
    if (status != SVG_OK) break;
    auto run = [&]() {
      return svg_attn_fwd(q, k, v, o, N, spec->num_heads, head_dim, scale, spec->head_kind, map,
                          0, stream);
    };
    status = run();  // untimed: first touch of the map and the inputs
    hipError_t he = hipSuccess;
    if (status == SVG_OK) he = hipEventRecord(ev[0], st);
    for (int32_t r = 0; r < reps && status == SVG_OK && he == hipSuccess; ++r) status = run();
    if (status == SVG_OK && he == hipSuccess) he = hipEventRecord(ev[1], st);
    if (status == SVG_OK && he == hipSuccess) he = hipEventSynchronize(ev[1]);
    float t = 0.f;
    if (status == SVG_OK && he == hipSuccess) he = hipEventElapsedTime(&t, ev[0], ev[1]);
    if (status == SVG_OK && he != hipSuccess) status = hip_fail(he, "timing the attention runs");
    if (status == SVG_OK) {
      ms[i] = t / (float)reps;
      if (ms[i] < ms[arg]) arg = i;
    }
    const std::string msg = g_last_error;
    const svg_status ds = svg_tile_map_destroy(map);
    if (status == SVG_OK) status = ds;
    else g_last_error = msg;  // keep the first failure's message
  }
  for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  if (status != SVG_OK) return status;
  *best = arg;
  return ok();
}

svg_status svg_route_heads(const svg_mask_spec* spec, const void* q, const void* k, const void* v,
                           int32_t head_dim, float scale, const int32_t* rows, int32_t n_rows,
                           void* stream, float* err, int32_t* kinds) {
  RouteArgs ra;
  const svg_status vs = route_validate(spec, q, k, v, head_dim, scale, rows, n_rows, kinds, ra);
  if (vs != SVG_OK) return vs;
  const int32_t H = spec->num_heads;
  const svg::RouteLayout L =
      svg::route_layout(ra.N, H, head_dim, n_rows, svg::route_slots(head_dim));
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_route_mu);
  if ((int)g_route_scratch.size() <= dev) g_route_scratch.resize(dev + 1);
  RouteScratch& rs = g_route_scratch[dev];
  if (rs.bytes < L.bytes) {
    if (rs.p) {
      e = hipFree(rs.p);
      rs = RouteScratch{};
      if (e != hipSuccess) return hip_fail(e, "hipFree");
    }
    e = hipMalloc(reinterpret_cast<void**>(&rs.p), (size_t)L.bytes);
    if (e != hipSuccess) {
      rs = RouteScratch{};
      return fail(SVG_ERR_OOM, "routing scratch of %lld bytes: %s", (long long)L.bytes,
                  hipGetErrorString(e));
    }
    rs.bytes = L.bytes;
  }
  char* scratch = rs.p;
  std::vector<float> err_h((size_t)H * 2);
  std::vector<int32_t> ordered((size_t)n_rows);
  order_rows(rows, n_rows, ra.S, ordered.data());
  e = hipMemcpyAsync(scratch + L.rows_off, ordered.data(), (size_t)n_rows * 4,
                     hipMemcpyHostToDevice, st);
  if (e == hipSuccess)
    e = svg::launch_route(q, k, v, scratch, L, ra.N, spec->frames, ra.S, H, head_dim, ra.W_f,
                          ra.W_s, spec->sink_first_frame ? 1 : 0, scale, n_rows, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(err_h.data(), scratch + L.err_off, err_h.size() * 4,
                       hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(kinds, scratch + L.kind_off, (size_t)H * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "routing kernels");
  if (err) std::memcpy(err, err_h.data(), err_h.size() * 4);
  return ok();
}

svg_status svg_route_heads_noalloc(const svg_mask_spec* spec, const void* q, const void* k,
                                   const void* v, int32_t head_dim, float scale,
                                   const int32_t* rows, int32_t n_rows, void* stream, float* err,
                                   int32_t* kinds) {
  RouteArgs ra;
  const svg_status vs = route_validate(spec, q, k, v, head_dim, scale, rows, n_rows, kinds, ra);
  if (vs != SVG_OK) return vs;
  const int32_t H = spec->num_heads;
  int64_t res_off = 0;
  const svg::RouteLayout L =
      svg::route_static_layout(ra.N, H, head_dim, n_rows, svg::route_slots(head_dim), &res_off);
  const int64_t need = res_off + (int64_t)H * 12;
  if (need > svg::kRouteStaticBytes)
    return fail(SVG_ERR_UNSUPPORTED,
                "routing without allocation needs %lld bytes of scratch for one head of %lld "
                "tokens, %d sampled rows and %d heads; the library's array holds %lld",
                (long long)need, (long long)ra.N, n_rows, H, (long long)svg::kRouteStaticBytes);
  char* sc = nullptr;
  hipError_t e = svg::route_static_scratch(&sc);
  if (e != hipSuccess) return hip_fail(e, "address of the routing scratch");
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  order_rows(rows, n_rows, ra.S, g_noalloc_rows);
  e = hipMemcpyAsync(sc + L.rows_off, g_noalloc_rows, (size_t)n_rows * 4, hipMemcpyHostToDevice,
                     st);
  if (e == hipSuccess)
    e = svg::launch_route_static(q, k, v, sc, L, res_off, ra.N, spec->frames, ra.S, H, head_dim,
                                 ra.W_f, ra.W_s, spec->sink_first_frame ? 1 : 0, scale, n_rows,
                                 st);
  // results to the caller's arrays: errors only when asked for
  if (e == hipSuccess && err)
    e = hipMemcpyAsync(err, sc + res_off, (size_t)H * 8, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(kinds, sc + res_off + (int64_t)H * 8, (size_t)H * 4,
                       hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "routing kernels");
  return ok();
}

}  // extern "C"
