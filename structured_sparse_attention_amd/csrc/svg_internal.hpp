// Internal declarations shared by the host API (svg_api.cpp) and the HIP
// kernel sources. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "svg_attn.h"

namespace svg {

// Per (head, Q tile) schedule row, int32 x 8 in device memory:
//   [0] n_full  [1] n_boundary  [2] sink_a  [3] sink_b  [4] hull_lo [5] hull_hi
constexpr int kRowInfo = 8;
// Per-row statistics, int64 x 8 (same order as svg_head_stats).
constexpr int kRowStats = 8;

struct MapGeometry {
  int64_t N;
  int32_t F, S, H;
  int32_t W_f, W_s, sink, round;
  int32_t BQ, BK, nQ, nK;
};

struct MapBuffers {
  int32_t* kinds = nullptr;     // [H]
  uint8_t* classes = nullptr;   // [H][nQ][nK]
  int32_t* rowinfo = nullptr;   // [H*nQ][kRowInfo]
  int32_t* entries = nullptr;   // [H*nQ][nK]: row r's entries start at r * nK
  int64_t* rowstats = nullptr;  // [H*nQ][kRowStats]
  int64_t capacity = 0;         // H*nQ*nK
};

// Write the head kinds (host array [H], values 0..2) to device memory from
// kernel arguments: queued on `stream`, the host array may go away at once.
hipError_t launch_set_kinds(const int32_t* host_kinds, int32_t H, int32_t* dev_kinds,
                            hipStream_t stream);

// Launch the tile-map kernel (classify and compact every row).
hipError_t launch_build_tile_map(const MapGeometry& g, const MapBuffers& b,
                                 hipStream_t stream);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int32_t head_dim;
  float scale;
  uint32_t flags;
};

// A work item as the attention kernel reads it: the plan's entry and the
// schedule row data of its unit, so that starting an item takes one load.
struct ItemDesc {
  int32_t unit, s0, s1, slot;        // PlanItem
  int32_t n_full, n_tiles, ebeg, sa;  // the row's FULL and executed tiles, its
  int32_t sb, head, q0, kind;         //   first entry, sink range; head, first
};                                    //   query row, head kind
static_assert(sizeof(ItemDesc) == 48, "three 16-byte loads");

// Work plan of the persistent attention launch (plan.hpp), device side.
// `dev` holds, as int32: a header [n_items, n_combine, n_slots, 0], then
// the queue bounds queue_ptr [n_xcd + 2] (queue x < n_xcd: XCD x's items;
// queue n_xcd: the shared tail) in a field of n_wg + 2 entries padded to a
// multiple of 4, then max_items ItemDesc (12 int32 each, queue by queue in
// queue order) and max_combine combine entries (PlanCombine, 4 int32 each).
// `counters` is a ring of kQueueRing sets of n_xcd + 1 queue positions;
// every launch takes the next set and zeroes it first.
constexpr int32_t kQueueRing = 256;
struct PlanBuffers {
  int32_t* dev = nullptr;
  int32_t* counters = nullptr;  // [kQueueRing][n_xcd + 1]
  float* part_o = nullptr;  // [max_slots][rows of a workgroup][128]
  float* part_ml = nullptr; // [max_slots][rows of a workgroup][2]
  int32_t n_wg = 0, n_xcd = 0;
  int64_t max_items = 0, max_slots = 0, max_combine = 0;
  int64_t ptr_ints() const { return (n_wg + 2 + 3) / 4 * 4; }
  int64_t items_off() const { return 4 + ptr_ints(); }
  int64_t combine_off() const { return items_off() + 12 * max_items; }
  int64_t dev_ints() const { return combine_off() + 4 * max_combine; }
};

// Query rows per workgroup (32 per wave) of the attention kernel for a Q
// tile size, and its waves; 0 when the size has no kernel.
int32_t attn_waves(int32_t tile_q);
constexpr int32_t kAttnQRowsPerWave = 32;
constexpr int32_t kAttnStepKeys = 64;   // keys per pipeline step
constexpr int32_t kAttnMaxHeadDim = 128;
// Cost of starting a work item, in steps (Q loads, stage-0 latency, epilogue).
constexpr int32_t kPlanItemOverhead = 4;
// Parts of a cut row are kept at least this many steps where possible.
constexpr int32_t kPlanMinPart = 32;
// Work units per block dealt to the XCDs in rounds (plan_persistent).
constexpr int32_t kPlanBlockUnits = 32;
// Share of the work kept for the shared tail of the launch (plan_persistent):
// enough to absorb XCDs that run about 5% apart (measured on MI355X: 3-6%
// between the fastest and the slowest XCD of a chip; 4% and 7% measured
// alike on the main workload).
constexpr double kPlanTail = 0.05;
// Relative cost of a 64-key step by head kind (spatial, temporal, dense),
// measured on the main workload's shape with the same kernel.
constexpr float kPlanStepWeight[3] = {1.030f, 1.000f, 0.985f};

// Launch the attention forward kernel for a built map and planned launch
// (queue positions from counter set `ring`, zeroed first), then the pass
// that merges the parts of cut rows. Returns hipErrorInvalidValue for a
// head_dim / tile size without an instance.
hipError_t launch_attn_fwd(const MapGeometry& g, const MapBuffers& b, const PlanBuffers& pl,
                           uint32_t ring, const AttnArgs& a, hipStream_t stream);
bool attn_supported(int32_t head_dim, int32_t tile_q, int32_t tile_k);

// Scratch of one routing call (byte offsets into one allocation).
struct RouteLayout {
  int64_t pitch;      // columns per V^T row
  int64_t split_len;  // keys per split (a multiple of 64)
  int64_t n_split;
  int64_t vt_off, rows_off, part_off, row_err_off, err_off, kind_off, bytes;
};
// slots: workgroups of the routing kernel the device holds at once (0 if
// unknown), which sets the number of key splits; max_split > 0 caps them.
RouteLayout route_layout(int64_t N, int32_t H, int32_t D, int32_t n_rows, int32_t slots,
                         int64_t max_split = 0);
// CUs x resident routing workgroups per CU on the current device, 0 on failure.
int route_slots(int32_t D);
// Queue the routing kernels; the sampled rows must already be at
// scratch + rows_off. Results: float [H][2] at err_off, int32 [H] at kind_off.
hipError_t launch_route(const void* q, const void* k, const void* v, char* scratch,
                        const RouteLayout& L, int64_t N, int32_t F, int32_t S, int32_t H,
                        int32_t D, int32_t W_f, int32_t W_s, int32_t sink, float scale,
                        int32_t n_rows, hipStream_t stream);

// Routing without allocation: a per-device static scratch of
// kRouteStaticBytes, used one head at a time.
constexpr int64_t kRouteStaticBytes = 48ll << 20;
// The calling thread's current device's scratch (device address).
hipError_t route_static_scratch(char** out);
// Layout of one head's routing in the scratch, and the offset of the
// results of all heads (float [H][2] errors, then int32 [H] kinds) after it.
// The caller checks results_off + H * 12 <= kRouteStaticBytes.
RouteLayout route_static_layout(int64_t N, int32_t H, int32_t D, int32_t n_rows, int32_t slots,
                                int64_t* results_off);
// Queue the routing kernels head by head in the scratch `sc`; the sampled
// rows must already be at sc + L.rows_off.
hipError_t launch_route_static(const void* q, const void* k, const void* v, char* sc,
                               const RouteLayout& L, int64_t results_off, int64_t N, int32_t F,
                               int32_t S, int32_t H, int32_t D, int32_t W_f, int32_t W_s,
                               int32_t sink, float scale, int32_t n_rows, hipStream_t stream);

// kinds: host array [H]; one launch per head.
hipError_t launch_permute_tokens(const void* src, void* dst, int32_t F,
                                 int32_t S, int32_t H, int32_t D,
                                 const int32_t* kinds, int32_t direction,
                                 hipStream_t stream);

}  // namespace svg

// Host side of the launch plan: pinned staging for the map's row info (in)
// and the plan image (out), filled by a host function queued on the build
// stream; the plan's statistics once it has run.
struct PlanJob {
  svg::MapGeometry geom;
  int32_t nsub = 1, wgq = 256;
  const int32_t* kinds = nullptr;   // the map's head kinds [H]
  int32_t* rowinfo_host = nullptr;  // pinned [H*nQ][kRowInfo]
  int32_t* image_host = nullptr;    // pinned, PlanBuffers::dev_ints()
  svg::PlanBuffers* plan = nullptr;
  int64_t items = 0, split_units = 0, slots = 0, max_load = 0, total_load = 0;
};

// The opaque map type of the public header.
struct svg_tile_map {
  svg::MapGeometry geom;
  svg::MapBuffers buf;
  svg::PlanBuffers plan;
  PlanJob job;
  std::vector<int32_t> kinds;
  int device = 0;
  hipEvent_t built = nullptr;  // recorded after every (re)build
  mutable std::atomic<uint32_t> launches{0};  // picks each launch's queue counters
  // Uses of the map are ordered on the device (they share its workspace):
  // `used` is recorded after every attention launch outside stream capture.
  hipEvent_t used = nullptr;
  mutable bool used_valid = false;
  mutable std::mutex mu;
};
