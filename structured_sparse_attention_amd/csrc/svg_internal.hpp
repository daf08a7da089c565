// Internal declarations shared by the host API (svg_api.cpp) and the HIP
// kernel sources. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  int32_t* row_ptr = nullptr;   // [H*nQ + 1]
  int32_t* entries = nullptr;   // [capacity]
  int64_t* rowstats = nullptr;  // [H*nQ][kRowStats]
  int64_t* stats = nullptr;     // [H][kRowStats]
  int64_t capacity = 0;
};

// Launch the tile-map kernels (classify, scan, compact, per-head stats).
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

// Launch the attention forward kernel for a built map. Returns
// hipErrorInvalidValue for a head_dim / tile size without an instance.
hipError_t launch_attn_fwd(const MapGeometry& g, const MapBuffers& b,
                           const AttnArgs& a, hipStream_t stream);
bool attn_supported(int32_t head_dim, int32_t tile_q, int32_t tile_k);

// Scratch of one routing call (byte offsets into one allocation).
struct RouteLayout {
  int64_t pitch;      // columns per V^T row
  int64_t split_len;  // keys per split (a multiple of 32)
  int64_t n_split;
  int64_t vt_off, rows_off, part_off, row_err_off, err_off, kind_off, bytes;
};
// slots: workgroups of the routing kernel the device holds at once (0 if
// unknown), which sets the number of key splits.
RouteLayout route_layout(int64_t N, int32_t H, int32_t D, int32_t n_rows, int32_t slots);
// CUs x resident routing workgroups per CU on the current device, 0 on failure.
int route_slots(int32_t D);
// Queue the routing kernels; the sampled rows must already be at
// scratch + rows_off. Results: float [H][2] at err_off, int32 [H] at kind_off.
hipError_t launch_route(const void* q, const void* k, const void* v, char* scratch,
                        const RouteLayout& L, int64_t N, int32_t F, int32_t S, int32_t H,
                        int32_t D, int32_t W_f, int32_t W_s, int32_t sink, float scale,
                        int32_t n_rows, hipStream_t stream);

// kinds: host array [H]; one launch per head.
hipError_t launch_permute_tokens(const void* src, void* dst, int32_t F,
                                 int32_t S, int32_t H, int32_t D,
                                 const int32_t* kinds, int32_t direction,
                                 hipStream_t stream);

}  // namespace svg

// The opaque map type of the public header.
struct svg_tile_map {
  svg::MapGeometry geom;
  svg::MapBuffers buf;
  std::vector<int32_t> kinds;
  int device = 0;
  hipEvent_t built = nullptr;  // recorded after every (re)build
};
