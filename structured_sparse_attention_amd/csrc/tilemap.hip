// Tile-map builder: classify every (BQ x BK) tile of every head as SKIP /
// FULL / BOUNDARY and compact, per (head, Q tile), the KV tiles to execute.
//
// Tile-aware masking: a tile whose existing pairs are all retained runs
// mask-free, a mixed tile runs the per-element predicate, an empty tile is
// skipped ("Google Speeds Up Video Diffusion on TPUs with Optimized Sparse
// Attention", "Efficient Kernel Implementation"; Newsbite "Summary").
//
// Counting is exact integer interval arithmetic. Rows of a Q tile are split
// into runs that share the mask-relevant coordinate (the frame for spatial
// heads in natural order, the raster index for temporal heads in
// spatial-major order); every row of a run keeps the same columns, so a
// tile's count is sum(run length x retained columns of the run in the tile).
//   spatial run (frame f):  window [max(0,f-Wf)*S, min(F,f+Wf+1)*S) united
//                           with the sink [0, S)
//   temporal run (index s): band [max(0,s-Ws)*F, min(S,s+Ws+1)*F) united with
//                           the sink, the multiples of F
// Temporal heads execute only the band hull of KV tiles plus the frame-0
// keys outside it (raster indices [0,a) and [b,S)), so that most tiles are
// skipped although the strided sink touches every tile.
#include "svg_internal.hpp"

namespace svg {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 32-bit counting: sequences are at most 2^30 tokens, and a tile holds at
// most BQ x BK <= 2^20 x 2^10 = 2^30 pairs (the host caps both tile sizes),
// so every per-tile quantity fits; only the sums over a row of tiles need 64
// bits.
__device__ __forceinline__ int span32(int a, int b) { return b > a ? b - a : 0; }
// min(lim, v + w + 1) without forming v + w + 1 (w may be near INT32_MAX)
__device__ __forceinline__ int upper(int v, int w, int lim) { return w >= lim - v ? lim : v + w + 1; }

struct Counts {
  int mask;    // retained pairs of the exact mask
  int contig;  // pairs of the contiguous part (spatial: all; temporal: band)
};

// Retained columns in [c0, c1) of one row whose run coordinate is v. For
// temporal heads C0 = ceil(c0 / F) and C1 = ceil(c1 / F) bound the sink
// columns (multiples of F) of the tile; the band ends are multiples of F,
// so the sink columns inside the band need no division.
__device__ __forceinline__ Counts row_columns(const MapGeometry& g, int kind, int v, int c0,
                                              int c1, int C0, int C1) {
  Counts r;
  if (kind == SVG_HEAD_SPATIAL) {
    const int lo = max(0, v - g.W_f) * g.S;
    const int hi = upper(v, g.W_f, g.F) * g.S;
    int n = span32(max(lo, c0), min(hi, c1));
    if (g.sink) {
      n += span32(c0, min(g.S, c1));
      n -= span32(max(lo, c0), min(min(hi, g.S), c1));
    }
    r.mask = n;
    r.contig = n;
  } else {  // temporal
    const int lo_s = max(0, v - g.W_s), hi_s = upper(v, g.W_s, g.S);
    const int band = span32(max(lo_s * g.F, c0), min(hi_s * g.F, c1));
    r.contig = band;
    r.mask = band + (g.sink ? (C1 - C0) - span32(max(lo_s, C0), min(hi_s, C1)) : 0);
  }
  return r;
}

template <int N>
__device__ void block_sum(int64_t (&v)[N], int64_t* lds) {
  // lds: kThreads/64 * N int64
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    int64_t x = v[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_down(x, off, 64);
    if (lane == 0) lds[wave * N + i] = x;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int64_t s = 0;
      for (int w = 0; w < kThreads / 64; ++w) s += lds[w * N + i];
      v[i] = s;
    }
  }
}

// Ordered compaction of one row's classes in [lo, hi] (all threads of the
// block): FULL ids ascending, then BOUNDARY ids ascending.
__device__ void compact_row(const uint8_t* cls_row, int lo, int hi, int32_t* out) {
  __shared__ int wave_tot[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int pos = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const uint8_t want = pass == 0 ? SVG_TILE_FULL : SVG_TILE_BOUNDARY;
    for (int c = lo; c <= hi; c += kThreads) {
      const int kt = c + threadIdx.x;
      const bool flag = kt <= hi && cls_row[kt] == want;
      const uint64_t m = __ballot(flag);
      const int before = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == 0) wave_tot[wave] = __popcll(m);
      __syncthreads();
      int off = 0, tot = 0;
      for (int w = 0; w < kThreads / 64; ++w) {
        off += w < wave ? wave_tot[w] : 0;
        tot += wave_tot[w];
      }
      if (flag) out[pos + off + before] = kt;
      pos += tot;
      __syncthreads();
    }
  }
}

// Classification of one row of tiles, then the row's compaction: FULL ids of
// the run range ascending, then BOUNDARY ids ascending, into the row's own
// nK entries (entries[row * nK ...]), so that no scan across rows is needed.
__global__ __launch_bounds__(kThreads) void classify_kernel(MapGeometry g, MapBuffers b) {
  const int qt = blockIdx.x, h = blockIdx.y;
  const int64_t row = (int64_t)h * g.nQ + qt;
  const int kind = b.kinds[h];
  const int64_t q0 = (int64_t)qt * g.BQ, q1 = min<int64_t>(g.N, q0 + g.BQ);
  const int64_t rows = q1 - q0;

  int64_t lo = 0, hi = g.nK - 1, sa = 0, sb = g.S;
  if (kind == SVG_HEAD_TEMPORAL) {
    const int64_t s0 = q0 / g.F, s1 = (q1 - 1) / g.F;
    lo = (max<int64_t>(0, s0 - g.W_s) * g.F) / g.BK;
    hi = ((min<int64_t>(g.S - 1, s1 + g.W_s) + 1) * g.F - 1) / g.BK;
    if (g.sink) {
      sa = cdiv(lo * g.BK, g.F);
      sb = cdiv(min<int64_t>(g.N, (hi + 1) * g.BK), g.F);
    }
  }
  const int64_t unit = (kind == SVG_HEAD_TEMPORAL) ? g.F : g.S;

  // skip, full, boundary, exec_full, exec_boundary, retained
  int64_t acc[6] = {0, 0, 0, 0, 0, 0};
  uint8_t* cls_row = b.classes + row * g.nK;
  const int N = (int)g.N, iq0 = (int)q0, iq1 = (int)q1, irows = (int)rows, iu = (int)unit;
  const int v0 = iq0 / iu, v1 = (iq1 - 1) / iu;
  for (int kt = threadIdx.x; kt < g.nK; kt += kThreads) {
    const int c0 = kt * g.BK, c1 = min(N, c0 + g.BK);
    const int area = irows * (c1 - c0);
    const int C0 = (c0 + g.F - 1) / g.F, C1 = (c1 + g.F - 1) / g.F;
    int cnt;
    if (kind == SVG_HEAD_DENSE) {
      cnt = area;
    } else {
      int mask = 0, contig = 0;
      for (int v = v0; v <= v1; ++v) {
        const int len = min(iq1, (v + 1) * iu) - max(iq0, v * iu);
        const Counts c = row_columns(g, kind, v, c0, c1, C0, C1);
        mask += len * c.mask;
        contig += len * c.contig;
      }
      cnt = mask;
      if (g.round == SVG_ROUND_TILE) {
        if (contig > 0)
          cnt = area;  // the contiguous part is rounded out to the whole tile
        else if (kind == SVG_HEAD_TEMPORAL)
          cnt = g.sink ? irows * (C1 - C0) : 0;  // exact strided sink
        else
          cnt = 0;
      }
    }
    const uint8_t c = cnt == 0 ? SVG_TILE_SKIP : (cnt == area ? SVG_TILE_FULL : SVG_TILE_BOUNDARY);
    cls_row[kt] = c;
    acc[0] += c == SVG_TILE_SKIP;
    acc[1] += c == SVG_TILE_FULL;
    acc[2] += c == SVG_TILE_BOUNDARY;
    const bool run = kt >= lo && kt <= hi;
    acc[3] += run && c == SVG_TILE_FULL;
    acc[4] += run && c == SVG_TILE_BOUNDARY;
    acc[5] += cnt;
  }
  __shared__ int64_t lds[kThreads / 64 * 6];
  block_sum(acc, lds);
  // (the barrier in block_sum follows every thread's class bytes, so the
  // whole block sees them)
  compact_row(cls_row, (int)lo, (int)hi, b.entries + row * g.nK);
  if (threadIdx.x == 0) {
    int32_t* ri = b.rowinfo + row * kRowInfo;
    ri[0] = (int32_t)acc[3];
    ri[1] = (int32_t)acc[4];
    ri[2] = (int32_t)sa;
    ri[3] = (int32_t)sb;
    ri[4] = (int32_t)lo;
    ri[5] = (int32_t)hi;
    ri[6] = 0;
    ri[7] = 0;
    int64_t* rs = b.rowstats + row * kRowStats;
    rs[0] = g.nK;
    rs[1] = acc[0];
    rs[2] = acc[1];
    rs[3] = acc[2];
    rs[4] = acc[3];
    rs[5] = acc[4];
    rs[6] = cdiv(sa, g.BK) + cdiv(g.S - sb, g.BK);
    rs[7] = acc[5];
  }
}

// Head kinds of up to kKindChunk heads, carried in the kernel arguments so
// that the build needs neither a host-to-device copy nor a wait for one.
constexpr int kKindChunk = 256;
struct KindChunk {
  int32_t h0, n;
  int8_t kind[kKindChunk];
};
__global__ __launch_bounds__(kKindChunk) void set_kinds_kernel(KindChunk c, int32_t* kinds) {
  if ((int)threadIdx.x < c.n) kinds[c.h0 + threadIdx.x] = c.kind[threadIdx.x];
}

}  // namespace

hipError_t launch_set_kinds(const int32_t* host_kinds, int32_t H, int32_t* dev_kinds,
                            hipStream_t stream) {
  for (int32_t h0 = 0; h0 < H; h0 += kKindChunk) {
    KindChunk c;
    c.h0 = h0;
    c.n = H - h0 < kKindChunk ? H - h0 : kKindChunk;
    for (int i = 0; i < kKindChunk; ++i) c.kind[i] = (int8_t)(i < c.n ? host_kinds[h0 + i] : 0);
    hipLaunchKernelGGL(set_kinds_kernel, dim3(1), dim3(kKindChunk), 0, stream, c, dev_kinds);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_build_tile_map(const MapGeometry& g, const MapBuffers& b,
                                 hipStream_t stream) {
  const dim3 rows_grid(g.nQ, g.H);
  hipLaunchKernelGGL(classify_kernel, rows_grid, dim3(kThreads), 0, stream, g, b);
  return hipGetLastError();
}

}  // namespace svg
