// Sampled head routing: each head goes to the spatial or the temporal mask
// according to how well each reproduces dense attention on a sample of query
// rows ("Google Speeds Up Video Diffusion on TPUs with Optimized Sparse
// Attention", "Sparse Attention Patterns"; "Accelerating Spatio-Temporal
// Attention for Video Diffusion on TPUs", Newsbite, summary). For every
// sampled row the three outputs -- every key, spatial mask, temporal mask --
// are computed; a head's error for a mask is the mean squared difference of
// that mask's outputs from the dense ones over the sampled rows and the d
// output columns, and the head takes the mask with the smaller error (the
// spatial one on a tie). Inputs are in the original frame-major order.
//
// Four kernels:
//   vt_kernel       V -> V^T per head ([d][pitch], zero padded), so that a
//                   lane fetches 8 consecutive keys of one dim with one
//                   16-byte load. HBM-bound, one read and one write of V.
//   route_partial   one wave per (head, mask, 32 sampled rows, key split):
//                   per step of 32 keys S^T = K Q^T with
//                   v_mfma_f32_32x32x16_bf16 (K from LDS, Q in VGPRs), the
//                   mask's keep bits, an online softmax (fp32, P rounded to
//                   bf16) and O^T += V^T P^T (V^T from LDS). One mask per
//                   wave keeps one O^T in registers (three would spill); the
//                   six waves of a workgroup share the K and V^T of a step.
//                   Writes (max, sum, O^T) per (row, split, mask).
//   route_rows      one workgroup per (sampled row, head): merges the splits,
//                   forms the three outputs and the row's squared errors.
//   route_decide    one workgroup per head: sums the rows' errors (float64,
//                   fixed order) and takes the decision.
#include "svg_internal.hpp"

#include <math.h>

#include <algorithm>
#include <mutex>

namespace svg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int RK = 32;  // keys per step
constexpr int RQ = 32;  // sampled rows per wave
constexpr int RW = 6;   // waves per workgroup: 3 masks x 2 row blocks, one key split

struct RouteParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vt;    // [H][D][pitch]
  const int32_t* rows;   // [n_rows], original-order query indices
  float* part;           // [H][n_rows][n_split][3][D + 2]
  float* err;            // [H][2]
  int32_t* kind;         // [H]
  int32_t n_rows, N, F, S, W_f, W_s, sink, pitch, n_split, split_len;
  float c;               // scale * log2(e)
};

// As in the attention kernel: with A row m of a 32-key block holding key
// sigma(m), accumulator v of a lane is key 16*(v/8) + 8*(lane/32) + v%8, so
// a lane's accumulators 8kk..8kk+7 are the B operand of the PV product for
// keys 16kk..16kk+15.
__device__ __forceinline__ int sigma(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// The values of lanes (lane & 31) and (lane & 31) + 32: the two halves of a
// row's keys.
__device__ __forceinline__ void halves(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// V^T of one head: thread (8-key group, 8-dim group) -> 8 loads, register
// transpose, 8 stores; columns past N are zero.
template <int D>
__global__ __launch_bounds__(256) void vt_kernel(const uint4* __restrict__ v,
                                                 uint4* __restrict__ vt, int64_t total, int32_t N,
                                                 int64_t pitch) {
  constexpr int DC = D / 8;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tid >= total) return;
  const int glo = (int)(tid & 7);
  int64_t r = tid >> 3;
  const int c = (int)(r % DC);
  r /= DC;
  const int64_t g8 = pitch / 64;
  const int64_t ghi = r % g8, h = r / g8;
  const int64_t col0 = (ghi * 8 + glo) * 8;
  const uint4* vh = v + h * (int64_t)N * DC;
  u16x8 in[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (col0 + i < N) x = vh[(col0 + i) * DC + c];
    in[i] = __builtin_bit_cast(u16x8, x);
  }
  uint4* dst = vt + ((h * D + 8 * c) * pitch + col0) / 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u16x8 y = {in[0][j], in[1][j], in[2][j], in[3][j],
                     in[4][j], in[5][j], in[6][j], in[7][j]};
    dst[j * (pitch / 8)] = __builtin_bit_cast(uint4, y);
  }
}

// Bits j in [a, b] (inclusive, clipped to [0, 31]).
__device__ __forceinline__ uint32_t bit_range(int a, int b) {
  a = max(a, 0);
  b = min(b, 31);
  if (a > b) return 0u;
  const uint32_t hi = b >= 31 ? ~0u : ((1u << (b + 1)) - 1u);
  return hi & ~((1u << a) - 1u);
}

// Keep bits of the 32 keys key0 + j (frame fk0 and raster index sk0 at
// j = 0) for a query at (fq, sq): x = 1 spatial, |fq - f| <= W_f; x = 2
// temporal, |sq - s| <= W_s; either or frame 0 with the sink. With S >= 32
// the keys span at most two frames, split at j = S - sk0, and each mask is
// one frame test or one interval of j per frame; shorter frames take the
// key-by-key path.
__device__ __forceinline__ uint32_t mask_bits(const RouteParams& p, int x, int fq, int sq,
                                              int fk0, int sk0) {
  if (p.S >= 32) {
    const int jw = p.S - sk0;  // first key of frame fk0 + 1
    const uint32_t lo = jw >= 32 ? ~0u : ((1u << jw) - 1u);
    auto frame_kept = [&](int f) { return abs(fq - f) <= p.W_f || (p.sink && f == 0); };
    if (x == 1) return (frame_kept(fk0) ? lo : 0u) | (frame_kept(fk0 + 1) ? ~lo : 0u);
    uint32_t m = (bit_range(sq - p.W_s - sk0, sq + p.W_s - sk0) & lo) |
                 (bit_range(sq - p.W_s - sk0 + p.S, sq + p.W_s - sk0 + p.S) & ~lo);
    if (p.sink && fk0 == 0) m |= lo;
    return m;
  }
  uint32_t m = 0;
  int f = fk0, sk = sk0;
  for (int j = 0; j < 32; ++j) {
    const bool snk = p.sink && f == 0;
    const bool kv = x == 1 ? (abs(fq - f) <= p.W_f || snk) : (abs(sq - sk) <= p.W_s || snk);
    m |= (uint32_t)kv << j;
    if (++sk == p.S) {
      sk = 0;
      ++f;
    }
  }
  return m;
}

// Workgroup: RW waves = 3 masks x 2 blocks of 32 sampled rows, all on the
// same key split, sharing each step's K rows and V^T slice through LDS (the
// global traffic is that of one wave, not six). A step's 32 K rows and
// d x 32 V^T values are fetched into registers one step ahead and written to
// LDS between two barriers. LDS rows are padded (K: 16 bytes per row; V^T:
// 80-byte rows) so that 16 lanes reading 16 rows at one column hit 16
// distinct 4-bank groups.
template <int D>
__global__ __launch_bounds__(RW * 64) void route_partial(RouteParams p) {
  constexpr int NDB = D / 32;
  constexpr int KC = D / 8;               // 16-byte chunks per K row
  constexpr int KROWB = 16 * (KC + 1);    // bytes per K row in LDS
  constexpr int VROWB = 80;               // bytes per V^T row (32 keys + pad)
  constexpr int NKCH = RK * KC, NCH = NKCH + D * (RK / 8);
  constexpr int PER = (NCH + RW * 64 - 1) / (RW * 64);
  constexpr float NEG_INF = -__builtin_huge_valf();
  __shared__ __attribute__((aligned(16))) char lds[RK * KROWB + D * VROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int x = wave % 3;                       // 0 dense, 1 spatial, 2 temporal
  const int rb = blockIdx.y * 2 + wave / 3;     // block of 32 sampled rows
  const int split = blockIdx.x, h = blockIdx.z;

  const size_t hoff = (size_t)h * p.N * D;
  const int ri = rb * RQ + l32;
  const bool rvalid = ri < p.n_rows;
  const int t = rvalid ? p.rows[ri] : 0;
  const int fq = t / p.S, sq = t - fq * p.S;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 q4 = make_uint4(0, 0, 0, 0);
    if (rvalid) q4 = *(const uint4*)(p.q + hoff + (size_t)t * D + 16 * ks + 8 * hl);
    qf[ks] = __builtin_bit_cast(bf16x8, q4);
  }
  const uint16_t* kh = p.k + hoff;
  const uint16_t* vth = p.vt + (size_t)h * D * p.pitch;

  // chunk c of a step: K row m (key sigma(m)), chunk c % KC; or V^T dim
  // (c - NKCH) / 4, keys 8 * ((c - NKCH) % 4) .. +7
  static_assert(PER <= 3, "at most three staged chunks per thread");
  uint4 pre0 = make_uint4(0, 0, 0, 0), pre1 = pre0, pre2 = pre0;
  auto fetch1 = [&](int key0, int j, uint4& r) __attribute__((always_inline)) {
    const int c = tid + j * RW * 64;
    if (c < NKCH) {
      const int m = c / KC, ch = c - m * KC;
      const int key = min(key0 + sigma(m), p.N - 1);
      r = *(const uint4*)(kh + (size_t)key * D + 8 * ch);
    } else if (c < NCH) {
      const int cv = c - NKCH, dim = cv >> 2, g = cv & 3;
      r = *(const uint4*)(vth + (size_t)dim * p.pitch + key0 + 8 * g);
    }
  };
  auto store1 = [&](int j, const uint4& r) __attribute__((always_inline)) {
    const int c = tid + j * RW * 64;
    if (c < NKCH) {
      const int m = c / KC, ch = c - m * KC;
      *(uint4*)(lds + m * KROWB + 16 * ch) = r;
    } else if (c < NCH) {
      const int cv = c - NKCH, dim = cv >> 2, g = cv & 3;
      *(uint4*)(lds + RK * KROWB + dim * VROWB + 16 * g) = r;
    }
  };
  auto fetch = [&](int key0) __attribute__((always_inline)) {
    fetch1(key0, 0, pre0);
    if constexpr (PER > 1) fetch1(key0, 1, pre1);
    if constexpr (PER > 2) fetch1(key0, 2, pre2);
  };
  auto store = [&]() __attribute__((always_inline)) {
    store1(0, pre0);
    if constexpr (PER > 1) store1(1, pre1);
    if constexpr (PER > 2) store1(2, pre2);
  };

  float m = NEG_INF, l = 0.f;
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;

  const int k0 = split * p.split_len, k1 = min(p.N, k0 + p.split_len);
  int fk0 = k0 / p.S, sk0 = k0 - fk0 * p.S;  // (frame, raster index) of key0
  fetch(k0);
  for (int key0 = k0; key0 < k1; key0 += RK, sk0 += RK) {
    while (sk0 >= p.S) {
      sk0 -= p.S;
      ++fk0;
    }
    __syncthreads();  // every wave is done with the previous step's LDS
    store();
    __syncthreads();
    if (key0 + RK < k1) fetch(key0 + RK);
    // S^T = K Q^T for keys key0 .. key0+31 (rows past N clamped; masked)
    f32x16 s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 a = *(const bf16x8*)(lds + l32 * KROWB + 32 * ks + 16 * hl);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
    }
    // keep bits of the step's 32 keys under mask x (bit j: key key0 + j),
    // then the lane's 16 (accumulator v: offset 16*(v/8) + 8hl + v%8)
    const int nval = k1 - key0;
    uint32_t keep = nval >= 32 ? ~0u : ((1u << nval) - 1u);
    if (x != 0) keep &= mask_bits(p, x, fq, sq, fk0, sk0);
    const uint32_t lk = ((keep >> (8 * hl)) & 0xFFu) | (((keep >> (16 + 8 * hl)) & 0xFFu) << 8);
    // online softmax in log2 units
    float mx = NEG_INF;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if ((lk >> v) & 1u) mx = fmaxf(mx, s[v] * p.c);
    {
      float a, b;
      halves(mx, a, b);
      mx = fmaxf(a, b);
    }
    const float mn = fmaxf(m, mx);
    const float alpha = mn == NEG_INF ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    float e[16], ls = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      e[v] = ((lk >> v) & 1u) ? __builtin_amdgcn_exp2f(s[v] * p.c - mn) : 0.f;
      ls += e[v];
    }
    l = l * alpha + ls;
    m = mn;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
    }
    // O^T += V^T P^T: V^T of dims 32db + l32, keys 16kk + 8hl .. +7
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint4 w = make_uint4(pack_bf16(e[8 * kk + 0], e[8 * kk + 1]),
                                 pack_bf16(e[8 * kk + 2], e[8 * kk + 3]),
                                 pack_bf16(e[8 * kk + 4], e[8 * kk + 5]),
                                 pack_bf16(e[8 * kk + 6], e[8 * kk + 7]));
      const bf16x8 pf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 vf = *(const bf16x8*)(lds + RK * KROWB + (32 * db + l32) * VROWB +
                                           32 * kk + 16 * hl);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
      }
    }
  }

  // (max, sum, O^T) of this split: O^T accumulator v of block db is dim
  // 32db + 8(v/4) + 4hl + v%4 of row l32.
  float lt;
  {
    float a, b;
    halves(l, a, b);
    lt = a + b;
  }
  if (!rvalid) return;
  float* out = p.part + ((((size_t)h * p.n_rows + ri) * p.n_split + split) * 3 + x) * (D + 2);
  if (hl == 0) {
    out[0] = m;
    out[1] = lt;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) out[2 + 32 * db + 8 * (v >> 2) + 4 * hl + (v & 3)] = o[db][v];
}

// One workgroup of D threads per (sampled row, head): merges the splits of
// the three outputs; writes the row's two squared-error sums (float64).
template <int D>
__global__ __launch_bounds__(D) void route_rows(RouteParams p, double* row_err) {
  const int ri = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const float* base = p.part + ((size_t)h * p.n_rows + ri) * p.n_split * 3 * (D + 2);
  float out[3];
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    float M = -__builtin_huge_valf();
    for (int sp = 0; sp < p.n_split; ++sp) M = fmaxf(M, base[(sp * 3 + x) * (D + 2)]);
    float L = 0.f, A = 0.f;
    for (int sp = 0; sp < p.n_split; ++sp) {
      const float* b = base + (sp * 3 + x) * (D + 2);
      const float w = b[0] == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(b[0] - M);
      L += b[1] * w;
      A += b[2 + d] * w;
    }
    out[x] = L > 0.f ? A / L : 0.f;
  }
  __shared__ double red[2][D];
  red[0][d] = (double)(out[1] - out[0]) * (double)(out[1] - out[0]);
  red[1][d] = (double)(out[2] - out[0]) * (double)(out[2] - out[0]);
  __syncthreads();
  for (int w = D / 2; w > 0; w >>= 1) {
    if (d < w) {
      red[0][d] += red[0][d + w];
      red[1][d] += red[1][d + w];
    }
    __syncthreads();
  }
  if (d == 0) {
    row_err[((size_t)h * p.n_rows + ri) * 2] = red[0][0];
    row_err[((size_t)h * p.n_rows + ri) * 2 + 1] = red[1][0];
  }
}

// One workgroup per head: sums the rows' errors in a fixed order and decides.
__global__ __launch_bounds__(256) void route_decide(RouteParams p, const double* row_err, int D) {
  const int h = blockIdx.x;
  double es = 0.0, et = 0.0;
  for (int ri = threadIdx.x; ri < p.n_rows; ri += 256) {
    es += row_err[((size_t)h * p.n_rows + ri) * 2];
    et += row_err[((size_t)h * p.n_rows + ri) * 2 + 1];
  }
  __shared__ double red[2][256];
  red[0][threadIdx.x] = es;
  red[1][threadIdx.x] = et;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      red[0][threadIdx.x] += red[0][threadIdx.x + w];
      red[1][threadIdx.x] += red[1][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double n = (double)p.n_rows * D;
    const double s = red[0][0] / n, tt = red[1][0] / n;
    p.err[2 * h] = (float)s;
    p.err[2 * h + 1] = (float)tt;
    p.kind[h] = s <= tt ? SVG_HEAD_SPATIAL : SVG_HEAD_TEMPORAL;
  }
}

}  // namespace

int route_slots(int32_t D) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const void* f = D == 128 ? reinterpret_cast<const void*>(&route_partial<128>)
                           : reinterpret_cast<const void*>(&route_partial<64>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, f, RW * 64, 0) != hipSuccess) return 0;
  return cus * per;
}

RouteLayout route_layout(int64_t N, int32_t H, int32_t D, int32_t n_rows, int32_t slots,
                         int64_t max_split) {
  RouteLayout L;
  L.pitch = (N + 63) / 64 * 64 + 64;  // a multiple of 64; keys past N read zeros
  const int64_t pairs = ((n_rows + RQ - 1) / RQ + 1) / 2;  // workgroups per (head, split)
  // Key splits. The time is about (rounds of resident workgroups) x (keys
  // per split), so take the split count that minimises rounds / splits, up
  // to about two rounds of workgroups (more splits cost partial results and
  // merging), the fewest on a tie: no partial last round idles most of the
  // chip. Without the occupancy figure, about 4096 waves in all.
  const int64_t per = (int64_t)H * pairs, kmax = (N + RK - 1) / RK;
  int64_t ns = (4096 + RW * per - 1) / (RW * per);
  if (slots > 0) {
    const int64_t hi = std::max<int64_t>(1, std::min<int64_t>(kmax, (2 * slots + per - 1) / per));
    ns = 1;
    for (int64_t c = 2; c <= hi; ++c) {
      const int64_t r = (c * per + slots - 1) / slots, rb = (ns * per + slots - 1) / slots;
      if (r * ns < rb * c) ns = c;  // r / c < rb / ns
    }
  }
  ns = std::max<int64_t>(1, std::min<int64_t>(ns, kmax));
  if (max_split > 0) ns = std::min(ns, max_split);
  L.split_len = ((N + ns - 1) / ns + RK - 1) / RK * RK;
  L.n_split = (N + L.split_len - 1) / L.split_len;
  const int64_t a = 256;
  auto up = [&](int64_t b) { return (b + a - 1) / a * a; };
  L.vt_off = 0;
  L.rows_off = up(L.vt_off + (int64_t)H * D * L.pitch * 2);
  L.part_off = up(L.rows_off + (int64_t)n_rows * 4);
  L.row_err_off = up(L.part_off + (int64_t)H * n_rows * L.n_split * 3 * (D + 2) * 4);
  L.err_off = up(L.row_err_off + (int64_t)H * n_rows * 2 * 8);
  L.kind_off = up(L.err_off + (int64_t)H * 2 * 4);
  L.bytes = up(L.kind_off + (int64_t)H * 4);
  return L;
}

hipError_t launch_route(const void* q, const void* k, const void* v, char* scratch,
                        const RouteLayout& L, int64_t N, int32_t F, int32_t S, int32_t H,
                        int32_t D, int32_t W_f, int32_t W_s, int32_t sink, float scale,
                        int32_t n_rows, hipStream_t stream) {
  RouteParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.vt = (const uint16_t*)(scratch + L.vt_off);
  p.rows = (const int32_t*)(scratch + L.rows_off);
  p.part = (float*)(scratch + L.part_off);
  p.err = (float*)(scratch + L.err_off);
  p.kind = (int32_t*)(scratch + L.kind_off);
  p.n_rows = n_rows;
  p.N = (int32_t)N;
  p.F = F;
  p.S = S;
  p.W_f = W_f;
  p.W_s = W_s;
  p.sink = sink;
  p.pitch = (int32_t)L.pitch;
  p.n_split = (int32_t)L.n_split;
  p.split_len = (int32_t)L.split_len;
  p.c = scale * 1.4426950408889634f;
  const int64_t total = (int64_t)H * (D / 8) * (L.pitch / 8);
  const dim3 vt_grid((unsigned)((total + 255) / 256));
  const dim3 grid((unsigned)L.n_split, (unsigned)(((n_rows + RQ - 1) / RQ + 1) / 2), (unsigned)H);
  double* row_err = (double*)(scratch + L.row_err_off);
  if (D == 128) {
    hipLaunchKernelGGL(vt_kernel<128>, vt_grid, dim3(256), 0, stream, (const uint4*)v,
                       (uint4*)(scratch + L.vt_off), total, (int32_t)N, L.pitch);
    hipLaunchKernelGGL(route_partial<128>, grid, dim3(RW * 64), 0, stream, p);
    hipLaunchKernelGGL(route_rows<128>, dim3(n_rows, H), dim3(128), 0, stream, p, row_err);
  } else if (D == 64) {
    hipLaunchKernelGGL(vt_kernel<64>, vt_grid, dim3(256), 0, stream, (const uint4*)v,
                       (uint4*)(scratch + L.vt_off), total, (int32_t)N, L.pitch);
    hipLaunchKernelGGL(route_partial<64>, grid, dim3(RW * 64), 0, stream, p);
    hipLaunchKernelGGL(route_rows<64>, dim3(n_rows, H), dim3(64), 0, stream, p, row_err);
  } else {
    return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(route_decide, dim3(H), dim3(256), 0, stream, p, (const double*)row_err, D);
  return hipGetLastError();
}

}  // namespace svg

// ---- Routing without allocation (svg_route_heads_noalloc) ----------------
// One scratch array per device, held until the process ends. Host code
// never passes its name to a kernel (in host code it stands for a host-side
// symbol); the device address comes from hipGetSymbolAddress, once per
// device, with that device current.
static __device__ __align__(256) char scratch[svg::kRouteStaticBytes];

namespace svg {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices] = {};
}  // namespace

hipError_t route_static_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

RouteLayout route_static_layout(int64_t N, int32_t H, int32_t D, int32_t n_rows, int32_t slots,
                                int64_t* results_off) {
  // One head at a time: V^T, rows, partial results and row errors of one
  // head, then every head's (errors, kind); the key splits shrink until the
  // layout fits the array.
  const int64_t kmax = (N + 31) / 32;
  RouteLayout L = route_layout(N, 1, D, n_rows, slots, 0);
  for (int64_t ns = L.n_split; ns >= 1; --ns) {
    L = route_layout(N, 1, D, n_rows, slots, std::min(ns, kmax));
    if (L.bytes + (int64_t)H * 16 + 256 <= kRouteStaticBytes) break;
  }
  *results_off = (L.bytes + 255) / 256 * 256;
  return L;
}

hipError_t launch_route_static(const void* q, const void* k, const void* v, char* sc,
                               const RouteLayout& L, int64_t results_off, int64_t N, int32_t F,
                               int32_t S, int32_t H, int32_t D, int32_t W_f, int32_t W_s,
                               int32_t sink, float scale, int32_t n_rows, hipStream_t stream) {
  const size_t head = (size_t)N * D * 2;
  for (int32_t h = 0; h < H; ++h) {
    // this head's (errors, kind) go to the shared result area
    RouteLayout Lh = L;
    Lh.err_off = results_off + (int64_t)h * 8;
    Lh.kind_off = results_off + (int64_t)H * 8 + (int64_t)h * 4;
    const hipError_t e =
        launch_route((const char*)q + h * head, (const char*)k + h * head,
                     (const char*)v + h * head, sc, Lh, N, F, S, 1, D, W_f, W_s, sink, scale,
                     n_rows, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace svg
