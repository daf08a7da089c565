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
//   vt_kernel       V -> V^T per head ([d][pitch], zero padded), keys
//                   reordered inside each 32-key chunk to the order in which
//                   the MFMA below holds its weights, so that a lane fetches
//                   its 8 keys of one dim with one 16-byte load. HBM-bound,
//                   one read and one write of V.
//   route_partial   one wave per (head, 16 sampled rows, key split), eight
//                   waves to a workgroup sharing each step's K rows and V^T
//                   slice through LDS. Per step of 64 keys: S^T = K Q^T once
//                   (v_mfma_f32_16x16x32_bf16, K from LDS, Q in VGPRs), the
//                   dense online-softmax weights P (fp32, rounded to bf16),
//                   the spatial and temporal weights as P with the masked
//                   keys zeroed, and O^T += V^T P^T for all three (one V^T
//                   fragment from LDS feeds three MFMAs). The three outputs
//                   share the dense running maximum, so a mask's weights are
//                   the dense ones; a mask whose kept weights would all fall
//                   below fp32's range under that maximum is caught after the
//                   merge and recomputed exactly. Writes (max, sum, O^T) per
//                   (row, split, output).
//   route_rows      one workgroup per (sampled row, head): merges the splits,
//                   forms the three outputs (the exact path where a mask's
//                   merged sum is too small to trust) and the row's squared
//                   errors.
//   route_decide    one workgroup per head: sums the rows' errors (float64,
//                   fixed order) and takes the decision.
#include "svg_internal.hpp"

#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace svg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int RK = 64;  // keys per step
constexpr int RQ = 16;  // sampled rows per wave
constexpr int RW = 8;   // waves per workgroup (one block of RQ rows each), one key split
// Running maxima may lag the true one by up to 2^kLazy before the
// accumulators are rescaled (weights stay below 2^kLazy).
constexpr float kLazy = 8.f;
// A mask's merged weight sum, in units of the dense maximum, below which
// its output is recomputed exactly: each lost weight is below 2^-126 and a
// row has fewer than 2^31 keys, so above this bound the lost share is below
// 2^-31.
constexpr float kExactBelow = 0x1p-64f;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// Reductions over the four lanes of a row (lanes n, n + 16, n + 32, n + 48):
// the 16-lane swap pairs rows {0,1} and {2,3} of the wave, the 32-lane swap
// the two halves.
__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Position 32c + 8gg + j of a V^T row holds key 32c + 4gg + j (j < 4) or
// 32c + 16 + 4gg + j - 4 (j >= 4): the keys whose weights lane group gg of
// the 16x16 MFMA holds for chunk c (accumulators of two 16-key blocks).
__device__ __forceinline__ int64_t vt_key(int64_t pos) {
  const int64_t j = pos & 7, gg = (pos >> 3) & 3;
  return (pos & ~(int64_t)31) + 4 * gg + (j < 4 ? j : 12 + j);
}

// V^T of one head: thread (8-position group, 8-dim group) -> 8 loads,
// register transpose, 8 stores; keys past N are zero.
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
    const int64_t key = vt_key(col0 + i);
    uint4 x = make_uint4(0, 0, 0, 0);
    if (key < N) x = vh[key * DC + c];
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

// A lane's 16 keep bits for the step's keys at relative positions [a, b]:
// bit 4mb + i stands for key 16mb + g4 + i (g4 = 4 * (lane / 16)), the key
// of the lane's accumulator i of 16-key block mb.
__device__ __forceinline__ uint32_t lane_bits(int a, int b, int g4) {
  a = max(a, -64);
  b = min(b, 128);
  const uint32_t w0 = bit_range(a, b) >> g4, w1 = bit_range(a - 32, b - 32) >> g4;
  return (w0 & 0xFu) | ((w0 >> 12) & 0xF0u) | ((w1 & 0xFu) << 8) | ((w1 >> 4) & 0xF000u);
}

struct RouteParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;     // [H][N][D], read by the exact path
  const uint16_t* vt;    // [H][D][pitch], keys reordered as vt_key states
  const int32_t* rows;   // [n_rows], original-order query indices
  float* part;           // [H][n_rows][n_split][3][D + 2]
  float* err;            // [H][2]
  int32_t* kind;         // [H]
  int32_t n_rows, N, F, S, W_f, W_s, sink, pitch, n_split, split_len;
  float c;               // scale * log2(e)
};

// Keep bits of the lane's 16 keys of the step at key0 (frame fk0, raster
// index sk0) for the query at (fq, sq): x = 1 spatial, |fq - f| <= W_f;
// x = 2 temporal, |sq - s| <= W_s; either or frame 0 with the sink. With
// S >= 64 the keys span at most two frames, split at relative key jb, and
// each mask keeps a whole frame or one interval of it; shorter frames take
// the key-by-key path.
// sq_lo and sq_hi bound the raster indices of the wave's rows: where the
// step lies in one frame and inside (or outside) every row's band, the
// temporal bits are decided for the whole wave without per-lane work. (The
// sampled rows are ordered by raster index, so a wave's band edges are close
// together and most steps take that path.)
__device__ __forceinline__ uint32_t lane_keep(const RouteParams& p, int x, int fq, int sq,
                                              int key0, int fk0, int sk0, int g4, int sq_lo,
                                              int sq_hi) {
  if (p.S >= RK) {
    const int jb = p.S - sk0;  // first key of frame fk0 + 1
    if (x == 2 && jb >= RK) {
      if (p.sink && fk0 == 0) return 0xFFFFu;
      if (sk0 >= sq_hi - p.W_s && sk0 + RK - 1 <= sq_lo + p.W_s) return 0xFFFFu;
      if (sk0 + RK - 1 < sq_lo - p.W_s || sk0 > sq_hi + p.W_s) return 0u;
    }
    if (x == 1) {
      auto kept = [&](int f) { return abs(fq - f) <= p.W_f || (p.sink && f == 0); };
      const bool ka = kept(fk0);
      if (jb >= RK) return ka ? 0xFFFFu : 0u;
      const uint32_t lo = lane_bits(0, jb - 1, g4);
      return (ka ? lo : 0u) | (kept(fk0 + 1) ? (~lo & 0xFFFFu) : 0u);
    }
    uint32_t m = (p.sink && fk0 == 0)
                     ? lane_bits(0, jb - 1, g4)
                     : lane_bits(max(sq - p.W_s - sk0, 0), min(sq + p.W_s - sk0, jb - 1), g4);
    if (jb < RK) m |= lane_bits(max(sq - p.W_s + jb, jb), sq + p.W_s + jb, g4);
    return m;
  }
  uint32_t m = 0;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int key = key0 + 16 * (v >> 2) + g4 + (v & 3);
    const int f = key / p.S, s = key - f * p.S;
    const bool snk = p.sink && f == 0;
    const bool kv = x == 1 ? (abs(fq - f) <= p.W_f || snk) : (abs(sq - s) <= p.W_s || snk);
    m |= (uint32_t)kv << v;
  }
  return m;
}

// Workgroup: RW waves, each its own 16 sampled rows, all on one key split.
// Stage (two buffers): the step's 64 K rows (2D + 32 bytes each) and the d
// V^T rows of its 64 keys (160 bytes each). A wave's operand read takes 16
// rows at 4 consecutive 16-byte columns; with these 32-byte pads the LDS
// serves it without bank conflicts, where 16-byte pads (right for 32 rows
// at 2 columns) cost a second pass (measured with the LDS bank-conflict
// counter). Each thread fetches its share of the next step's stage into
// registers one step ahead and writes it after the current step's compute;
// one barrier per step.
template <int D>
__global__ __launch_bounds__(RW * 64) void route_partial(RouteParams p) {
  constexpr int NKC = D / 32, NDB = D / 16;
  constexpr int KROWB = 2 * D + 32, VROWB = 2 * RK + 32;
  constexpr int KBYTES = RK * KROWB, STB = KBYTES + D * VROWB;
  constexpr int KCH = D / 8;  // 16-byte chunks per K row
  constexpr int NKCH = RK * KCH, NCH = NKCH + D * (RK / 8);
  constexpr int NT = RW * 64, PER = NCH / NT;
  static_assert(NKCH % NT == 0 && NCH % NT == 0 && PER <= 4, "whole staging rounds");
  constexpr float NEG_INF = -__builtin_huge_valf();
  __shared__ __attribute__((aligned(16))) char lds[2 * STB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15, g4 = 4 * g;
  const int split = blockIdx.x, h = blockIdx.z;
  const int rb = blockIdx.y * RW + wave;  // block of 16 sampled rows
  const bool wvalid = rb * RQ < p.n_rows;
  const int ri = rb * RQ + n;
  const bool rvalid = ri < p.n_rows;
  // lanes past the last row stand in for it (their results are not written)
  const int t = p.rows[min(ri, p.n_rows - 1)];
  const int fq = t / p.S, sq = t - fq * p.S;
  int sq_lo = sq, sq_hi = sq;  // over the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    sq_lo = min(sq_lo, __shfl_xor(sq_lo, o));
    sq_hi = max(sq_hi, __shfl_xor(sq_hi, o));
  }
  sq_lo = __builtin_amdgcn_readfirstlane(sq_lo);
  sq_hi = __builtin_amdgcn_readfirstlane(sq_hi);
  const size_t hoff = (size_t)h * p.N * D;
  // B operand of S^T: row n, dims 32kc + 8g .. +7
  bf16x8 qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    uint4 q4 = make_uint4(0, 0, 0, 0);
    if (rvalid) q4 = *(const uint4*)(p.q + hoff + (size_t)t * D + 32 * kc + 8 * g);
    qf[kc] = __builtin_bit_cast(bf16x8, q4);
  }
  const uint16_t* kh = p.k + hoff;
  const uint16_t* vth = p.vt + (size_t)h * D * p.pitch;

  // chunk c of a stage: K row c / KCH (key0 + row, clamped to N - 1; masked),
  // 16 bytes c % KCH; then V^T dim (c - NKCH) / 8, positions 8 * (c % 8) .. +7
  static_assert(PER == 2 || PER == 4, "two or four staged chunks per thread");
  uint4 pre0, pre1, pre2, pre3;  // separate values: an array here would live in scratch
  auto fetch1 = [&](int key0, int j, uint4& r) __attribute__((always_inline)) {
    const int c = tid + j * NT;
    // uniform base + 32-bit lane offset (one head's K and V^T stay below
    // 2 GiB): no 64-bit address per lane has to stay live across the loop
    if (j < NKCH / NT) {
      const int key = min(key0 + c / KCH, p.N - 1);
      r = *(const uint4*)((const char*)kh + (uint32_t)(key * (2 * D) + 16 * (c % KCH)));
    } else {
      const int cv = c - NKCH;
      r = *(const uint4*)((const char*)(vth + key0) +
                          (uint32_t)(2 * ((cv >> 3) * p.pitch + 8 * (cv & 7))));
    }
  };
  auto store1 = [&](char* buf, int j, const uint4& r) __attribute__((always_inline)) {
    const int c = tid + j * NT;
    if (j < NKCH / NT) {
      *(uint4*)(buf + (c / KCH) * KROWB + 16 * (c % KCH)) = r;
    } else {
      const int cv = c - NKCH;
      *(uint4*)(buf + KBYTES + (cv >> 3) * VROWB + 16 * (cv & 7)) = r;
    }
  };
  auto fetch = [&](int key0) __attribute__((always_inline)) {
    fetch1(key0, 0, pre0);
    fetch1(key0, 1, pre1);
    if constexpr (PER == 4) {
      fetch1(key0, 2, pre2);
      fetch1(key0, 3, pre3);
    }
  };
  auto store = [&](char* buf) __attribute__((always_inline)) {
    store1(buf, 0, pre0);
    store1(buf, 1, pre1);
    if constexpr (PER == 4) {
      store1(buf, 2, pre2);
      store1(buf, 3, pre3);
    }
  };

  float m = NEG_INF, ld = 0.f, ls = 0.f, lt = 0.f;  // lane partial sums
  f32x4 od[NDB], os[NDB], ot[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) od[db][i] = os[db][i] = ot[db][i] = 0.f;

  const int k0 = split * p.split_len, k1 = min(p.N, k0 + p.split_len);
  int fk0 = k0 / p.S, sk0 = k0 - fk0 * p.S;  // (frame, raster index) of key0
  fetch(k0);
  store(lds);
  if (k0 + RK < k1) fetch(k0 + RK);
  __syncthreads();
  int it = 0;
  for (int key0 = k0; key0 < k1; key0 += RK, ++it) {
    const char* buf = lds + (it & 1) * STB;
    if (wvalid) {
      // S^T = K Q^T: accumulator i of block mb is key 16mb + 4g + i of row n
      // every K fragment is read before the first MFMA, so that the reads'
      // latencies overlap
      bf16x8 ka[4][NKC];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
          ka[mb][kc] = *(const bf16x8*)(buf + (16 * mb + n) * KROWB + 64 * kc + 16 * g);
      f32x4 s[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[mb][i] = 0.f;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[mb][kc], qf[kc], s[mb], 0, 0, 0);
      // V^T fragments of the first 32 keys, read while the weights are formed
      bf16x8 va[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        va[db] = *(const bf16x8*)(buf + KBYTES + (16 * db + n) * VROWB + 16 * g);
      const int nval = k1 - key0;  // keys of the split left (the step's are valid below it)
      float mx = NEG_INF;
      if (nval >= RK) {
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v >> 2][v & 3]);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (16 * (v >> 2) + g4 + (v & 3) < nval) mx = fmaxf(mx, s[v >> 2][v & 3]);
      }
      mx = row_max4(mx) * p.c;
      // lazy rescale: rows whose maximum rose by more than 2^kLazy take it
      const bool grow = mx > m + kLazy;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? mx : m;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mn) : 1.f;
        m = mn;
        ld *= alpha;
        ls *= alpha;
        lt *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            od[db][i] *= alpha;
            os[db][i] *= alpha;
            ot[db][i] *= alpha;
          }
      }
      // dense weights of the lane's 16 keys
      float e[16], rs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) e[v] = __builtin_amdgcn_exp2f(fmaf(s[v >> 2][v & 3], p.c, -m));
      if (nval < RK) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (16 * (v >> 2) + g4 + (v & 3) >= nval) e[v] = 0.f;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) rs += e[v];
      ld += rs;
      // B operands of the PV product: chunk c2 is e[8c2 .. 8c2 + 7]
      uint32_t pd[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) pd[k] = pack_bf16(e[2 * k], e[2 * k + 1]);
      // masked weights: where every lane keeps all or none of its keys the
      // mask zeroes whole packed words, else each weight
      auto masked = [&](uint32_t lk, uint32_t* px, float& lx) __attribute__((always_inline)) {
        if (!__builtin_amdgcn_ballot_w64(lk != 0u && lk != 0xFFFFu)) {
          const uint32_t mk = lk ? ~0u : 0u;
#pragma unroll
          for (int k = 0; k < 8; ++k) px[k] = pd[k] & mk;
          lx += lk ? rs : 0.f;
        } else {
          float ex[16], sx = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            ex[v] = __uint_as_float(__float_as_uint(e[v]) &
                                    (uint32_t)__builtin_amdgcn_sbfe((int)lk, v, 1));
            sx += ex[v];
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) px[k] = pack_bf16(ex[2 * k], ex[2 * k + 1]);
          lx += sx;
        }
      };
      // A mask that keeps none of the step's keys for any row of the wave
      // adds nothing to its output: its weights and MFMAs are skipped (the
      // sums with zero weights are the same values).
      uint32_t ps[8], pt[8];
      const uint32_t lks = lane_keep(p, 1, fq, sq, key0, fk0, sk0, g4, sq_lo, sq_hi);
      const bool any_s = __builtin_amdgcn_ballot_w64(lks != 0u) != 0;
      if (any_s) masked(lks, ps, ls);
      const uint32_t lkt = lane_keep(p, 2, fq, sq, key0, fk0, sk0, g4, sq_lo, sq_hi);
      const bool any_t = __builtin_amdgcn_ballot_w64(lkt != 0u) != 0;
      if (any_t) masked(lkt, pt, lt);
      // O^T += V^T P^T: V^T of dims 16db + n, positions 32c2 + 8g .. +7
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16x8 bd = __builtin_bit_cast(
            bf16x8, make_uint4(pd[4 * c2], pd[4 * c2 + 1], pd[4 * c2 + 2], pd[4 * c2 + 3]));
        const bf16x8 bs = __builtin_bit_cast(
            bf16x8, make_uint4(ps[4 * c2], ps[4 * c2 + 1], ps[4 * c2 + 2], ps[4 * c2 + 3]));
        const bf16x8 bt = __builtin_bit_cast(
            bf16x8, make_uint4(pt[4 * c2], pt[4 * c2 + 1], pt[4 * c2 + 2], pt[4 * c2 + 3]));
        bf16x8 vb[NDB];  // the next 32 keys' fragments, read during these MFMAs
        if (c2 == 0) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            vb[db] = *(const bf16x8*)(buf + KBYTES + (16 * db + n) * VROWB + 64 + 16 * g);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          od[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], bd, od[db], 0, 0, 0);
        if (any_s) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            os[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], bs, os[db], 0, 0, 0);
        }
        if (any_t) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            ot[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], bt, ot[db], 0, 0, 0);
        }
        if (c2 == 0) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) va[db] = vb[db];
        }
      }
    }
    if (key0 + RK < k1) {
      store(lds + ((it + 1) & 1) * STB);
      if (key0 + 2 * RK < k1) fetch(key0 + 2 * RK);
    }
    __syncthreads();
    sk0 += RK;
    while (sk0 >= p.S) {
      sk0 -= p.S;
      ++fk0;
    }
  }

  // (max, sum, O^T) of this split for the three outputs: accumulator i of
  // block db is dim 16db + 4g + i of row n.
  ld = row_sum4(ld);
  ls = row_sum4(ls);
  lt = row_sum4(lt);
  // The lane's row and group again, from the lane count: kept live across
  // the loop they would take registers the loop needs.
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int ge = lane_e >> 4, ri_e = rb * RQ + (lane_e & 15);
  if (ri_e >= p.n_rows) return;
  float* out = p.part + (((size_t)h * p.n_rows + ri_e) * p.n_split + split) * 3 * (D + 2);
  if (ge == 0) {
    out[0] = m;
    out[1] = ld;
    out[D + 2] = m;
    out[D + 3] = ls;
    out[2 * (D + 2)] = m;
    out[2 * (D + 2) + 1] = lt;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 2 + 16 * db + 4 * ge + i;
      out[d] = od[db][i];
      out[D + 2 + d] = os[db][i];
      out[2 * (D + 2) + d] = ot[db][i];
    }
}

// Output x (1 spatial, 2 temporal) of sampled row t, computed directly:
// the kept keys' scores in fp32, their maximum, then the normalised sum of
// exp2(score - maximum) V. D threads; sh holds 2D floats. For rows whose
// kept weights all fall far below the dense maximum (see kExactBelow).
template <int D>
__device__ float exact_output(const RouteParams& p, int h, int t, int x, float* sh) {
  const int d = threadIdx.x;
  const size_t hoff = (size_t)h * p.N * D;
  const int fq = t / p.S, sq = t - fq * p.S;
  __syncthreads();
  sh[d] = bf16_to_f32(p.q[hoff + (size_t)t * D + d]);
  __syncthreads();
  auto kept = [&](int j) {
    const int f = j / p.S, s = j - f * p.S;
    const bool snk = p.sink && f == 0;
    return x == 1 ? (abs(fq - f) <= p.W_f || snk) : (abs(sq - s) <= p.W_s || snk);
  };
  auto score = [&](int j) {
    const uint16_t* kr = p.k + hoff + (size_t)j * D;
    float acc = 0.f;
    for (int i = 0; i < D; ++i) acc = fmaf(sh[i], bf16_to_f32(kr[i]), acc);
    return acc * p.c;
  };
  float mx = -__builtin_huge_valf();
  for (int j = d; j < p.N; j += D)
    if (kept(j)) mx = fmaxf(mx, score(j));
  sh[D + d] = mx;
  __syncthreads();
  for (int w = D / 2; w > 0; w >>= 1) {
    if (d < w) sh[D + d] = fmaxf(sh[D + d], sh[D + d + w]);
    __syncthreads();
  }
  mx = sh[D];
  __syncthreads();
  float o = 0.f, l = 0.f;
  for (int base = 0; base < p.N; base += D) {
    const int j = base + d;
    sh[D + d] = (j < p.N && kept(j)) ? __builtin_amdgcn_exp2f(score(j) - mx) : 0.f;
    __syncthreads();
    const int cnt = min(D, p.N - base);
    for (int jj = 0; jj < cnt; ++jj) {
      const float wj = sh[D + jj];
      l += wj;
      o = fmaf(wj, bf16_to_f32(p.v[hoff + (size_t)(base + jj) * D + d]), o);
    }
    __syncthreads();
  }
  return o / l;
}

// One workgroup of D threads per (sampled row, head): merges the splits of
// the three outputs; writes the row's two squared-error sums (float64). The
// splits' maxima and sums are spread over the threads and reduced within
// each wave, then across the waves through LDS; each thread then sums its
// output column over the splits in order, with the weights of D splits at a
// time staged in LDS, so that the column's loads are independent of each
// other and can be in flight together.
template <int D>
__global__ __launch_bounds__(D) void route_rows(RouteParams p, double* row_err) {
  constexpr int NWV = D / 64;  // waves
  const int ri = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const float* base = p.part + ((size_t)h * p.n_rows + ri) * p.n_split * 3 * (D + 2);
  __shared__ float sh[2 * D];
  __shared__ float wsh[3][D], rsh[3][NWV];
  constexpr float NEG_INF = -__builtin_huge_valf();
  // the three values' maxima (take_max) or sums over the block; every thread
  // gets the same results
  auto reduce3 = [&](float (&v)[3], bool take_max) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 3; ++x) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float u = __shfl_xor(v[x], o);
        v[x] = take_max ? fmaxf(v[x], u) : v[x] + u;
      }
      if ((d & 63) == 0) rsh[x][d >> 6] = v[x];
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      v[x] = rsh[x][0];
#pragma unroll
      for (int i = 1; i < NWV; ++i) v[x] = take_max ? fmaxf(v[x], rsh[x][i]) : v[x] + rsh[x][i];
    }
    __syncthreads();
  };
  float M[3] = {NEG_INF, NEG_INF, NEG_INF};
  for (int sp = d; sp < p.n_split; sp += D)
#pragma unroll
    for (int x = 0; x < 3; ++x) M[x] = fmaxf(M[x], base[(sp * 3 + x) * (D + 2)]);
  reduce3(M, true);
  float L[3] = {0.f, 0.f, 0.f}, A[3] = {0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < p.n_split; c0 += D) {
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      float w = 0.f;
      if (c0 + d < p.n_split) {
        const float* b = base + ((c0 + d) * 3 + x) * (D + 2);
        w = b[0] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(b[0] - M[x]);
        L[x] += b[1] * w;
      }
      wsh[x][d] = w;
    }
    __syncthreads();
    const int cnt = min(D, p.n_split - c0);
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const float* a = base + (c0 * 3 + x) * (D + 2) + 2 + d;
#pragma unroll 8
      for (int j = 0; j < cnt; ++j) A[x] += a[(size_t)j * 3 * (D + 2)] * wsh[x][j];
    }
    __syncthreads();
  }
  reduce3(L, false);
  float out[3];
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    // every thread holds the same L: the branch is uniform
    if (x > 0 && !(L[x] >= kExactBelow)) out[x] = exact_output<D>(p, h, p.rows[ri], x, sh);
    else out[x] = L[x] > 0.f ? A[x] / L[x] : 0.f;
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
  const int64_t pairs = ((n_rows + RQ - 1) / RQ + RW - 1) / RW;  // workgroups per (head, split)
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
  p.v = (const uint16_t*)v;
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
  const dim3 grid((unsigned)L.n_split, (unsigned)(((n_rows + RQ - 1) / RQ + RW - 1) / RW),
                  (unsigned)H);
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
  const int64_t kmax = (N + RK - 1) / RK;
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
