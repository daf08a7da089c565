// Structured-sparse attention forward for gfx950 (MI355X).
//
// One workgroup of NW waves computes 32*NW query rows of one head (one map Q
// tile, or a slice of it) against the KV tiles its schedule lists: FULL tiles
// (mask-free), then BOUNDARY tiles (per-element predicate), then -- temporal
// heads only -- the frame-0 keys outside the band hull, read at a stride of F
// rows (mask-free). This is the full/boundary split of the pages' kernel
// ("Google Speeds Up Video Diffusion on TPUs with Optimized Sparse
// Attention", "Efficient Kernel Implementation"; Newsbite "Summary").
//
// Work per 64-key step and wave (32 queries, head dim D):
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16, K from LDS (A), Q in VGPRs (B).
//                  Every lane owns one query column, so the row max and row
//                  sum are in-lane plus one v_permlane32_swap.
//   P^T = exp2(S^T * c - m * c), c = scale * log2(e), rounded to bf16.
//   O^T += V^T P^T V^T from LDS with the gfx950 transposing read
//                  ds_read_b64_tr_b16 (A), P^T from VGPRs (B).
// The row maximum is refreshed lazily: O and the row sum are rescaled only
// when a new maximum exceeds the reference by more than 8 in log2 units, so
// exp2 values stay below 2^8 and the final O / l is unchanged.
//
// K and V move from HBM straight into LDS (global_load_lds_dwordx4, no VGPR
// staging), double-buffered: the loads of step j+1 are in flight while step j
// computes. LDS rows are padded (K by 16 bytes, V by 32) so that every read
// is bank-conflict free and every read address is a per-lane base plus a
// compile-time offset; K rows are stored in the order the S^T accumulator
// layout needs for P^T to be the B operand of the PV product as it stands.
// Workgroups are remapped so that consecutive Q tiles of a head run on the
// same XCD and share its L2.
#include "svg_internal.hpp"

#include <math.h>

namespace svg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int CK = 64;  // keys per pipeline step
constexpr int QW = 32;  // query rows per wave

template <int D>
struct Layout {
  static constexpr int NCH = D / 8;          // 16-byte chunks per row
  static constexpr int KSLOTS = NCH + 1;     // K row + one pad slot
  static constexpr int VSLOTS = NCH + 2;     // V row + two pad slots
  static constexpr int KROW = 16 * KSLOTS;   // bytes per K row in LDS
  static constexpr int VROW = 16 * VSLOTS;   // bytes per V row in LDS
  static constexpr int KTILE = CK * KROW;
  static constexpr int VTILE = CK * VROW;
  static constexpr int KLOADS = KTILE / 1024;  // 1 KiB wave-wide DMA loads
  static constexpr int VLOADS = VTILE / 1024;
  static constexpr int BUF = KTILE + VTILE;
  static_assert(KTILE % 1024 == 0 && VTILE % 1024 == 0, "tiles must be whole KiB");
};

struct KParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int32_t N, F, S, W_f, W_s, sink;
  int32_t BQ, BK, nQ, nsub, total_wg, cpt;
  const int32_t* kinds;
  const int32_t* rowinfo;
  const int32_t* row_ptr;
  const int32_t* entries;
  float c;             // scale * log2(e)
  float thr;           // lazy-rescale threshold in raw score units
  int32_t mask_all;    // evaluate the mask on every executed step
  int32_t round_tile;  // the map rounds the contiguous mask part to whole tiles
};

struct Step {
  int32_t base;    // kernel-layout row of the step's first key
  int32_t stride;  // rows between consecutive keys (1, or F for sink keys)
  int32_t ncols;   // valid keys in this step (<= CK; <= 0 possible)
  int32_t pred;    // evaluate the head mask / column limit per element
};

// Accumulator v of a 32x32 MFMA output sits in row 8*(v/4) + 4*(lane/32) +
// v%4. LDS row m of a K block holds key sigma(m), so accumulator v of a lane
// is key 16*(v/8) + 8*(lane/32) + v%8: a lane's 8 consecutive accumulators
// are 8 consecutive keys, the B-operand slice the PV product needs from it.
__device__ __forceinline__ int sigma(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

__device__ __forceinline__ int xcd_remap(int i, int T) {
  const int x = i & 7, j = i >> 3, per = T >> 3, rem = T & 7;
  return x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

// Values of this lane and of lane ^ 32.
__device__ __forceinline__ void halves(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ Step step_at(const KParams& p, int j, int n_tile_steps, int n_full,
                                        int ebeg, int n_s1, int sa, int sb) {
  Step s;
  if (j < n_tile_steps) {
    const int e = j / p.cpt, part = j - e * p.cpt;
    const int kt = p.entries[ebeg + e];
    const int c0 = kt * p.BK + part * CK;
    const int end = min(p.N, kt * p.BK + p.BK);
    s.base = c0;
    s.stride = 1;
    s.ncols = min(CK, end - c0);
    s.pred = (e >= n_full) | p.mask_all | (s.ncols < CK);
  } else {
    const int js = j - n_tile_steps;
    int s0, lim;
    if (js < n_s1) {
      s0 = js * CK;
      lim = sa;
    } else {
      s0 = sb + (js - n_s1) * CK;
      lim = p.S;
    }
    s.base = s0 * p.F;
    s.stride = p.F;
    s.ncols = min(CK, lim - s0);
    s.pred = p.mask_all | (s.ncols < CK);
  }
  return s;
}

// Queue the DMA of one step's K and V rows into an LDS buffer. Each wave-wide
// load moves 64 x 16 bytes to 1 KiB of consecutive LDS; lane t fills slot t.
// Pad slots re-read chunk 0 of their row (in bounds, never read back).
template <int D, int NW>
__device__ __forceinline__ void issue_loads(const KParams& p, const uint16_t* Kh,
                                            const uint16_t* Vh, const Step& s, char* buf,
                                            int wave, int lane) {
  using Lt = Layout<D>;
  constexpr int TOTAL = Lt::KLOADS + Lt::VLOADS;
#pragma unroll
  for (int i0 = 0; i0 < TOTAL; i0 += NW) {
    const int i = i0 + wave;
    if (i < TOTAL) {
      const bool isv = i >= Lt::KLOADS;
      const int blk = isv ? i - Lt::KLOADS : i;
      const int slot = blk * 64 + lane;
      int prow, c;
      if (isv) {
        prow = slot / Lt::VSLOTS;
        c = slot - prow * Lt::VSLOTS;
      } else {
        prow = slot / Lt::KSLOTS;
        c = slot - prow * Lt::KSLOTS;
      }
      const int r = isv ? prow : ((prow & ~31) | sigma(prow & 31));
      const int rr = r < s.ncols ? r : 0;
      const int krow = min(s.base + rr * s.stride, p.N - 1);
      const uint16_t* src = (isv ? Vh : Kh) + (size_t)krow * D + (c < Lt::NCH ? c : 0) * 8;
      char* dst = buf + (isv ? Lt::KTILE : 0) + blk * 1024;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
    }
  }
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(KParams p) {
  using Lt = Layout<D>;
  constexpr int WGQ = NW * QW;
  constexpr float NEG_INF = -__builtin_huge_valf();
  __shared__ __attribute__((aligned(1024))) char buf0[Lt::BUF];
  __shared__ __attribute__((aligned(1024))) char buf1[Lt::BUF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, l32 = lane & 31;

  const int L = xcd_remap(blockIdx.x, p.total_wg);
  const int row = L / p.nsub, sub = L - row * p.nsub;
  const int h = row / p.nQ, qt = row - h * p.nQ;
  const int wg_q = qt * p.BQ + sub * WGQ;
  if (wg_q >= p.N) return;  // whole workgroup past a ragged last Q tile
  const int kind = p.kinds[h];

  const int32_t* ri = p.rowinfo + (size_t)row * kRowInfo;
  const int n_full = ri[0], n_tiles = ri[0] + ri[1], sa = ri[2], sb = ri[3];
  const int ebeg = p.row_ptr[row];
  const int n_tile_steps = n_tiles * p.cpt;
  const int n_s1 = (sa + CK - 1) / CK;
  const int n_steps = n_tile_steps + n_s1 + (p.S - sb + CK - 1) / CK;

  const size_t head_off = (size_t)h * p.N * D;
  const uint16_t* Qh = p.q + head_off;
  const uint16_t* Kh = p.k + head_off;
  const uint16_t* Vh = p.v + head_off;

  // Start the first K/V transfer before anything else.
  if (n_steps > 0)
    issue_loads<D, NW>(p, Kh, Vh, step_at(p, 0, n_tile_steps, n_full, ebeg, n_s1, sa, sb), buf0,
                       wave, lane);

  // ---- Q fragments (B operand of S^T = K Q^T) and this lane's mask bounds.
  const int q = wg_q + wave * QW + l32;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (q < p.N) x = *(const uint4*)(Qh + (size_t)q * D + ks * 16 + hl * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }
  int wlo = 0, whi = p.N, slim = 0;
  bool msink = false;
  if (kind == SVG_HEAD_SPATIAL) {
    const int f = q / p.S;
    wlo = max(0, f - p.W_f) * p.S;
    whi = min(p.F, f + p.W_f + 1) * p.S;
    slim = p.sink ? p.S : 0;
  } else if (kind == SVG_HEAD_TEMPORAL) {
    const int s = q / p.F;
    wlo = max(0, s - p.W_s) * p.F;
    whi = min(p.S, s + p.W_s + 1) * p.F;
    msink = p.sink != 0;
  }
  if (p.round_tile && kind != SVG_HEAD_DENSE) {
    // Tile-aligned mask: a pair is kept when its (BQ x BK) tile holds any pair
    // of the contiguous mask part, so the bound is the same for every row of
    // the map's Q tile: the union of its rows' windows (or bands), widened to
    // whole KV tiles; the spatial sink [0, S) is widened the same way and the
    // temporal strided sink stays exact.
    const int t0 = qt * p.BQ, t1 = min(p.N, t0 + p.BQ) - 1;
    if (kind == SVG_HEAD_SPATIAL) {
      wlo = max(0, t0 / p.S - p.W_f) * p.S;
      whi = min(p.F, t1 / p.S + p.W_f + 1) * p.S;
    } else {
      wlo = max(0, t0 / p.F - p.W_s) * p.F;
      whi = min(p.S, t1 / p.F + p.W_s + 1) * p.F;
    }
    wlo = wlo / p.BK * p.BK;
    whi = min(p.N, (whi + p.BK - 1) / p.BK * p.BK);
    if (slim > 0) slim = min(p.N, (slim + p.BK - 1) / p.BK * p.BK);
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m_ref = NEG_INF, l_sum = 0.f;

  // Per-lane LDS read bases (the rest of every address is a constant).
  const int g = lane >> 4, j16 = lane & 15;
  const int k_lane = l32 * Lt::KROW + 16 * hl;
  const int v_lane = Lt::KTILE + (8 * (g >> 1) + (j16 >> 2)) * Lt::VROW + 32 * (g & 1) +
                     8 * (j16 & 3);

  if (n_steps > 0) wait_dma();
  __syncthreads();

  // One step: compute on `cbuf` while the next step's K/V stream into
  // `nbuf`. The two buffers are distinct LDS objects and the loop is unrolled
  // by two, so the compiler can tell that the reads of this step never alias
  // the DMA in flight and does not wait for it before reading.
  auto run_step = [&](const char* cbuf, char* nbuf, int j) __attribute__((always_inline)) {
    const Step cur = step_at(p, j, n_tile_steps, n_full, ebeg, n_s1, sa, sb);
    if (j + 1 < n_steps)
      issue_loads<D, NW>(p, Kh, Vh, step_at(p, j + 1, n_tile_steps, n_full, ebeg, n_s1, sa, sb),
                         nbuf, wave, lane);

    // S^T = K Q^T: 64 keys x 32 queries
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
    const char* kp_lane = cbuf + k_lane;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *(const bf16x8*)(kp_lane + kb * 32 * Lt::KROW + ks * 32);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }

    // mask: column limit of short steps, head predicate on boundary tiles
    if (cur.pred) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kl = 32 * kb + 16 * (v >> 3) + 8 * hl + (v & 7);
          const int kp = cur.base + kl * cur.stride;
          const bool in = (kp >= wlo && kp < whi) || kp < slim || (msink && kp % p.F == 0);
          if (!(kl < cur.ncols && in)) s[kb][v] = NEG_INF;
        }
    }

    // online softmax, lazy rescaling
    float mx = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    {
      float a, b;
      halves(mx, a, b);
      mx = fmaxf(a, b);
    }
    const bool need = mx > m_ref + p.thr;
    if (__builtin_amdgcn_ballot_w64(need)) {
      float alpha = 1.f;
      if (need) {
        alpha = __builtin_amdgcn_exp2f((m_ref - mx) * p.c);
        m_ref = mx;
      }
      l_sum *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
    }
    const float mc = m_ref == NEG_INF ? 0.f : m_ref * p.c;
    bf16x8 pf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int v = 8 * (kk & 1) + 2 * t;
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][v], p.c, -mc));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][v + 1], p.c, -mc));
        l_sum += e0 + e1;
        w[t] = pack_bf16(e0, e1);
      }
      pf[kk] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }

    // O^T += V^T P^T
    const char* vp_lane = cbuf + v_lane;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vp_lane + (16 * kk) * Lt::VROW + 64 * db));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vp_lane + (16 * kk + 4) * Lt::VROW + 64 * db));
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], o[db], 0, 0, 0);
      }

    wait_dma();
    __syncthreads();
  };

  for (int j = 0; j < n_steps; j += 2) {
    run_step(buf0, buf1, j);
    if (j + 1 < n_steps) run_step(buf1, buf0, j + 1);
  }

  // ---- epilogue: O = O^T / l, bf16 (round to nearest even)
  float la, lb;
  halves(l_sum, la, lb);
  const float lt = la + lb;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (q < p.N) {
    uint16_t* orow = p.o + head_off + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 w;
        w.x = pack_bf16(o[db][4 * i + 0] * inv, o[db][4 * i + 1] * inv);
        w.y = pack_bf16(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
        *(uint2*)(orow + 32 * db + 8 * i + 4 * hl) = w;
      }
  }
}

int waves_for(int32_t tile_q) {
  if (tile_q % 256 == 0) return 8;
  if (tile_q == 128) return 4;
  if (tile_q == 64) return 2;
  if (tile_q == 32) return 1;
  return 0;
}

template <int D, int NW>
hipError_t launch(const KParams& kp, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW>), dim3(kp.total_wg), dim3(NW * 64), 0, stream, kp);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int nw, const KParams& kp, hipStream_t stream) {
  switch (nw) {
    case 8: return launch<D, 8>(kp, stream);
    case 4: return launch<D, 4>(kp, stream);
    case 2: return launch<D, 2>(kp, stream);
    default: return launch<D, 1>(kp, stream);
  }
}

}  // namespace

bool attn_supported(int32_t head_dim, int32_t tile_q, int32_t tile_k) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (waves_for(tile_q) == 0) return false;
  return tile_k >= 32 && tile_k <= 1024 && tile_k % 32 == 0;
}

hipError_t launch_attn_fwd(const MapGeometry& g, const MapBuffers& b, const AttnArgs& a,
                           hipStream_t stream) {
  if (!attn_supported(a.head_dim, g.BQ, g.BK)) return hipErrorInvalidValue;
  const int nw = waves_for(g.BQ);
  const int wgq = nw * QW;
  KParams kp;
  kp.q = (const uint16_t*)a.q;
  kp.k = (const uint16_t*)a.k;
  kp.v = (const uint16_t*)a.v;
  kp.o = (uint16_t*)a.o;
  kp.N = (int32_t)g.N;
  kp.F = g.F;
  kp.S = g.S;
  kp.W_f = g.W_f;
  kp.W_s = g.W_s;
  kp.sink = g.sink;
  kp.BQ = g.BQ;
  kp.BK = g.BK;
  kp.nQ = g.nQ;
  kp.nsub = g.BQ / wgq;
  kp.cpt = (g.BK + CK - 1) / CK;
  const int64_t total = (int64_t)g.H * g.nQ * kp.nsub;
  if (total > INT32_MAX) return hipErrorInvalidConfiguration;
  kp.total_wg = (int32_t)total;
  kp.kinds = b.kinds;
  kp.rowinfo = b.rowinfo;
  kp.row_ptr = b.row_ptr;
  kp.entries = b.entries;
  kp.c = a.scale * 1.4426950408889634f;
  kp.thr = 8.0f / kp.c;
  kp.mask_all = (a.flags & SVG_ATTN_MASK_ALL_TILES) ? 1 : 0;
  kp.round_tile = g.round == SVG_ROUND_TILE ? 1 : 0;
  if (kp.total_wg <= 0) return hipSuccess;
  return a.head_dim == 128 ? launch_d<128>(nw, kp, stream) : launch_d<64>(nw, kp, stream);
}

}  // namespace svg
