// Structured-sparse attention forward for gfx950 (MI355X).
//
// One workgroup computes WGQ query rows of one head (a slice of one map Q
// tile) against the KV tiles its schedule lists: FULL tiles ascending
// (mask-free), BOUNDARY tiles ascending (per-element predicate), then -- for
// temporal heads -- the frame-0 sink keys outside the band hull, read at
// stride F rows (mask-free). This is the full/boundary split of the pages'
// kernel ("Google Speeds Up Video Diffusion on TPUs with Optimized Sparse
// Attention", "Efficient Kernel Implementation"; Newsbite "Summary").
//
// Per 64-key step the kernel computes the transposed score block
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, Q
// held in VGPRs as the B operand). In that layout every lane owns whole query
// columns, so the online-softmax row max / sum are in-lane, plus one exchange
// between the two 32-lane halves. The probabilities P^T stay in registers and
// feed O^T += V^T P^T directly as the B operand; V is staged to LDS
// transposed so that its A operand is one 16-byte LDS read. The row maximum
// is refreshed lazily: O and the row sum are rescaled only when a new
// maximum exceeds the reference by more than 2^8 (exact: the final O / l is
// unchanged by the choice of reference, and exp2 values stay below 2^8).
// K and V steps are double-buffered in LDS with global loads issued one step
// ahead. Workgroups are remapped so that consecutive Q tiles of a head run on
// the same XCD and share its L2.
#include "svg_internal.hpp"

#include <math.h>

namespace svg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int CK = 64;  // keys per pipeline step

struct KParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int32_t N, F, S, W_f, W_s, sink;
  int32_t BQ, BK, nQ, nsub, total_wg;
  const int32_t* kinds;
  const int32_t* rowinfo;
  const int32_t* row_ptr;
  const int32_t* entries;
  float c;       // scale * log2(e)
  float thr;     // lazy-rescale threshold in raw score units
  int32_t mask_all;
  int32_t round_tile;  // the map rounds the contiguous mask part to whole tiles
};

struct Step {
  int32_t base;    // kernel-layout row of the step's first key
  int32_t stride;  // rows between consecutive keys (1, or F for sink keys)
  int32_t ncols;   // valid keys in this step (<= CK; <= 0 possible)
  int32_t pred;    // evaluate the head mask per element
};

// Lane m of a 32-row A operand loads key row sigma(m), so that accumulator v
// of a 32x32 MFMA output holds key 16*(v/8) + 8*(lane/32) + v%8: each lane's
// 8 consecutive accumulators are 8 consecutive keys, which is exactly the
// B-operand slice the P^T V^T product needs from that lane.
__device__ __forceinline__ int sigma(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

template <int D>
__device__ __forceinline__ int kswz(int row) { return row & (D / 8 - 1); }
__device__ __forceinline__ int vswz(int d) { return d & (CK / 8 - 1); }

__device__ __forceinline__ int xcd_remap(int i, int T) {
  const int x = i & 7, j = i >> 3, per = T >> 3, rem = T & 7;
  return x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

__device__ __forceinline__ uint32_t half_of(const uint4& x, int e) {
  uint32_t word;
  switch (e >> 1) {
    case 0: word = x.x; break;
    case 1: word = x.y; break;
    case 2: word = x.z; break;
    default: word = x.w; break;
  }
  return (e & 1) ? (word >> 16) : (word & 0xffffu);
}

template <int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(KParams p) {
  constexpr int NT = NW * 64;
  constexpr int WGQ = NW * QB * 32;
  constexpr int DC = D / 8;                 // 16-byte chunks per row
  constexpr int KSEG = CK * DC / NT;        // K 16-byte segments per thread
  constexpr int VUNITS = (CK / 4) * DC;     // V units of 4 keys x 8 dims
  constexpr int VUPT = (VUNITS + NT - 1) / NT;  // V units per thread (last may idle)
  static_assert(KSEG >= 1 && (CK * DC) % NT == 0, "K step must split evenly");
  constexpr float NEG_INF = -__builtin_huge_valf();

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][CK * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * CK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;

  const int L = xcd_remap(blockIdx.x, p.total_wg);
  const int row = L / p.nsub, sub = L - row * p.nsub;
  const int h = row / p.nQ, qt = row - h * p.nQ;
  const int q_start = qt * p.BQ + sub * WGQ;
  if (q_start >= p.N) return;
  const int kind = p.kinds[h];

  const int32_t* ri = p.rowinfo + (size_t)row * kRowInfo;
  const int n_full = ri[0], n_tiles = ri[0] + ri[1], sa = ri[2], sb = ri[3];
  const int ebeg = p.row_ptr[row];
  const int cpt = (p.BK + CK - 1) / CK;
  const int n_tile_steps = n_tiles * cpt;
  const int n_s1 = (sa + CK - 1) / CK;
  const int n_steps = n_tile_steps + n_s1 + (p.S - sb + CK - 1) / CK;

  auto step_at = [&](int j) -> Step {
    Step s;
    if (j < n_tile_steps) {
      const int e = j / cpt, part = j - e * cpt;
      const int kt = p.entries[ebeg + e];
      const int c0 = kt * p.BK + part * CK;
      const int end = min(p.N, kt * p.BK + p.BK);
      s.base = c0;
      s.stride = 1;
      s.ncols = min(CK, end - c0);
      s.pred = (e >= n_full) | p.mask_all;
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
      s.pred = p.mask_all;
    }
    return s;
  };

  const size_t head_off = (size_t)h * p.N * D;
  const uint16_t* Qh = p.q + head_off;
  const uint16_t* Kh = p.k + head_off;
  const uint16_t* Vh = p.v + head_off;

  // ---- Q fragments (B operand of S^T = K Q^T) and per-query mask bounds.
  bf16x8 qf[QB][D / 16];
  int qpos[QB], win_lo[QB], win_hi[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qpos[qb] = q_start + (wave * QB + qb) * 32 + l32;
    const bool ok = qpos[qb] < p.N;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (ok) x = *(const uint4*)(Qh + (size_t)qpos[qb] * D + ks * 16 + hl * 8);
      qf[qb][ks] = __builtin_bit_cast(bf16x8, x);
    }
    if (kind == SVG_HEAD_SPATIAL) {
      const int f = qpos[qb] / p.S;
      win_lo[qb] = max(0, f - p.W_f) * p.S;
      win_hi[qb] = min(p.F, f + p.W_f + 1) * p.S;
    } else if (kind == SVG_HEAD_TEMPORAL) {
      const int s = qpos[qb] / p.F;
      win_lo[qb] = max(0, s - p.W_s) * p.F;
      win_hi[qb] = min(p.S, s + p.W_s + 1) * p.F;
    } else {
      win_lo[qb] = 0;
      win_hi[qb] = p.N;
    }
  }
  int sink_lim = (kind == SVG_HEAD_SPATIAL && p.sink) ? p.S : 0;
  const bool sink_mod = kind == SVG_HEAD_TEMPORAL && p.sink;
  if (p.round_tile && kind != SVG_HEAD_DENSE) {
    // Tile-aligned mask: a pair is kept when its (BQ x BK) tile holds any pair
    // of the contiguous mask part, so the bound is the same for every row of
    // the map's Q tile: the union of its rows' windows (or bands), widened to
    // whole KV tiles; the spatial sink [0, S) is widened the same way and the
    // temporal strided sink stays exact.
    const int t0 = qt * p.BQ, t1 = min(p.N, t0 + p.BQ) - 1;
    int lo, hi;
    if (kind == SVG_HEAD_SPATIAL) {
      lo = max(0, t0 / p.S - p.W_f) * p.S;
      hi = min(p.F, t1 / p.S + p.W_f + 1) * p.S;
    } else {
      lo = max(0, t0 / p.F - p.W_s) * p.F;
      hi = min(p.S, t1 / p.F + p.W_s + 1) * p.F;
    }
    lo = lo / p.BK * p.BK;
    hi = min(p.N, (hi + p.BK - 1) / p.BK * p.BK);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      win_lo[qb] = lo;
      win_hi[qb] = hi;
    }
    if (sink_lim > 0) sink_lim = min(p.N, (sink_lim + p.BK - 1) / p.BK * p.BK);
  }

  f32x16 o[D / 32][QB];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][qb][v] = 0.f;
  float m_ref[QB], l_sum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = NEG_INF;
    l_sum[qb] = 0.f;
  }

  // ---- staging: global -> registers -> LDS
  uint4 kst[KSEG];
  uint4 vst[VUPT * 4];
  auto load_step = [&](const Step& s) {
#pragma unroll
    for (int i = 0; i < KSEG; ++i) {
      const int g = tid + NT * i;
      const int r = g / DC, cc = g % DC;
      const int kr = r < s.ncols ? r : 0;
      const int pos = min(s.base + kr * s.stride, p.N - 1);
      kst[i] = *(const uint4*)(Kh + (size_t)pos * D + cc * 8);
    }
#pragma unroll
    for (int i = 0; i < VUPT; ++i) {
      const int u = tid + NT * i;
      if (VUNITS % NT != 0 && u >= VUNITS) break;
      const int kg = u / DC, dc = u % DC;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = 4 * kg + r;
        const int kr = rr < s.ncols ? rr : 0;
        const int pos = min(s.base + kr * s.stride, p.N - 1);
        vst[4 * i + r] = *(const uint4*)(Vh + (size_t)pos * D + dc * 8);
      }
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KSEG; ++i) {
      const int g = tid + NT * i;
      const int r = g / DC, cc = g % DC;
      *(uint4*)&Ks[buf][r * D + ((cc ^ kswz<D>(r)) * 8)] = kst[i];
    }
#pragma unroll
    for (int i = 0; i < VUPT; ++i) {
      const int u = tid + NT * i;
      if (VUNITS % NT != 0 && u >= VUNITS) break;
      const int kg = u / DC, dc = u % DC;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = dc * 8 + e;
        uint2 w;
        w.x = half_of(vst[4 * i + 0], e) | (half_of(vst[4 * i + 1], e) << 16);
        w.y = half_of(vst[4 * i + 2], e) | (half_of(vst[4 * i + 3], e) << 16);
        *(uint2*)&Vt[buf][d * CK + (((kg >> 1) ^ vswz(d)) * 8) + (kg & 1) * 4] = w;
      }
    }
  };

  if (n_steps > 0) {
    load_step(step_at(0));
    store_step(0);
  }
  __syncthreads();

  for (int j = 0; j < n_steps; ++j) {
    const Step cur = step_at(j);
    const bool has_next = j + 1 < n_steps;
    if (has_next) load_step(step_at(j + 1));
    const uint16_t* Kb = Ks[j & 1];
    const uint16_t* Vb = Vt[j & 1];

    // S^T = K Q^T for 64 keys x WGQ/NW queries
    f32x16 s[CK / 32][QB];
#pragma unroll
    for (int kb = 0; kb < CK / 32; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][qb][v] = 0.f;
      const int kr = kb * 32 + sigma(l32);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int ch = 2 * ks + hl;
        const bf16x8 a = *(const bf16x8*)&Kb[kr * D + ((ch ^ kswz<D>(kr)) * 8)];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], s[kb][qb], 0, 0, 0);
      }
    }

    // masking: column limit of ragged steps, head predicate on boundary tiles
    if (cur.pred || cur.ncols < CK) {
#pragma unroll
      for (int kb = 0; kb < CK / 32; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kl = kb * 32 + 16 * (v >> 3) + 8 * hl + (v & 7);
          const int kp = cur.base + kl * cur.stride;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            bool keep = kl < cur.ncols;
            if (cur.pred) {
              const bool in_win = kp >= win_lo[qb] && kp < win_hi[qb];
              keep = keep && (in_win || kp < sink_lim || (sink_mod && (kp % p.F) == 0));
            }
            if (!keep) s[kb][qb][v] = NEG_INF;
          }
        }
    }

    // online softmax with lazy rescaling
    bool any_rescale = false;
    float alpha[QB], mc[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < CK / 32; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][qb][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const bool need = mx > m_ref[qb] + p.thr;
      alpha[qb] = 1.f;
      if (need) {
        alpha[qb] = __builtin_amdgcn_exp2f((m_ref[qb] - mx) * p.c);
        m_ref[qb] = mx;
      }
      any_rescale |= need;
      mc[qb] = m_ref[qb] == NEG_INF ? 0.f : m_ref[qb] * p.c;
    }
    if (__ballot(any_rescale)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_sum[qb] *= alpha[qb];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[db][qb][v] *= alpha[qb];
      }
    }

    // P^T = exp2(S^T * c - m c), then O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < CK / 32; ++kb) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        bf16x8 pb[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][8 * g + t], p.c, -mc[qb]));
            l_sum[qb] += e;
            pb[qb][t] = (__bf16)e;
          }
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int d = db * 32 + l32;
          const int ch = 4 * kb + 2 * g + hl;
          const bf16x8 a = *(const bf16x8*)&Vb[d * CK + ((ch ^ vswz(d)) * 8)];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb], o[db][qb], 0, 0, 0);
        }
      }
    }

    if (has_next) store_step((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, bf16 (round to nearest even)
  uint16_t* Oh = p.o + head_off;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_sum[qb] + __shfl_xor(l_sum[qb], 32, 64);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qpos[qb] < p.N) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int d = db * 32 + 8 * v4 + 4 * hl;
          uint2 w;
          const __bf16 b0 = (__bf16)(o[db][qb][4 * v4 + 0] * inv);
          const __bf16 b1 = (__bf16)(o[db][qb][4 * v4 + 1] * inv);
          const __bf16 b2 = (__bf16)(o[db][qb][4 * v4 + 2] * inv);
          const __bf16 b3 = (__bf16)(o[db][qb][4 * v4 + 3] * inv);
          w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
          w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
          *(uint2*)(Oh + (size_t)qpos[qb] * D + d) = w;
        }
    }
  }
}

struct Config {
  int nw, qb;
};

Config pick_config(int32_t tile_q) {
  if (tile_q % 256 == 0) return {4, 2};
  if (tile_q == 128) return {2, 2};
  if (tile_q == 64) return {1, 2};
  if (tile_q == 32) return {1, 1};
  return {0, 0};
}

template <int D, int NW, int QB>
hipError_t launch(const KParams& kp, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW, QB>), dim3(kp.total_wg), dim3(NW * 64), 0,
                     stream, kp);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Config& c, const KParams& kp, hipStream_t stream) {
  if (c.nw == 4) return launch<D, 4, 2>(kp, stream);
  if (c.nw == 2) return launch<D, 2, 2>(kp, stream);
  if (c.qb == 2) return launch<D, 1, 2>(kp, stream);
  return launch<D, 1, 1>(kp, stream);
}

}  // namespace

bool attn_supported(int32_t head_dim, int32_t tile_q, int32_t tile_k) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (pick_config(tile_q).nw == 0) return false;
  return tile_k >= 32 && tile_k <= 1024 && tile_k % 32 == 0;
}

hipError_t launch_attn_fwd(const MapGeometry& g, const MapBuffers& b, const AttnArgs& a,
                           hipStream_t stream) {
  if (!attn_supported(a.head_dim, g.BQ, g.BK)) return hipErrorInvalidValue;
  const Config c = pick_config(g.BQ);
  const int wgq = c.nw * c.qb * 32;
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
  return a.head_dim == 128 ? launch_d<128>(c, kp, stream) : launch_d<64>(c, kp, stream);
}

}  // namespace svg
