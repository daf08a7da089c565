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
//   O^T += V^T P^T V^T from LDS (A), P^T from VGPRs (B).
// The row maximum is refreshed lazily: O and the row sum are rescaled only
// when a new maximum exceeds the reference by more than 8 in log2 units, so
// exp2 values stay below 2^8 and the final O / l is unchanged.
//
// Staging. The LDS issues about one wave-wide read every six cycles whatever
// its width, so both MFMA operands are read with ds_read_b128 (16 per step
// each for K and V^T). K moves from HBM straight into LDS (buffer_load ...
// lds, no VGPRs). V is stored transposed: each lane loads 8 keys x 2 dims
// with dword buffer loads, transposes them with v_perm_b32 and writes two
// 16-byte V^T rows; strided sink keys take the same path. Both are
// double-buffered: the transfers for step j+1 are in flight while step j
// computes. LDS rows are padded (K 272 bytes, V^T 144) so that 16 lanes
// reading 16 consecutive rows at one column hit 16 distinct 4-bank groups of
// the 64 banks, and every read address is a per-lane base plus a constant.
// K rows are stored in the order the S^T accumulator layout needs for P^T to
// be the B operand of the PV product as it stands. Workgroups are remapped so
// that consecutive Q tiles of a head run on the same XCD and share its L2.
#include "svg_internal.hpp"

#include <math.h>

namespace svg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int CK = 64;  // keys per pipeline step
constexpr int QW = 32;  // query rows per wave

template <int D, int NW>
struct Layout {
  static constexpr int NCH = D / 8;              // 16-byte chunks per K row
  static constexpr int KSLOTS = NCH + 1;         // K row + one pad slot
  static constexpr int KROW = 16 * KSLOTS;       // bytes per K row in LDS
  static constexpr int KTILE = CK * KROW;
  static constexpr int KLOADS = KTILE / 1024;    // 1 KiB wave-wide DMA loads
  static constexpr int KPW = (KLOADS + NW - 1) / NW;  // DMA loads per wave
  static constexpr int VTROW = 16 * (CK / 8 + 1);     // bytes per V^T row (one dim)
  static constexpr int VTILE = D * VTROW;
  static constexpr int BUF = KTILE + VTILE;
  // V transpose units: 8 keys x 2 dims, one per lane and round
  static constexpr int VUNITS = (CK / 8) * (D / 2);
  static constexpr int VUPL = (VUNITS + NW * 64 - 1) / (NW * 64);  // units per lane
  static_assert(KTILE % 1024 == 0, "K tile must be whole KiB");
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

// Descriptor of step j: `part` (0..cpt-1) of tile `kt` when `tile`, else
// sink step js = j - (tile steps) of a temporal head: raster indices [0, a)
// then [b, S), 64 per step, read at rows s * F.
__device__ __forceinline__ Step make_step(const KParams& p, bool tile, bool bnd, int kt,
                                          int part, int js, int n_s1, int sa, int sb) {
  Step s;
  if (tile) {
    const int c0 = kt * p.BK + part * CK;
    const int end = min(p.N, kt * p.BK + p.BK);
    s.base = c0;
    s.stride = 1;
    s.ncols = min(CK, end - c0);
    s.pred = bnd | p.mask_all | (s.ncols < CK);
  } else {
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

// Row of key r (0..63) of a step, clamped into the sequence (keys past
// `ncols` are masked; their row only has to be readable).
__device__ __forceinline__ int key_row(const KParams& p, const Step& s, int r) {
  return min(s.base + (r < s.ncols ? r : 0) * s.stride, p.N - 1);
}

// Staging of one step's K (DMA into LDS) and V (dword loads into VGPRs, then
// transposed into LDS). The (row, chunk) a lane fetches is fixed per load, so
// its byte offset from the step's first row is computed once, for
// consecutive rows and for rows F apart (sink steps). Full steps then pass
// those persistent registers as they are and put everything that changes in
// the scalar offset: no address register is rewritten while its load is in
// flight, which would make the compiler wait for the loads before the next
// LDS read. Short steps (ragged tails) clamp rows per lane and wait for their
// loads at once (rare). K pad slots re-read chunk 0 of their row (in bounds,
// never read back).
template <int D, int NW>
struct Stage {
  using Lt = Layout<D, NW>;
  static constexpr int ROWB = 2 * D;  // bytes per K/V row in HBM
  static constexpr int SH = D == 128 ? 8 : 7;
  uint32_t koff[Lt::KPW], koffF[Lt::KPW];    // K: offsets, rows 1 / F apart
  uint32_t voff[Lt::VUPL], voffF[Lt::VUPL];  // V: offset of key 0 of the unit
  uint32_t vx[Lt::VUPL][8];                  // V: 8 keys x 2 dims in flight

  __device__ __forceinline__ void init(int wave, int lane, int F) {
#pragma unroll
    for (int i = 0; i < Lt::KPW; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int prow = slot / Lt::KSLOTS, c = slot - prow * Lt::KSLOTS;
      const int r = (prow & ~31) | sigma(prow & 31);
      const int cb = 16 * (c < Lt::NCH ? c : 0);
      koff[i] = (uint32_t)(r * ROWB + cb);
      koffF[i] = (uint32_t)(r * F * ROWB + cb);
    }
#pragma unroll
    for (int u = 0; u < Lt::VUPL; ++u) {
      const int unit = u * NW * 64 + wave * 64 + lane;
      const int dp = unit % (D / 2), kg = unit / (D / 2);
      voff[u] = (uint32_t)(8 * kg * ROWB + 4 * dp);
      voffF[u] = (uint32_t)(8 * kg * F * ROWB + 4 * dp);
    }
  }

  __device__ __forceinline__ bool unit_ok(int u, int wave, int lane) const {
    return Lt::VUNITS % (NW * 64) == 0 || u * NW * 64 + wave * 64 + lane < Lt::VUNITS;
  }
  __device__ __forceinline__ bool k_ok(int i, int wave) const {
    return Lt::KLOADS % NW == 0 || i * NW + wave < Lt::KLOADS;
  }

  // Full step with fixed per-lane offsets `ko` / `vo` and key pitch `pitch`
  // bytes (ROWB or F * ROWB).
  __device__ __forceinline__ void issue_full(const char* kbase,
                                             __amdgpu_buffer_rsrc_t vrs, uint32_t base,
                                             uint32_t pitch, const uint32_t (&ko)[Lt::KPW],
                                             const uint32_t (&vo)[Lt::VUPL], char* buf,
                                             int wave, int lane) {
    const char* kb = kbase + base;
#pragma unroll
    for (int i = 0; i < Lt::KPW; ++i)
      if (k_ok(i, wave))
        __builtin_amdgcn_global_load_lds(kb + ko[i], (lds_void*)(buf + (i * NW + wave) * 1024), 16,
                                         0, 0);
#pragma unroll
    for (int u = 0; u < Lt::VUPL; ++u)
      if (unit_ok(u, wave, lane)) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
          vx[u][r] = __builtin_amdgcn_raw_buffer_load_b32(vrs, vo[u], base + r * pitch, 0);
      }
  }

  // Queue step `s`: K DMA into `buf`, V loads into vx.
  __device__ __forceinline__ void issue(const KParams& p, const char* kbase,
                                        __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                        const Step& s, char* buf, int wave, int lane) {
    const uint32_t base = (uint32_t)s.base * ROWB;
    if (s.ncols == CK && s.stride == 1) {
      issue_full(kbase, vrs, base, ROWB, koff, voff, buf, wave, lane);
    } else if (s.ncols == CK) {
      issue_full(kbase, vrs, base, (uint32_t)p.F * ROWB, koffF, voffF, buf, wave, lane);
    } else {
#pragma unroll
      for (int i = 0; i < Lt::KPW; ++i)
        if (k_ok(i, wave)) {
          const int r = (int)(koff[i] >> SH);
          const uint32_t off = (uint32_t)key_row(p, s, r) * ROWB + (koff[i] & (ROWB - 1));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              krs, (lds_void*)(buf + (i * NW + wave) * 1024), 16, off, 0, 0, 0);
        }
#pragma unroll
      for (int u = 0; u < Lt::VUPL; ++u)
        if (unit_ok(u, wave, lane)) {
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const int kr = (int)(voff[u] >> SH) + r;
            const uint32_t off = (uint32_t)key_row(p, s, kr) * ROWB + (voff[u] & (ROWB - 1));
            vx[u][r] = __builtin_amdgcn_raw_buffer_load_b32(vrs, off, 0, 0);
          }
        }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the temporaries are free again
    }
  }

  // Transpose the staged V (after its loads completed) into V^T in `buf`.
  __device__ __forceinline__ void store_vt(char* buf, int wave, int lane) const {
#pragma unroll
    for (int u = 0; u < Lt::VUPL; ++u) {
      if (unit_ok(u, wave, lane)) {
        const int unit = u * NW * 64 + wave * 64 + lane;
        const int dp = unit % (D / 2), kg = unit / (D / 2);
        uint4 lo, hi;  // dims 2dp and 2dp+1, keys 8kg .. 8kg+7
        lo.x = __builtin_amdgcn_perm(vx[u][1], vx[u][0], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(vx[u][3], vx[u][2], 0x05040100u);
        lo.z = __builtin_amdgcn_perm(vx[u][5], vx[u][4], 0x05040100u);
        lo.w = __builtin_amdgcn_perm(vx[u][7], vx[u][6], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(vx[u][1], vx[u][0], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(vx[u][3], vx[u][2], 0x07060302u);
        hi.z = __builtin_amdgcn_perm(vx[u][5], vx[u][4], 0x07060302u);
        hi.w = __builtin_amdgcn_perm(vx[u][7], vx[u][6], 0x07060302u);
        char* vt = buf + Lt::KTILE + 2 * dp * Lt::VTROW + 16 * kg;
        *(uint4*)vt = lo;
        *(uint4*)(vt + Lt::VTROW) = hi;
      }
    }
  }
};

// Walks the steps of one schedule row in order. The row's KV tile ids are
// read 64 at a time into one VGPR per wave (lane i holds entry 64 * chunk +
// i), the next 64 prefetched, and picked with v_readlane: no memory round
// trip on the step path. The (entry, part) position advances one step at a
// time.
struct Cursor {
  const int32_t* ents;  // the row's tile ids
  int n_tiles, n_full, n_s1, sa, sb;
  int chunk, e, part, js;
  int e_cur, e_nxt;

  __device__ __forceinline__ int load(int c, int lane) const {
    const int idx = c * 64 + lane;
    return idx < n_tiles ? ents[idx] : 0;
  }
  __device__ __forceinline__ void init(const int32_t* row_ents, int nt, int nf, int ns1, int a,
                                       int b, int lane) {
    ents = row_ents;
    n_tiles = nt;
    n_full = nf;
    n_s1 = ns1;
    sa = a;
    sb = b;
    chunk = e = part = js = 0;
    e_cur = load(0, lane);
    e_nxt = load(1, lane);
  }
  // descriptor of the current step; the cursor moves one step on
  __device__ __forceinline__ Step take(const KParams& p, int lane) {
    const bool tile = e < n_tiles;
    int kt = 0;
    if (tile) {
      if ((e >> 6) != chunk) {  // entries are visited in order: next chunk
        e_cur = e_nxt;
        ++chunk;
        e_nxt = load(chunk + 1, lane);
      }
      kt = __builtin_amdgcn_readlane(e_cur, __builtin_amdgcn_readfirstlane(e & 63));
    }
    const Step st = make_step(p, tile, e >= n_full, kt, part, js, n_s1, sa, sb);
    if (tile) {
      if (++part == p.cpt) {
        part = 0;
        ++e;
      }
    } else {
      ++js;
    }
    return st;
  }
};

// vmcnt(0), as an instruction the compiler accounts for
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(KParams p) {
  using Lt = Layout<D, NW>;
  constexpr int WGQ = NW * QW;
  constexpr int NS = 2 * (D / 16);  // MFMAs of S^T per step: (d-step, key block)
  constexpr int NDB = D / 32;       // 32-row blocks of O^T
  constexpr int NPV = 4 * NDB;      // MFMAs of O^T per step: (16-key step, d block)
  constexpr int PD = 4;             // LDS operand prefetch depth, in MFMAs
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
  const int head_bytes = p.N * D * 2;
  const char* kbytes = (const char*)(p.k + head_off);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + head_off), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + head_off), (short)0, head_bytes, 0x00020000);

  Stage<D, NW> stg;
  stg.init(wave, lane, p.F);
  // Start the first K/V transfer before anything else.
  Cursor cur_pos;
  cur_pos.init(p.entries + ebeg, n_tiles, n_full, n_s1, sa, sb, lane);
  Step nxt = {0, 1, 0, 0};
  if (n_steps > 0) {
    nxt = cur_pos.take(p, lane);
    stg.issue(p, kbytes, krs, vrs, nxt, buf0, wave, lane);
  }

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

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m_ref = NEG_INF, l_sum = 0.f;

  // Per-lane LDS read bases (the rest of every address is a constant).
  const int k_lane = l32 * Lt::KROW + 16 * hl;
  const int v_lane = Lt::KTILE + l32 * Lt::VTROW + 16 * hl;
  // A operand of S^T MFMA i (d-step i/2, key block i%2): 32 keys x 16 dims.
  auto kread = [&](const char* kb, int i) __attribute__((always_inline)) {
    return *(const bf16x8*)(kb + (i & 1) * 32 * Lt::KROW + (i >> 1) * 32);
  };
  // A operand of O^T MFMA i (16-key step i/NDB, d block i%NDB): 32 dims x 16
  // keys, 8 consecutive keys of one dim per lane.
  auto vread = [&](const char* vb, int i) __attribute__((always_inline)) {
    const int kk = i / NDB, db = i % NDB;
    return *(const bf16x8*)(vb + 32 * db * Lt::VTROW + 32 * kk);
  };

  if (n_steps > 0) {
    wait_vmem();
    stg.store_vt(buf0, wave, lane);
  }
  __syncthreads();

  // One step: compute on `cbuf` while the next step's K/V stream towards
  // `nbuf`. The two buffers are distinct LDS objects and the loop is unrolled
  // by two, so the compiler can tell that the reads of this step never alias
  // the DMA in flight and does not wait for it before reading.
  auto run_step = [&](const char* cbuf, char* nbuf, int j) __attribute__((always_inline)) {
    const Step cur = nxt;
    const bool more = j + 1 < n_steps;
    if (more) {
      nxt = cur_pos.take(p, lane);
      stg.issue(p, kbytes, krs, vrs, nxt, nbuf, wave, lane);
    }

    // S^T = K Q^T: 64 keys x 32 queries, K operands read PD MFMAs ahead; the
    // first V operands load under the last MFMAs.
    const char* kb = cbuf + k_lane;
    const char* vb = cbuf + v_lane;
    f32x16 s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb2][v] = 0.f;
    bf16x8 ka[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) ka[i] = kread(kb, i);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const bf16x8 a = ka[i % PD];
      if (i + PD < NS) ka[i % PD] = kread(kb, i + PD);
      s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i >> 1], s[i & 1], 0, 0, 0);
    }
    bf16x8 va[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) va[i] = vread(vb, i);
    // Keep the reads ahead of their MFMAs (the default schedule assumes a
    // far shorter LDS latency): transfers first, PD K reads, one K read per
    // MFMA, then the first V operands under the last MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x020, Lt::KPW + 8 * Lt::VUPL, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, PD, 0);
#pragma unroll
    for (int i = 0; i < NS - PD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }

    // mask: column limit of short steps, head predicate on boundary tiles.
    // The keep bits of the lane's 32 keys are built in a rolled loop (small
    // code, rare path), then applied.
    if (cur.pred) {
      uint32_t keep = 0;
#pragma nounroll
      for (int e = 0; e < 32; ++e) {
        const int kl = 32 * (e >> 4) + 16 * ((e >> 3) & 1) + 8 * hl + (e & 7);
        const int kp = cur.base + kl * cur.stride;
        const bool in = (kp >= wlo && kp < whi) || kp < slim || (msink && kp % p.F == 0);
        keep |= (uint32_t)(kl < cur.ncols && in) << e;
      }
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (!((keep >> (16 * kb2 + v)) & 1u)) s[kb2][v] = NEG_INF;
    }

    // online softmax, lazy rescaling
    float mx = NEG_INF;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb2][v]);
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
      for (int db = 0; db < NDB; ++db)
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

    // O^T += V^T P^T, V operands read PD MFMAs ahead
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const bf16x8 a = va[i % PD];
      if (i + PD < NPV) va[i % PD] = vread(vb, i + PD);
      o[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[i / NDB], o[i % NDB], 0, 0, 0);
    }

    // the next step's V arrived during this step: transpose it into LDS
    wait_vmem();
    if (more) stg.store_vt(nbuf, wave, lane);
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
    for (int db = 0; db < NDB; ++db)
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
