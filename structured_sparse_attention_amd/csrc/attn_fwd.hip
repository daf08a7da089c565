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
// Schedule. A wave cannot overlap its own MFMAs with its own VALU work, but
// the two waves of a SIMD can overlap each other's. With eight waves the
// workgroup forms two groups, one wave of each per SIMD, and every step has
// two phases: while group 0 runs the MFMA phase of step t (PV of step t-1,
// then S^T of step t), group 1 runs the softmax of step t-1; then group 0
// runs the softmax of step t while group 1 runs its MFMA phase. Only a
// barrier at the end of the step synchronises the groups (the phases share
// no LDS data), so when one phase runs short the two waves of a SIMD share
// the matrix pipe instead of one of them waiting. All memory work rides in
// the wave that is otherwise idle between MFMAs: group 0 issues the next
// step's loads inside its MFMA phase, group 1 transposes V (reads during its
// softmax, writes during its MFMA phase). With fewer waves every wave runs
// both phases in turn.
//
// Staging. K rows and V rows move from HBM straight into LDS (buffer_load
// ... lds, no VGPRs), one step ahead, into two buffers used in turn. V is
// transposed once per step inside LDS (ds_read_b64_tr_b16, then 16-byte
// writes) so that both MFMA operands are read with ds_read_b128: the LDS
// issues about one wave-wide read every four cycles whatever its width. LDS
// rows are padded (272 bytes, and 144 for V^T) so that 16 lanes reading 16
// consecutive rows at one column hit 16 distinct 4-bank groups of the 64
// banks. K rows are stored in the order the S^T accumulator layout needs for
// P^T to be the B operand of the PV product as it stands; V rows in an order
// that keeps the transposing reads free of bank conflicts. A step's first
// row is folded into the base of its buffer resources, so the loads need no
// per-lane address arithmetic and rows past the sequence read as zeros.
//
// Dispatch. The launch is persistent: one workgroup per compute unit, each
// taking work items from its XCD's queue of the map's plan (plan.hpp), and
// then from a tail shared by all XCDs: a work item is a range of steps of
// one workgroup-sized slice of a schedule row. The plan keeps the Q tiles an
// XCD works on at one time neighbours (they share their KV tiles in its L2)
// and ends the XCD's workgroups level by cutting its last rows between them;
// the shared tail, cut into parts that shrink towards its end, evens out
// XCDs that run at different speeds. A cut row's parts write their
// unnormalised O, running maximum and row sum to partial slots, and
// combine_kernel merges them after the launch.
#include "svg_internal.hpp"

#include <math.h>
#include <stddef.h>

#include <type_traits>

namespace svg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int CK = 64;  // keys per pipeline step
constexpr int QW = 32;  // query rows per wave

template <int D, int NW>
struct Layout {
  static constexpr int NCH = D / 8;              // 16-byte chunks per K/V row
  static constexpr int KSLOTS = NCH + 1;         // row + one pad slot
  static constexpr int KROW = 16 * KSLOTS;       // bytes per K/V row in LDS
  static constexpr int KTILE = CK * KROW;        // one step's K rows (and V rows)
  static constexpr int KLOADS = KTILE / 1024;    // 1 KiB wave-wide DMA loads per tile
  static constexpr int VTROW = 16 * (CK / 8 + 1);  // bytes per V^T row (one dim)
  static constexpr int VTILE = D * VTROW;
  // One buffer: K rows | V^T | V rows.
  static constexpr int VT_OFF = KTILE;
  static constexpr int VR_OFF = KTILE + VTILE;
  static constexpr int BUF = 2 * KTILE + VTILE;
  // With eight waves, group 0 (waves 0-3) issues every HBM load and group 1
  // (waves 4-7) transposes V; with fewer waves every wave does both.
  static constexpr int NL = NW == 8 ? NW / 2 : NW;  // loader waves
  static constexpr int NT = NW == 8 ? NW / 2 : NW;  // transposer waves
  static constexpr int LPW = (KLOADS + NL - 1) / NL;  // K (and V) loads per loader wave
  static constexpr int TCH = D * (CK / 8);            // V^T chunks (8 keys x 1 dim) per step
  static constexpr int TPW = TCH / (NT * 64);         // chunks per transposer lane
  static_assert(KTILE % 1024 == 0, "K tile must be whole KiB");
  static_assert(TCH % (NT * 64) == 0, "V^T chunks must split evenly over the lanes");
  static_assert(VR_OFF % 1024 == 0, "DMA destinations must stay 1 KiB aligned");
};

struct KParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int32_t N, F, S, W_f, W_s, sink;
  int32_t BQ, BK, nQ, nsub, cpt;
  const int32_t* entries;
  const int32_t* item_ptr;  // queue bounds [n_xcd + 2]: XCD x's queue, then the shared tail
  const int4* items;        // ItemDesc, three int4 each (see svg_internal.hpp)
  int32_t* counters;        // this launch's queue positions [n_xcd + 1], zeroed
  int32_t n_xcd;
  // bounds every plan entry is checked against
  int32_t H, n_units, max_items, max_slots, n_k_tiles, entry_cap;
  float* part_o;            // [slot][rows of a workgroup][D], unnormalised O
  float2* part_ml;          // [slot][rows of a workgroup]: (running max, row sum)
  float c;             // scale * log2(e)
  float thr;           // lazy-rescale threshold in raw score units
  int32_t mask_all;    // evaluate the mask on every executed step
  int32_t round_tile;  // the map rounds the contiguous mask part to whole tiles
};

// Kernel arguments needed only where a work item starts or ends are read
// there again, with volatile loads from the argument segment that the
// compiler cannot hoist: kept live across the step loop they would crowd the
// scalar registers that the step machinery needs (and spill into vector
// lanes read back inside the MFMA phase). The kernel's one argument is the
// KParams struct at offset 0 of the segment.
template <typename T, size_t OFF>
__device__ __forceinline__ T kernarg_reload() {
  typedef __attribute__((address_space(4))) const char* kptr;
  typedef __attribute__((address_space(4))) const volatile T* vptr;
  return *(vptr)((kptr)__builtin_amdgcn_kernarg_segment_ptr() + OFF);
}
#define ARG(field) (kernarg_reload<decltype(KParams::field), offsetof(KParams, field)>())

// The same for fields of a work item that the item's end needs again.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 reload_int4(const int4* p) { return *(const volatile i32x4*)p; }

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

// V rows are stored in another order: LDS row m holds key vkey(m), so that
// the four keys 4b..4b+3 of a 16-key block sit 4 rows apart. A transposing
// read of 4 keys x 64 dims then spans rows 4 x 272 bytes apart, 16 banks
// apart, and its 32 lanes of 8 bytes hit 64 distinct banks (with
// consecutive rows they would hit the same banks 2 to 4 times).
__device__ __forceinline__ int vkey(int m) {
  return (m & ~15) | ((m & 3) << 2) | ((m >> 2) & 3);
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
// then [b, S), 64 per step, read at rows s * F. Both forms are computed and
// selected, so that the step path has no branch (scalar selects only).
__device__ __forceinline__ Step make_step(const KParams& p, int ti, int bnd, int kt, int part,
                                          int js, int n_s1, int sa, int sb) {
  const bool tile = ti != 0;
  const int c0 = kt * p.BK + part * CK;
  const int tend = min(p.N, kt * p.BK + p.BK);
  const bool first = js < n_s1;
  const int s0 = first ? js * CK : sb + (js - n_s1) * CK;
  const int lim = first ? sa : p.S;
  Step s;
  s.base = tile ? c0 : s0 * p.F;
  s.stride = tile ? 1 : p.F;
  s.ncols = min(CK, tile ? tend - c0 : lim - s0);
  s.pred = (ti & bnd) | p.mask_all | (int)((uint32_t)(s.ncols - CK) >> 31);
  return s;
}

// Staging of one step. K rows and V rows move from HBM straight into LDS
// (buffer_load ... lds, no VGPRs), both in the same padded row layout (LDS
// row m of a 32-row K block holds key sigma(m); LDS row m of V holds key
// vkey(m)). The (row, chunk) a lane fetches in load j is fixed, so its byte
// offset from the step's first row is too: one table for steps of
// consecutive rows, one for sink steps at a stride of F rows. The step's
// first row goes into the base of the buffer resources, whose record count
// ends at the end of the sequence: rows past it read as zeros (the buffer
// range check), rows past the step's column count are masked, and a load
// costs no address arithmetic. Pad slots re-read chunk 0 of their row (never
// read back).
//
// V is then transposed inside LDS once per step: each 16-lane group reads 4
// keys x 16 dims with one ds_read_b64_tr_b16 (lane j gets dim j of the 4
// keys), two such reads give each lane 8 keys of one dim, written as one
// 16-byte V^T row slot. The PV product then reads V^T with ds_read_b128.
template <int D, int NW>
struct Stage {
  using Lt = Layout<D, NW>;
  static constexpr int ROWB = 2 * D;  // bytes per K/V row in HBM
  // Byte offsets from the step's first row, per load: K and V rows, for
  // consecutive rows and at a row stride of F (saturated: past the end).
  uint32_t koff[Lt::LPW], koffs[Lt::LPW], voff[Lt::LPW], voffs[Lt::LPW];

  __device__ __forceinline__ void init(int wl, int lane, int F) {
    auto put = [&](int r, uint32_t byte, uint32_t& o, uint32_t& os) {
      o = (uint32_t)(r * ROWB) + byte;
      const uint64_t fs = (uint64_t)r * (uint64_t)F * ROWB + byte;
      os = fs < 0x80000000ull ? (uint32_t)fs : 0x80000000u;
    };
#pragma unroll
    for (int i = 0; i < Lt::LPW; ++i) {
      // a wave with no load i repeats its load i-1
      const int si = i == 0 || k_ok(i, wl) ? i : i - 1;
      const int slot = (si * Lt::NL + wl) * 64 + lane;
      const int prow = slot / Lt::KSLOTS, c = slot - prow * Lt::KSLOTS;
      const uint32_t byte = 16 * (c < Lt::NCH ? c : 0);
      put((prow & ~31) | sigma(prow & 31), byte, koff[i], koffs[i]);
      put(vkey(prow), byte, voff[i], voffs[i]);
    }
  }

  // Buffer resources of a step: K and V of the head from the step's first
  // row (clamped to the end of the sequence) to the end of the sequence.
  struct Src {
    __amdgpu_buffer_rsrc_t k, v;
  };
  __device__ __forceinline__ static Src src(const KParams& p, const uint16_t* kh,
                                            const uint16_t* vh, const Step& s) {
    const int b = min(s.base, p.N);
    const int n = (p.N - b) * ROWB;
    const size_t e = (size_t)b * D;
    return {__builtin_amdgcn_make_buffer_rsrc((void*)(kh + e), (short)0, n, 0x00020000),
            __builtin_amdgcn_make_buffer_rsrc((void*)(vh + e), (short)0, n, 0x00020000)};
  }

  __device__ __forceinline__ bool k_ok(int i, int wl) const {
    return Lt::KLOADS % Lt::NL == 0 || i * Lt::NL + wl < Lt::KLOADS;
  }

  // Load pair j (K and V rows of one 1 KiB slot) of step `s` into `buf`,
  // without a branch: a wave that has no load j repeats its load j-1 (the
  // same bytes to the same place). wl1k = 1024 * wl, the wave's slot; the
  // caller launders it once per step, so that the destination of each load
  // is one scalar add there rather than a register held across the loop.
  __device__ __forceinline__ void load(const Src& sr, const Step& s, char* buf, int wl, int wl1k,
                                       int j) const {
    // (the tables already hold the repeated load; indices stay compile-time
    // constants, which keeps the tables in registers)
    const bool ok = j == 0 || k_ok(j, wl);
    const bool one = s.stride == 1;
    const uint32_t ko = one ? koff[j] : koffs[j];
    const uint32_t vo = one ? voff[j] : voffs[j];
    const int at = (ok ? j * Lt::NL * 1024 : (j - 1) * Lt::NL * 1024) + wl1k;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr.k, (lds_void*)(buf + at), 16, ko, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr.v, (lds_void*)(buf + Lt::VR_OFF + at), 16, vo,
                                             0, 0, 0);
  }

  // V rows of `src` -> V^T of `dst` (this transposer wave's share). Chunk
  // c = (t * NT + wt) * 64 + lane is dim c % D of key group c / D; a 16-lane
  // group covers 16 consecutive dims of one key group. An address is a
  // per-lane part, a per-wave part and a per-pass part; the per-wave part is
  // added to the per-lane base once (it does not depend on the pass, see
  // tr_split_ok), so that every pass adds a compile-time offset only.
  struct TrLane {
    int rd, wr;
  };
  __device__ __forceinline__ static TrLane tr_lane(int lane, int wt) {
    const int q = lane >> 4, jj = lane & 15;
    return {(jj >> 2) * 4 * Lt::KROW + 2 * (16 * q + 4 * (jj & 3)) + tr_rd(wt, 0, 0) -
                tr_rd(0, 0, 0),
            (16 * q + jj) * Lt::VTROW + tr_wr(wt, 0) - tr_wr(0, 0)};
  }
  // offsets of pass t of wave wt: read offsets of keys 8g..8g+3 and
  // 8g+4..8g+7 (key 16a + 4b + i sits in V row 16a + 4i + b) and the write
  // offset
  __host__ __device__ static constexpr int tr_rd(int wt, int t, int half) {
    const int u = t * Lt::NT + wt, dd = (u % (D / 64)) * 64, g = u / (D / 64);
    const int pr = 16 * (g >> 1) + 2 * (g & 1) + half;
    return Lt::VR_OFF + pr * Lt::KROW + 2 * dd;
  }
  __host__ __device__ static constexpr int tr_wr(int wt, int t) {
    const int u = t * Lt::NT + wt, dd = (u % (D / 64)) * 64, g = u / (D / 64);
    return Lt::VT_OFF + dd * Lt::VTROW + 16 * g;
  }
  // The offsets split into a wave part and a pass part for every transposer
  // wave and pass.
  __host__ __device__ static constexpr bool tr_split_ok() {
    for (int wt = 0; wt < Lt::NT; ++wt)
      for (int t = 0; t < Lt::TPW; ++t) {
        for (int half = 0; half < 2; ++half)
          if (tr_rd(wt, t, half) != tr_rd(0, t, half) + tr_rd(wt, 0, 0) - tr_rd(0, 0, 0))
            return false;
        if (tr_wr(wt, t) != tr_wr(0, t) + tr_wr(wt, 0) - tr_wr(0, 0)) return false;
      }
    return true;
  }
  __device__ __forceinline__ static i16x8 tr_read(const char* src, const TrLane& tl, int t) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(src + tr_rd(0, t, 0) + tl.rd));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(src + tr_rd(0, t, 1) + tl.rd));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ __forceinline__ static void tr_write(char* dst, const TrLane& tl, int t,
                                                  const i16x8& x) {
    *(i16x8*)(dst + tr_wr(0, t) + tl.wr) = x;
  }
  __device__ __forceinline__ static void transpose(const char* src, char* dst, const TrLane& tl) {
#pragma unroll
    for (int t = 0; t < Lt::TPW; ++t) tr_write(dst, tl, t, tr_read(src, tl, t));
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
  // Position at step s0 of the row: tile steps (cpt per tile) come first,
  // then the sink steps.
  __device__ __forceinline__ void init(const int32_t* row_ents, int nt, int nf, int ns1, int a,
                                       int b, int lane, int cpt, int s0) {
    ents = row_ents;
    n_tiles = nt;
    n_full = nf;
    n_s1 = ns1;
    sa = a;
    sb = b;
    if (s0 < nt * cpt) {
      e = s0 / cpt;
      part = s0 - e * cpt;
      js = 0;
    } else {
      e = nt;
      part = 0;
      js = s0 - nt * cpt;
    }
    chunk = e >> 6;
    e_cur = load(chunk, lane);
    e_nxt = load(chunk + 1, lane);
  }
  // Refill the window when the next step starts a new 64-entry chunk (the
  // only branch of the cursor; rare).
  __device__ __forceinline__ void refill(int lane) {
    if (e < n_tiles && (e >> 6) != chunk) {  // entries are visited in order
      e_cur = e_nxt;
      ++chunk;
      e_nxt = load(chunk + 1, lane);
    }
  }
  // Descriptor of the next step; the cursor moves one step on. Branch-free,
  // so that it can run between the MFMAs of a phase. Past the last step it
  // yields descriptors of rows that are never used.
  __device__ __forceinline__ Step next(const KParams& p) {
    // (integer arithmetic rather than selects on comparisons, which the
    // compiler would widen through vector registers)
    const int ti = (int)((uint32_t)(e - n_tiles) >> 31);     // e < n_tiles
    const int bnd = (int)((uint32_t)(n_full - 1 - e) >> 31);  // e >= n_full
    const int kt = __builtin_amdgcn_readlane(e_cur, __builtin_amdgcn_readfirstlane(e & 63));
    const Step st = make_step(p, ti, bnd, kt, part, js, n_s1, sa, sb);
    const int last = 1 - min(1, p.cpt - part - 1);           // part + 1 == cpt
    e += ti * last;
    part += ti * (1 - last * (part + 1));                    // part + 1, or 0 after the last
    js += 1 - ti;
    return st;
  }
};

// vmcnt(0), as an instruction the compiler accounts for
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Workgroup barrier after this wave's LDS operations completed. Unlike
// __syncthreads() it does not also wait for outstanding global loads.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// Border between the two phases of a step: the scheduler must not move work
// across it, since softmax work sunk into the MFMA phase (or the reverse)
// would run on the wave's own VALU beside its MFMAs instead of beside the
// partner wave's. (No barrier: within a step the groups read only the
// current stage and write only the next one.)
__device__ __forceinline__ void phase_fence() { __builtin_amdgcn_sched_barrier(0); }

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(KParams p) {
  using Lt = Layout<D, NW>;
  constexpr int WGQ = NW * QW;
  constexpr int NS = 2 * (D / 16);  // MFMAs of S^T per step: (d-step, key block)
  constexpr int NDB = D / 32;       // 32-row blocks of O^T
  constexpr int NPV = 4 * NDB;      // MFMAs of O^T per step: (16-key step, d block)
  constexpr int NM = NPV + NS;      // MFMAs of one M phase
  constexpr int PD = 4;             // LDS operand prefetch depth, in MFMAs
  constexpr int LS = NM / Lt::LPW < 3 ? (NM / Lt::LPW < 1 ? 1 : NM / Lt::LPW) : 3;  // MFMAs per load pair
  // Eight waves form two groups, one wave of each per SIMD, that alternate
  // between the MFMA phase and the softmax phase.
  constexpr bool PP = NW == 8;
  constexpr float NEG_INF = -__builtin_huge_valf();
  __shared__ __attribute__((aligned(1024))) char buf0[Lt::BUF];
  __shared__ __attribute__((aligned(1024))) char buf1[Lt::BUF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, l32 = lane & 31;
  const int grp = PP && wave >= NW / 2 ? 1 : 0;

  // Group 0 (every wave with fewer than eight) issues the HBM loads, group 1
  // (every wave with fewer than eight) transposes V.
  const bool loader = !PP || grp == 0;
  const int wl = wave, wt = PP ? wave - NW / 2 : wave;
  static_assert(Stage<D, NW>::tr_split_ok(), "transpose offsets must split into wave and pass parts");
  const typename Stage<D, NW>::TrLane tl = Stage<D, NW>::tr_lane(lane, wt);
  Stage<D, NW> stg;
  if (loader) stg.init(wl, lane, p.F);
  // The V rows of both stages start as zeros: a row past the sequence reads
  // as zero, and should its LDS slot be left unwritten instead, the slot
  // still holds a finite value (zero or an earlier row), so that P = 0 times
  // it stays 0 in O.
  for (int off = threadIdx.x * 16; off < Lt::KTILE; off += NW * 64 * 16) {
    *(uint4*)(buf0 + Lt::VR_OFF + off) = make_uint4(0, 0, 0, 0);
    *(uint4*)(buf1 + Lt::VR_OFF + off) = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();  // the zeros land before any load writes LDS

  // (every plan entry is checked against the buffers' bounds: a plan that
  // is wrong cannot make the kernel read or write out of range)
  // Work items come from this XCD's queue, in the plan's order, to
  // whichever workgroup of the XCD asks first: the plan decides what runs
  // and roughly when; the queue lets the workgroups that really finish
  // first take the next item, so that neighbouring Q tiles keep running
  // together and share their KV tiles in the L2.
  // Once the XCD's queue is empty, the workgroup takes items from the
  // shared tail (queue n_xcd), whose parts shrink towards its end: XCDs do
  // not run equally fast, and the tail lets the faster ones take more.
  __shared__ int s_take, s_queue;
  uint32_t xcc = __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & 0xF;  // XCC_ID
  if ((int)xcc >= p.n_xcd) xcc = blockIdx.x % p.n_xcd;
  int queue = xcc;  // (thread 0's copy decides)
  for (;;) {
    __syncthreads();  // every wave has read the previous position
    if (threadIdx.x == 0) {
      int t = atomicAdd(p.counters + queue, 1);
      if (queue != p.n_xcd && t >= p.item_ptr[queue + 1] - p.item_ptr[queue]) {
        queue = p.n_xcd;
        t = atomicAdd(p.counters + queue, 1);
      }
      s_take = t;
      s_queue = queue;
    }
    __syncthreads();
    const int qs = __builtin_amdgcn_readfirstlane(s_queue);
    const int q_begin = max(0, p.item_ptr[qs]);
    const int q_end = min(p.item_ptr[qs + 1], p.max_items);
    const int it = q_begin + __builtin_amdgcn_readfirstlane(s_take);
    if (it >= q_end) break;
    // the item and its row: (unit, first step, end step, partial slot),
    // (FULL tiles, executed tiles, first entry, sink a), (sink b, head,
    // first query row, head kind)
    const int4* idp = ARG(items) + 3 * (size_t)it;
    const int4 item = idp[0], ib = idp[1], ic = idp[2];
    const int n_full = ib.x, n_tiles = ib.y, ebeg = ib.z, sa = ib.w, sb = ic.x;
    const int h = ic.y, wg_q = ic.z, kind = ic.w;
    if (item.x < 0 || item.x >= ARG(n_units) || item.w >= ARG(max_slots) || h < 0 ||
        h >= ARG(H) || wg_q < 0 || wg_q >= p.N || n_full < 0 || n_full > n_tiles ||
        n_tiles > ARG(n_k_tiles) || ebeg < 0 || ebeg > ARG(entry_cap) - n_tiles || sa < 0 ||
        sa > p.S || sb < sa || sb > p.S)
      continue;
    const int BQ = ARG(BQ), qt = wg_q / BQ;

    const int n_tile_steps = n_tiles * p.cpt;
    const int n_s1 = (sa + CK - 1) / CK;
    const int n_row_steps = n_tile_steps + n_s1 + (p.S - sb + CK - 1) / CK;
    // this item's steps (the last part of a row runs to its end)
    const int s_first = max(0, min(item.y, n_row_steps));
    const int n_steps = max(0, min(item.z, n_row_steps) - s_first);

    const size_t head_off = (size_t)h * p.N * D;
    const uint16_t* Qh = ARG(q) + head_off;
    const uint16_t* Kh = p.k + head_off;
    const uint16_t* Vh = p.v + head_off;

    // Stage 0's V^T area starts as zeros, which the first MFMA phase
    // multiplies by P = 0. (Nobody reads it now: the previous item ended with
    // a barrier after its last LDS access, and the loads below go elsewhere.)
    for (int off = threadIdx.x * 16; off < Lt::VTILE; off += NW * 64 * 16)
      *(uint4*)(buf0 + Lt::VT_OFF + off) = make_uint4(0, 0, 0, 0);
    // Stage 0 holds the first step's K and V rows.
    Cursor cur_pos;
    cur_pos.init(ARG(entries) + ebeg, n_tiles, n_full, n_s1, sa, sb, lane, p.cpt, s_first);
    Step st_t = {0, 1, 0, 0};
    if (n_steps > 0) {
      st_t = cur_pos.next(p);
      if (loader)
#pragma unroll
        for (int j = 0; j < Lt::LPW; ++j)
          stg.load(Stage<D, NW>::src(p, Kh, Vh, st_t), st_t, buf0, wl, wl * 1024, j);
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
    const int W_f = ARG(W_f), W_s = ARG(W_s), sink = ARG(sink);
    if (kind == SVG_HEAD_SPATIAL) {
      const int f = q / p.S;
      wlo = max(0, f - W_f) * p.S;
      whi = min(p.F, f + W_f + 1) * p.S;
      slim = sink ? p.S : 0;
    } else if (kind == SVG_HEAD_TEMPORAL) {
      const int s = q / p.F;
      wlo = max(0, s - W_s) * p.F;
      whi = min(p.S, s + W_s + 1) * p.F;
      msink = sink != 0;
    }
    if (ARG(round_tile) && kind != SVG_HEAD_DENSE) {
      // Tile-aligned mask: a pair is kept when its (BQ x BK) tile holds any pair
      // of the contiguous mask part, so the bound is the same for every row of
      // the map's Q tile: the union of its rows' windows (or bands), widened to
      // whole KV tiles; the spatial sink [0, S) is widened the same way and the
      // temporal strided sink stays exact.
      const int t0 = qt * BQ, t1 = min(p.N, t0 + BQ) - 1;
      if (kind == SVG_HEAD_SPATIAL) {
        wlo = max(0, t0 / p.S - W_f) * p.S;
        whi = min(p.F, t1 / p.S + W_f + 1) * p.S;
      } else {
        wlo = max(0, t0 / p.F - W_s) * p.F;
        whi = min(p.S, t1 / p.F + W_s + 1) * p.F;
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
    f32x16 s[2];   // S^T of a step, from its MFMA phase to its softmax phase
    bf16x8 pf[4];  // P^T of a step, from its softmax phase to the next MFMA phase
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) pf[kk] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));

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
    auto opread = [&](const char* kb, const char* vb, int i) __attribute__((always_inline)) {
      return i < NPV ? vread(vb, i) : kread(kb, i - NPV);
    };

    // MFMA phase on the stage in `cb`: O^T += V^T P^T for the previous step,
    // then S^T = K Q^T for this one; operands read PD MFMAs ahead. The wave is
    // idle between its MFMAs, so other memory work rides along: side.at(i)
    // emits it after MFMA i and side.pattern(i) places it in the schedule.
    auto mphase = [&](const char* cb, auto&& side) __attribute__((always_inline)) {
      const char* kb = cb + k_lane;
      const char* vb = cb + v_lane;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb2][v] = 0.f;
      bf16x8 a[PD];
#pragma unroll
      for (int i = 0; i < PD; ++i) a[i] = opread(kb, vb, i);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        const bf16x8 x = a[i % PD];
        if (i + PD < NM) a[i % PD] = opread(kb, vb, i + PD);
        if (i < NPV) {
          o[i % NDB] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, pf[i / NDB], o[i % NDB], 0, 0, 0);
        } else {
          const int k = i - NPV;
          s[k & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, qf[k >> 1], s[k & 1], 0, 0, 0);
        }
        side.at(i);
      }
      // Keep the reads ahead of their MFMAs (the default schedule assumes a
      // far shorter LDS latency).
      __builtin_amdgcn_sched_group_barrier(0x100, PD, 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + PD < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        side.pattern(i);
      }
    };

    // Softmax phase of step `cur`: mask, lazy running maximum, P^T = exp2(...)
    // in bf16 and the row sum.
    auto vphase = [&](const Step& cur) __attribute__((always_inline)) {
      // mask: column limit of short steps, head predicate on boundary tiles.
      // Key kl of the step sits at row base + kl * stride, so the window, the
      // spatial sink and the column limit are intervals of kl and the strided
      // sink (rows that are multiples of F) is a pattern shared by the wave:
      // the step's 64 keep bits form one 64-bit mask per lane, of which the
      // lane keeps the bytes of its own keys (8-key groups 2c + hl).
      if (cur.pred) {
        const int sd = cur.stride;
        auto kl_at = [&](int x) __attribute__((always_inline)) {  // first key at or past row x
          const int d = x - cur.base;
          int k = 0;
          if (d > 0) k = sd == 1 ? d : (d + sd - 1) / sd;
          return min(k, 64);
        };
        auto ge = [](int a) __attribute__((always_inline)) {  // keys a..63
          return a >= 64 ? 0ull : ~0ull << a;
        };
        uint64_t m = (ge(kl_at(wlo)) & ~ge(kl_at(whi))) | ~ge(kl_at(slim));
        if (msink) {
          uint64_t pat = 0;
          if (sd == 1) {
            for (int k = (p.F - cur.base % p.F) % p.F; k < 64; k += p.F) pat |= 1ull << k;
          } else if (cur.base % p.F == 0) {
            pat = ~0ull;  // a stride of F keeps the row residue mod F
          }
          m |= pat;
        }
        m &= ~ge(max(cur.ncols, 0));
        const uint32_t keep = __builtin_amdgcn_perm((uint32_t)(m >> 32), (uint32_t)m,
                                                    hl ? 0x07050301u : 0x06040200u);
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (!((keep >> (16 * kb2 + v)) & 1u)) s[kb2][v] = NEG_INF;
      }
      // P^T = exp2(S^T c - m_ref c) in bf16 and this lane's part of the row sum
      // (plain adds: v_dot2 cannot issue while the partner wave's MFMAs run)
      auto expo = [&]() __attribute__((always_inline)) {
        const float mc = m_ref == NEG_INF ? 0.f : m_ref * p.c;
        float ls[2] = {0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          uint32_t w[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int v = 8 * (kk & 1) + 2 * t;
            const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][v], p.c, -mc));
            const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][v + 1], p.c, -mc));
            ls[t & 1] += e0 + e1;
            w[t] = pack_bf16(e0, e1);
          }
          pf[kk] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        }
        return ls[0] + ls[1];
      };
      // The lazy reference m_ref only has to keep every value at most 2^8. A
      // partial row sum of at most 2^8 (finite) proves that for the lane's
      // keys, so the row maximum is needed only when some lane's sum exceeds
      // it or no reference exists yet: then the maximum over both halves of
      // the row is taken, O and the row sum are rescaled when it grew by more
      // than 8 in log2 units, and the values are computed again.
      float ls = expo();
      if (__builtin_amdgcn_ballot_w64(!(ls <= 256.f) || m_ref == NEG_INF)) {
        float mx = NEG_INF;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb2][v]);
        {
          float x0, x1;
          halves(mx, x0, x1);
          mx = fmaxf(x0, x1);
        }
        const bool need = mx > m_ref + p.thr;
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
        ls = expo();
      }
      l_sum += ls;
    };

    if (n_steps > 0) {
      cur_pos.refill(lane);
      Step st_next = cur_pos.next(p);  // step 1 (rows never used when there is none)
      wait_vmem();
      __syncthreads();  // stage 0 and the zero V^T visible to every wave

      // Iteration t works on the buffer `cb` that holds the K rows of step t,
      // V^T of step t-1 and the V rows of step t, and fills `nb` for step t+1.
      // Group 0 runs the MFMA phase of step t (PV of step t-1, S^T of step t)
      // with the loads of the K and V rows of step t+1 into `nb` woven in,
      // then the softmax of step t. Group 1 runs the softmax of step t-1, then
      // the MFMA phase of step t with the transpose of V of step t into V^T of
      // `nb` woven in. The softmax phases carry no memory work, and the waves
      // of a SIMD alternate: one runs its MFMAs while the other runs its
      // softmax. Within the iteration every LDS read is of `cb`, complete since
      // the iteration began, and every write is to `nb`, which nobody reads
      // until the next one, so a single barrier closes the iteration once the
      // loads and V^T writes have landed. Iteration n_steps only finishes
      // the last PV product (its S^T reads K rows that are not loaded and is
      // never used). One loop per group (the group is a compile-time constant
      // in each), so that the two phase orders are never merged.
      auto run = [&](auto grp_c) __attribute__((always_inline)) {
        constexpr int G = decltype(grp_c)::value;
        Step st_prev = st_t;
        auto iter = [&](const char* cb, char* nb, int t) __attribute__((always_inline)) {
          const bool has_v = t < n_steps;
          // The descriptor of step t+2 is computed off the critical path: by
          // group 0 between the MFMAs of its MFMA phase, by group 1 with its
          // softmax (scalar work interleaved with MFMAs would delay them).
          cur_pos.refill(lane);
          Step st_nn;
          if constexpr (G == 0) {
            // One K+V load pair every LS-th MFMA (every third when there are
            // few). After the last step they fetch rows of the last step again
            // into a stage nobody reads.
            struct DmaSide {
              const Stage<D, NW>& stg;
              typename Stage<D, NW>::Src sr;
              const Step& st;
              char* nb;
              int wl, wl1k;
              __device__ __forceinline__ void at(int i) const {
                if (i % LS == 0 && i / LS < Lt::LPW) stg.load(sr, st, nb, wl, wl1k, i / LS);
              }
              __device__ __forceinline__ void pattern(int i) const {
                if (i % LS == 0 && i / LS < Lt::LPW)
                  __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
              }
            };
            static_assert(Lt::LPW <= NM, "every load pair needs an MFMA slot");
            if (!PP) Stage<D, NW>::transpose(cb, nb, tl);
            st_nn = cur_pos.next(p);
            // (laundered once per step: see Stage::load)
            int wl1k = wl * 1024;
            asm volatile("" : "+s"(wl1k));
            mphase(cb,
                   DmaSide{stg, Stage<D, NW>::src(p, Kh, Vh, st_next), st_next, nb, wl, wl1k});
            if (PP) phase_fence();
            if (has_v) vphase(st_t);
          } else {
            // The transpose reads its V rows at the start of the softmax phase
            // (the VALU-bound phase issues them almost for free) and writes V^T
            // during the MFMA phase, long after the reads have landed, so no
            // write waits. After the last step it fills a V^T nobody reads.
            i16x8 trbuf[Lt::TPW];
#pragma unroll
            for (int j = 0; j < Lt::TPW; ++j) trbuf[j] = Stage<D, NW>::tr_read(cb, tl, j);
            st_nn = cur_pos.next(p);
            if (t > 0) vphase(st_prev);
            phase_fence();
            // write j after MFMA 4j+2
            struct TrSide {
              char* nb;
              const typename Stage<D, NW>::TrLane& tl;
              const i16x8 (&buf)[Lt::TPW];
              __device__ __forceinline__ void at(int i) const {
#pragma unroll
                for (int j = 0; j < Lt::TPW; ++j)
                  if (i == 4 * j + 2) Stage<D, NW>::tr_write(nb, tl, j, buf[j]);
              }
              __device__ __forceinline__ void pattern(int i) const {
#pragma unroll
                for (int j = 0; j < Lt::TPW; ++j)
                  if (i == 4 * j + 2) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
              }
            };
            static_assert(4 * Lt::TPW + 2 < NM || !PP, "transpose writes must fit the phase");
            mphase(cb, TrSide{nb, tl, trbuf});
          }
          // (pinned here: the scheduler would otherwise hoist the wait into
          // the phases above)
          __builtin_amdgcn_sched_barrier(0);
          wait_vmem();
          barrier_lds();
          st_prev = st_t;
          st_t = st_next;
          st_next = st_nn;
        };
        for (int t = 0; t <= n_steps; t += 2) {
          iter(buf0, buf1, t);
          if (t + 1 <= n_steps) iter(buf1, buf0, t + 1);
        }
      };
      if (grp == 0)
        run(std::integral_constant<int, 0>{});
      else
        run(std::integral_constant<int, 1>{});
    }

    // ---- epilogue. A whole row: O = O^T / l in bf16 (round to nearest even).
    // A part of a cut row: the unnormalised O^T, the running maximum and the
    // row sum to its partial slot, for combine_kernel.
    float la, lb;
    halves(l_sum, la, lb);
    const float lt = la + lb;
    // (the slot and the head read again, not held across the steps)
    const int4* idq = ARG(items) + 3 * (size_t)it;
    const int slot = __builtin_amdgcn_readfirstlane(reload_int4(idq)[3]);
    const int h_end = __builtin_amdgcn_readfirstlane(reload_int4(idq + 2)[1]);
    if (slot < 0) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      if (q < p.N) {
        uint16_t* orow = ARG(o) + (size_t)h_end * p.N * D + (size_t)q * D;
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
    } else {
      const size_t r = (size_t)slot * WGQ + wave * QW + l32;
      float* po = ARG(part_o) + r * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(float4*)(po + 32 * db + 8 * i + 4 * hl) =
              make_float4(o[db][4 * i + 0], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]);
      if (hl == 0) ARG(part_ml)[r] = make_float2(m_ref, lt);
    }
  }  // work items
}

// Merge the parts of cut rows: with M the largest running maximum over a
// row's parts and w_i = 2^((m_i - M) c), O = sum_i w_i O_i / sum_i w_i l_i,
// rounded to bf16 as the attention kernel rounds whole rows. A workgroup
// takes one block of CRB query rows of one combine entry: it first puts each
// row's normalised weights w_i / L in LDS, then streams the parts' O rows
// (coalesced 16-byte loads) into per-thread sums. Entries past the plan's
// count exit at once.
struct CombineParams {
  uint16_t* o;
  const float* part_o;
  const float2* part_ml;
  const int32_t* header;  // [1]: combine entries
  const int4* combine;    // (unit, first slot, parts, -)
  int32_t N, nQ, BQ, nsub, n_units, max_slots;
  float c;
};

constexpr int CRB = 64;   // query rows per combine workgroup
constexpr int CPC = 16;   // parts weighted per pass

template <int D, int WGQ>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int RB = WGQ < CRB ? WGQ : CRB;
  constexpr int NB = WGQ / RB;         // row blocks per entry
  constexpr int PER = RB * (D / 4) / 256;  // float4 sums per thread
  static_assert(RB * (D / 4) % 256 == 0, "row block must split over the threads");
  constexpr float NEG_INF = -__builtin_huge_valf();
  __shared__ float wts[CPC][RB];
  const int ei = blockIdx.x / NB, rb = blockIdx.x - ei * NB;
  if (ei >= p.header[1]) return;
  const int4 e = p.combine[ei];
  if (e.x < 0 || e.x >= p.n_units || e.y < 0 || e.z < 1 || e.z > p.max_slots - e.y) return;
  const int row = e.x / p.nsub, sub = e.x - row * p.nsub;
  const int h = row / p.nQ, qt = row - h * p.nQ;
  const int r0 = rb * RB;                      // first row of the block within the slice
  const int q0 = qt * p.BQ + sub * WGQ + r0;   // its query row
  const int t = threadIdx.x;
  // every row's largest maximum and weighted sum (thread t < RB: row t)
  float M = NEG_INF, L = 0.f;
  if (t < RB) {
    for (int i = 0; i < e.z; ++i) M = fmaxf(M, p.part_ml[(size_t)(e.y + i) * WGQ + r0 + t].x);
    for (int i = 0; i < e.z; ++i) {
      const float2 ml = p.part_ml[(size_t)(e.y + i) * WGQ + r0 + t];
      L += ml.x == NEG_INF ? 0.f : ml.y * __builtin_amdgcn_exp2f((ml.x - M) * p.c);
    }
  }
  const float invL = L > 0.f ? 1.f / L : 0.f;
  float4 acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < e.z; i0 += CPC) {
    const int np = min(CPC, e.z - i0);
    __syncthreads();  // the previous pass is done with the weights
    if (t < RB)
      for (int i = 0; i < np; ++i) {
        const float2 ml = p.part_ml[(size_t)(e.y + i0 + i) * WGQ + r0 + t];
        wts[i][t] = ml.x == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((ml.x - M) * p.c) * invL;
      }
    __syncthreads();
    for (int i = 0; i < np; ++i) {
      const float* po = p.part_o + ((size_t)(e.y + i0 + i) * WGQ + r0) * D;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int idx = t + 256 * j, r = idx / (D / 4);
        const float wgt = wts[i][r];
        const float4 x = *(const float4*)(po + 4 * idx);
        acc[j].x += x.x * wgt;
        acc[j].y += x.y * wgt;
        acc[j].z += x.z * wgt;
        acc[j].w += x.w * wgt;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int idx = t + 256 * j, r = idx / (D / 4), c4 = idx - r * (D / 4);
    if (q0 + r >= p.N) continue;
    uint2 out;
    out.x = pack_bf16(acc[j].x, acc[j].y);
    out.y = pack_bf16(acc[j].z, acc[j].w);
    *(uint2*)(p.o + ((size_t)h * p.N + q0 + r) * D + 4 * c4) = out;
  }
}

int waves_for(int32_t tile_q) {
  if (tile_q % 256 == 0) return 8;
  if (tile_q == 128) return 4;
  if (tile_q == 64) return 2;
  if (tile_q == 32) return 1;
  return 0;
}

// Zero a launch's queue positions (a kernel rather than a memset, so that
// the launch sequence can also be captured into a graph).
__global__ __launch_bounds__(64) void zero_counters_kernel(int32_t* c, int32_t n) {
  for (int i = threadIdx.x; i < n; i += 64) c[i] = 0;
}

template <int D, int NW>
hipError_t launch(const KParams& kp, const CombineParams& cp, int n_wg, int n_combine,
                  hipStream_t stream) {
  hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(64), 0, stream, kp.counters,
                     kp.n_xcd + 1);
  hipError_t e0 = hipGetLastError();
  if (e0 != hipSuccess) return e0;
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW>), dim3(n_wg), dim3(NW * 64), 0, stream, kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RB = NW * QW < CRB ? NW * QW : CRB;
  hipLaunchKernelGGL((combine_kernel<D, NW * QW>), dim3(n_combine * (NW * QW / RB)), dim3(256),
                     0, stream, cp);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int nw, const KParams& kp, const CombineParams& cp, int n_wg, int n_combine,
                    hipStream_t stream) {
  switch (nw) {
    case 8: return launch<D, 8>(kp, cp, n_wg, n_combine, stream);
    case 4: return launch<D, 4>(kp, cp, n_wg, n_combine, stream);
    case 2: return launch<D, 2>(kp, cp, n_wg, n_combine, stream);
    default: return launch<D, 1>(kp, cp, n_wg, n_combine, stream);
  }
}

}  // namespace

int32_t attn_waves(int32_t tile_q) { return waves_for(tile_q); }

bool attn_supported(int32_t head_dim, int32_t tile_q, int32_t tile_k) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (waves_for(tile_q) == 0) return false;
  return tile_k >= 32 && tile_k <= 1024 && tile_k % 32 == 0;
}

hipError_t launch_attn_fwd(const MapGeometry& g, const MapBuffers& b, const PlanBuffers& pl,
                           uint32_t ring, const AttnArgs& a, hipStream_t stream) {
  if (!attn_supported(a.head_dim, g.BQ, g.BK) || pl.n_wg <= 0) return hipErrorInvalidValue;
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
  kp.entries = b.entries;
  kp.item_ptr = pl.dev + 4;
  kp.counters = pl.counters + (size_t)(ring % kQueueRing) * (pl.n_xcd + 1);
  kp.n_xcd = pl.n_xcd;
  kp.items = (const int4*)(pl.dev + pl.items_off());
  kp.H = g.H;
  kp.n_units = (int32_t)((int64_t)g.H * g.nQ * kp.nsub);
  kp.n_k_tiles = g.nK;
  kp.entry_cap = (int32_t)b.capacity;
  kp.max_items = (int32_t)pl.max_items;
  kp.max_slots = (int32_t)pl.max_slots;
  kp.part_o = pl.part_o;
  kp.part_ml = (float2*)pl.part_ml;
  kp.c = a.scale * 1.4426950408889634f;
  kp.thr = 8.0f / kp.c;
  kp.mask_all = (a.flags & SVG_ATTN_MASK_ALL_TILES) ? 1 : 0;
  kp.round_tile = g.round == SVG_ROUND_TILE ? 1 : 0;
  CombineParams cp;
  cp.o = kp.o;
  cp.part_o = pl.part_o;
  cp.part_ml = (const float2*)pl.part_ml;
  cp.header = pl.dev;
  cp.combine = (const int4*)(pl.dev + pl.combine_off());
  cp.N = kp.N;
  cp.nQ = g.nQ;
  cp.BQ = g.BQ;
  cp.nsub = kp.nsub;
  cp.n_units = kp.n_units;
  cp.max_slots = kp.max_slots;
  cp.c = kp.c;
  const int n_combine = (int)pl.max_combine;
  return a.head_dim == 128 ? launch_d<128>(nw, kp, cp, pl.n_wg, n_combine, stream)
                           : launch_d<64>(nw, kp, cp, pl.n_wg, n_combine, stream);
}

}  // namespace svg
