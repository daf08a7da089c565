/*
 * svg_attn.h -- C ABI of libsvgattn: exact structured-sparse attention over
 * video-latent tokens, Sparse VideoGen spatial / temporal head masks, on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed. Self-attention of a video diffusion transformer over
 * N = F*S latent tokens (F frames of S = Hh*Ww tokens), restricted per head by
 * a structured mask ("Google Speeds Up Video Diffusion on TPUs with Optimized
 * Sparse Attention", section "Sparse Attention Patterns"):
 *     O = softmax(Q K^T * scale, masked to M) V     per head,
 * with bf16 inputs and outputs and fp32 accumulation. Head masks, with
 * (f, s) = (frame, raster index) of a token:
 *   SPATIAL:  keep (q,k) iff |f_q - f_k| <= frame_window  or  f_k == 0
 *   TEMPORAL: keep (q,k) iff |s_q - s_k| <= temporal_band or  f_k == 0
 *   DENSE:    keep every pair
 * The "or f_k == 0" term is the first-frame attention sink kept by both masks
 * ("Accelerating Spatio-Temporal Attention for Video Diffusion on TPUs",
 * Newsbite, "Interesting facts"); it applies when sink_first_frame != 0.
 *
 * Token layout ("kernel layout"). Spatial and dense heads use the natural,
 * frame-major order p = f*S + s. Temporal heads use the spatial-major order
 * p = s*F + f, which turns the spatial band into a contiguous run (the pages
 * note that the two head kinds need different token orders, Newsbite,
 * "Interesting facts"). The caller passes temporal heads' rows already
 * re-ordered (svg_permute_tokens does it) and gets O back in the same order.
 *
 * Tile map. Every (BQ x BK) tile of a head's score matrix, in kernel layout,
 * is SKIP (no retained pair), FULL (all existing pairs retained) or BOUNDARY
 * (mixed) -- the tile-aware masking of the pages' "Efficient Kernel
 * Implementation" section. FULL tiles run a mask-free path; only BOUNDARY
 * tiles evaluate the mask per element. Last row / column tiles are ragged
 * when N is not a multiple of BQ / BK; classes count existing elements only.
 * Temporal heads execute the hull of KV tiles that hold band pairs plus, as a
 * separate mask-free segment, the frame-0 keys outside that hull (raster
 * indices [0, a) and [b, S), at kernel rows s*F): the result is exact and
 * most tiles are skipped.
 *
 * Tile-aligned mode (SVG_ROUND_TILE; StreamingMeme lead paragraph, Newsbite
 * "Summary"): the contiguous part of each mask (spatial: all of it; temporal:
 * the band) is rounded outward to whole tiles and the temporal frame-0 sink
 * is kept exactly. No executed tile then needs masking. The attention result
 * is exact attention under that enlarged mask.
 *
 * Conventions for every entry point:
 *   - Returns SVG_OK or a negative svg_status; never throws, never aborts.
 *     svg_last_error() gives a message for the last failure of this thread.
 *   - Arguments are validated before any HIP call; a failed validation leaves
 *     all outputs untouched.
 *   - "stream" is a hipStream_t passed as void* (NULL = default stream). Work
 *     is queued on it and the call returns without waiting, unless stated.
 *   - Device pointers are memory of the current HIP device.
 */
#ifndef SVG_ATTN_H
#define SVG_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVG_ABI_VERSION 1

typedef enum svg_status {
  SVG_OK = 0,
  SVG_ERR_INVALID_ARG = -1,    /* null pointer, out-of-range value          */
  SVG_ERR_UNSUPPORTED = -2,    /* head_dim / tile size without a kernel     */
  SVG_ERR_SHAPE_MISMATCH = -3, /* arguments disagree with the tile map      */
  SVG_ERR_ALIGNMENT = -4,      /* device pointer not 16-byte aligned        */
  SVG_ERR_HIP = -5,            /* a HIP runtime call failed                 */
  SVG_ERR_OOM = -6             /* device or host allocation failed          */
} svg_status;

typedef enum svg_head_kind {
  SVG_HEAD_SPATIAL = 0,
  SVG_HEAD_TEMPORAL = 1,
  SVG_HEAD_DENSE = 2
} svg_head_kind;

typedef enum svg_round_mode {
  SVG_ROUND_EXACT = 0, /* the exact masks                                    */
  SVG_ROUND_TILE = 1   /* contiguous mask parts rounded outward to tiles     */
} svg_round_mode;

typedef enum svg_tile_class {
  SVG_TILE_SKIP = 0,
  SVG_TILE_FULL = 1,
  SVG_TILE_BOUNDARY = 2
} svg_tile_class;

typedef enum svg_permute_dir {
  SVG_TO_KERNEL_LAYOUT = 0,   /* dst[h][layout(t)] = src[h][t]              */
  SVG_TO_ORIGINAL_LAYOUT = 1  /* dst[h][t] = src[h][layout(t)]              */
} svg_permute_dir;

/* Attention flags. */
#define SVG_ATTN_MASK_ALL_TILES 1u /* evaluate the mask on every executed tile
                                      (ablation: no mask-free fast path)     */

/* Mask specification. All fields are read during svg_build_tile_map; the
 * head_kind array is copied, the caller keeps ownership. Limits: frames,
 * grid_h, grid_w >= 1; N = frames*grid_h*grid_w <= 2^30; 1 <= num_heads <=
 * 4096; frame_window >= 0; temporal_band >= 0. */
typedef struct svg_mask_spec {
  int32_t frames;            /* F                                            */
  int32_t grid_h;            /* Hh: latent rows per frame                    */
  int32_t grid_w;            /* Ww: latent columns per frame (S = Hh*Ww)     */
  int32_t num_heads;         /* H                                            */
  const int32_t* head_kind;  /* host array [num_heads] of svg_head_kind      */
  int32_t frame_window;      /* W_f: spatial heads keep |f - f'| <= W_f      */
  int32_t temporal_band;     /* W_s: temporal heads keep |s - s'| <= W_s     */
  int32_t sink_first_frame;  /* nonzero: keep every key of frame 0           */
  int32_t round_mode;        /* svg_round_mode                               */
} svg_mask_spec;

/* Opaque, device-resident tile map. One map may serve any number of
 * svg_attn_fwd calls, on any streams of the device it was built on. Its
 * uses share the map's workspace (schedule, launch plan, partial results of
 * cut rows), so the library orders them on the device in the order the
 * calls are made: each svg_attn_fwd and svg_tile_map_rebuild waits on its
 * stream, without blocking the host, for the map's last build and last
 * attention launch. Under stream capture these waits are skipped (an event
 * recorded outside a capture cannot be waited for inside it) and the caller
 * orders the uses of one map. */
typedef struct svg_tile_map svg_tile_map;

typedef struct svg_tile_map_info {
  int64_t seq_len;           /* N                                            */
  int32_t num_heads;         /* H                                            */
  int32_t tile_q, tile_k;    /* BQ, BK                                       */
  int32_t num_q_tiles;       /* nQ = ceil(N / BQ)                            */
  int32_t num_k_tiles;       /* nK = ceil(N / BK)                            */
  int32_t frames, tokens_per_frame;
  int64_t entry_capacity;    /* size of the schedule's entry buffer          */
} svg_tile_map_info;

/* Per-head statistics of a built map (all int64). */
typedef struct svg_head_stats {
  int64_t tiles;          /* nQ * nK                                          */
  int64_t skip, full, boundary;  /* logical classes of the whole map          */
  int64_t exec_full;      /* FULL tiles the schedule executes                 */
  int64_t exec_boundary;  /* BOUNDARY tiles the schedule executes             */
  int64_t exec_sink;      /* sink keys outside the temporal hull, counted in
                             groups of BK per Q tile                          */
  int64_t retained_pairs; /* |M| (exact) or |M'| (tile-aligned)               */
} svg_head_stats;

/* Statistics of the map's launch plan (see svg_build_tile_map). Loads are in
 * 64-key steps plus a fixed cost per work item. */
typedef struct svg_plan_info {
  int32_t workgroups;     /* persistent workgroups: one per compute unit      */
  int32_t xcds;           /* workgroup i runs on XCD i mod xcds               */
  int64_t work_items;     /* items over all workgroups                        */
  int64_t split_rows;     /* workgroup-sized row slices cut into parts        */
  int64_t partial_slots;  /* parts of cut slices (partial results written)    */
  int64_t max_load;       /* cost of the busiest workgroup                    */
  int64_t total_load;     /* cost summed over the workgroups                  */
} svg_plan_info;

/* A3+A4: classify every tile of every head and compact, per (head, Q tile),
 * the KV tiles to execute: FULL ids ascending, then BOUNDARY ids ascending,
 * plus the temporal sink split (a, b). Then plan the attention launch: one
 * workgroup per compute unit, taking work items (a range of 64-key steps of
 * a workgroup-sized slice of a schedule row) from its XCD's queue and then
 * from a tail queue shared by all XCDs. The slices an XCD works on at one
 * time are neighbouring Q tiles; the last slices of each XCD's share are
 * cut between its workgroups so that they end together; the tail (about 5%
 * of the work, in parts that shrink towards its end) evens out XCDs that
 * run at different speeds. The plan is computed on the host from the map's
 * row counts by a host function queued on `stream` and then copied to the
 * device. Everything is queued on `stream` and the call returns without
 * waiting. Allocates the map's device buffers (class map, schedule, plan,
 * and up to 5 x (compute units) partial results of (query rows of a
 * workgroup) x 128 fp32 values for cut slices: 160 MiB for 256-row
 * workgroups on 256 compute units) and pinned host staging, all freed by
 * svg_tile_map_destroy.
 * Supported tile sizes: tile_q in {32, 64, 128} or a multiple of 256 up to
 * 2^20; tile_k a multiple of 32 in [32, 1024].
 * Errors: INVALID_ARG (null spec/out/head_kind, bad sizes or kinds),
 * UNSUPPORTED (tile sizes), OOM, HIP. On error *out is left unchanged. */
svg_status svg_build_tile_map(const svg_mask_spec* spec, int32_t tile_q,
                              int32_t tile_k, void* stream,
                              svg_tile_map** out);

/* Recompute the class map and schedule of an existing map in place, with no
 * allocation (the same kernels as svg_build_tile_map), on `stream` of the
 * map's device, which must be current. The launch plan depends only on the
 * mask specification and is kept. Errors: INVALID_ARG (null map, other
 * device current), HIP. */
svg_status svg_tile_map_rebuild(svg_tile_map* map, void* stream);

/* Sizes of a map. Host-only, no HIP call. */
svg_status svg_tile_map_info_get(const svg_tile_map* map, svg_tile_map_info* out);

/* Copy per-head statistics to host `per_head[num_heads]`. Synchronises the
 * map's build stream. Errors: INVALID_ARG, SHAPE_MISMATCH (num_heads), HIP. */
svg_status svg_tile_map_stats(const svg_tile_map* map, svg_head_stats* per_head,
                              int32_t num_heads);

/* Copy the class map, uint8 [H][nQ][nK] row-major (svg_tile_class values),
 * to host memory of n bytes (n must equal H*nQ*nK). Synchronous. */
svg_status svg_tile_map_copy_classes(const svg_tile_map* map, uint8_t* host,
                                     size_t n);

/* Copy the schedule to host memory (synchronous). With R = H*nQ rows
 * (row = h*nQ + qt):
 *   row_ptr[R+1]   entries[row_ptr[r] .. row_ptr[r+1]) are row r's KV tiles
 *   n_full[R]      the first n_full[r] of them are FULL, the rest BOUNDARY
 *   sink_ab[2R]    (a, b): sink raster indices [0,a) and [b,S) run mask-free
 *   entries[n_entries], n_entries >= row_ptr[R]
 * Any of the four pointers may be NULL to skip it. */
svg_status svg_tile_map_copy_schedule(const svg_tile_map* map, int32_t* row_ptr,
                                      int32_t* n_full, int32_t* sink_ab,
                                      int32_t* entries, size_t n_entries);

/* Statistics of the map's launch plan. Waits for the build. Errors:
 * INVALID_ARG (null pointers), HIP. */
svg_status svg_tile_map_plan_info(const svg_tile_map* map, svg_plan_info* out);

/* Free a map (NULL is accepted). Waits for its last build and its last
 * attention launch. */
svg_status svg_tile_map_destroy(svg_tile_map* map);

/* A5-A8: O = softmax(scale * Q K^T masked to M) V for every head.
 *   q, k, v, o: device bf16 [num_heads][seq_len][head_dim], row-major, 16-byte
 *               aligned, in each head's kernel layout; o must not overlap
 *               q, k or v. The caller owns all four.
 *   head_dim:   64 or 128. scale > 0 and finite (normally 1/sqrt(head_dim)).
 *               One head (seq_len * head_dim * 2 bytes) must be under 2 GiB.
 *   head_kind:  host [num_heads]; must equal the kinds the map was built with.
 *   map:        built for the same seq_len and num_heads, on the current
 *               device (its buffers live there).
 *   flags:      0 or SVG_ATTN_MASK_ALL_TILES.
 * Rows with no retained key would give 0 (the masks here always keep one).
 * Errors: INVALID_ARG (also: the current device is not the map's),
 * UNSUPPORTED (head_dim, head size), SHAPE_MISMATCH (seq_len, num_heads, head
 * kinds vs the map), ALIGNMENT, HIP (launch failure). */
svg_status svg_attn_fwd(const void* q, const void* k, const void* v, void* o,
                        int64_t seq_len, int32_t num_heads, int32_t head_dim,
                        float scale, const int32_t* head_kind,
                        const svg_tile_map* map, uint32_t flags, void* stream);

/* Tile-size search. The pages pick tile sizes by measured latency, not by
 * the least boundary work ("Google Speeds Up Video Diffusion on TPUs with
 * Optimized Sparse Attention", "Tile size tuning"; Newsbite, "Interesting
 * facts" and "Actionable takeaways"). For each candidate i, (tile_q[i],
 * tile_k[i]): build a tile map for `spec`, run svg_attn_fwd once untimed,
 * then `reps` times between two HIP events on `stream`, and store the mean
 * milliseconds per call in ms[i] (host array [n_cand]); *best receives the
 * index of the smallest. q, k, v, o are as for svg_attn_fwd, with seq_len,
 * num_heads and head kinds taken from `spec`; o is overwritten. scale as for
 * svg_attn_fwd. Synchronous: returns after the last run has finished; maps
 * are freed before it returns.
 * Limits: 1 <= n_cand <= 256, 1 <= reps <= 1000.
 * Errors: INVALID_ARG (null pointers, counts), UNSUPPORTED (a candidate or
 * head_dim without a kernel; all candidates are checked before the first
 * run), the errors of svg_build_tile_map and svg_attn_fwd, HIP. */
svg_status svg_autotune_tiles(const svg_mask_spec* spec, const void* q,
                              const void* k, const void* v, void* o,
                              int32_t head_dim, float scale,
                              const int32_t* tile_q, const int32_t* tile_k,
                              int32_t n_cand, int32_t reps, void* stream,
                              float* ms, int32_t* best);

/* Sampled head routing ("Google Speeds Up Video Diffusion on TPUs with
 * Optimized Sparse Attention", "Sparse Attention Patterns": the mask of each
 * head, spatial or temporal, is chosen from a sample). For every
 * head and every sampled query row, attention is computed with every key,
 * under the spatial mask and under the temporal mask (the masks of `spec`:
 * frame_window, temporal_band, sink_first_frame). The error of a mask is the
 * mean squared difference between its outputs and the dense ones over the
 * sampled rows and the head_dim output columns; kinds[h] receives the mask
 * with the smaller error (SVG_HEAD_SPATIAL on a tie).
 *   spec:   frames, grid_h, grid_w, num_heads and the two windows are read;
 *           head_kind and round_mode are ignored (head_kind may be NULL).
 *   q, k, v: device bf16 [num_heads][N][head_dim], 16-byte aligned, in the
 *           ORIGINAL frame-major order (routing precedes the layout step).
 *   head_dim: 64 or 128; scale > 0 and finite (normally 1/sqrt(head_dim)).
 *   rows:   host int32 [n_rows], original-order query indices in [0, N),
 *           drawn by the caller; 1 <= n_rows <= 65536; repeats allowed.
 *   err:    host float [num_heads][2] (spatial, temporal error), or NULL.
 *   kinds:  host int32 [num_heads].
 * The scores use bf16 inputs and fp32 accumulation; P is rounded to bf16
 * for the PV product, as in svg_attn_fwd. Uses one device scratch (V^T of
 * every head, num_heads*head_dim*(N+128)*2 bytes at most, plus per-split
 * partial results of about 1.6 KB per sampled row, head and split; about
 * 240 MB for 75,600 tokens, 10 heads, d = 128 and 756 rows), allocated on
 * the first call that needs it and kept per device, the largest so far,
 * until the process ends. Calls take a lock for their whole duration, so
 * calls from several host threads run one after another.
 * Synchronous: returns after the results are on the host.
 * Errors: INVALID_ARG, UNSUPPORTED (head_dim), ALIGNMENT, OOM, HIP. */
svg_status svg_route_heads(const svg_mask_spec* spec, const void* q,
                           const void* k, const void* v, int32_t head_dim,
                           float scale, const int32_t* rows, int32_t n_rows,
                           void* stream, float* err, int32_t* kinds);

/* svg_route_heads without any allocation, for callers that cannot allocate
 * device memory during the call (code under graph capture, tight serving
 * loops, harnesses that forbid allocation). Same arguments, results and
 * errors as svg_route_heads, plus UNSUPPORTED when the work does not fit
 * the library's scratch. The scratch is one 48 MiB device array per GPU
 * (kept until the process ends), used one head at a time: it must hold one
 * head's V^T (head_dim x (N + 128) bf16 values at most), the sampled rows,
 * their partial results over at least one key split (n_rows x 3 x
 * (head_dim + 2) floats per split) and their row errors, plus 12 bytes per
 * head; at head_dim 128 a head of up to about 130,000 tokens fits with a
 * few thousand sampled rows. Every call on one GPU uses the same array;
 * within a process the calls take a lock for their whole duration (they are
 * synchronous), so calls from several host threads run one after another,
 * on any GPU. Work that other code queues on the same GPU while a call runs
 * does not touch the array. Nothing in the array needs clearing between
 * calls: every value a call reads, it has written. Synchronous, like
 * svg_route_heads. */
svg_status svg_route_heads_noalloc(const svg_mask_spec* spec, const void* q,
                                   const void* k, const void* v,
                                   int32_t head_dim, float scale,
                                   const int32_t* rows, int32_t n_rows,
                                   void* stream, float* err, int32_t* kinds);

/* Token re-ordering between the original frame-major order t = f*S + s and
 * each head's kernel layout (temporal heads: p = s*F + f; other heads: p = t,
 * a plain copy). src, dst: device bf16 [num_heads][frames*tokens_per_frame]
 * [head_dim], 16-byte aligned, not overlapping. head_dim a multiple of 8, at
 * most 1024; one head (frames * tokens_per_frame * head_dim * 2 bytes) under
 * 2 GiB. head_kind: host [num_heads]. Queued on `stream` (one launch per run
 * of consecutive heads of one kind). Errors: INVALID_ARG, UNSUPPORTED
 * (head_dim, head size), ALIGNMENT, HIP. */
svg_status svg_permute_tokens(const void* src, void* dst, int32_t frames,
                              int32_t tokens_per_frame, int32_t num_heads,
                              int32_t head_dim, const int32_t* head_kind,
                              int32_t direction, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* svg_last_error(void);

/* SVG_ABI_VERSION of the library. */
int32_t svg_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SVG_ATTN_H */
