/*
 * tdp.h — tiled-data-parallel (TDP) latent tiling on one MI355X (gfx950).
 *
 * The hot path is three operations, after the pages that describe TDP:
 *   plan    split a patchified (frames, height, width) latent into
 *           count-specified overlapping tiles, with trapezoidal windows
 *           (LTX-2 docs, "Tiled Data Parallelism (TDP)", sections "What it is"
 *           and "API"; mold issue #673, "Scope" and "A bug found while
 *           porting");
 *   extract gather each tile's latent rows, its normalized positions and the
 *           conditioning tokens it keeps (TDP docs, "Position normalization"
 *           and "Shared negative (reference) positions");
 *   blend   add the tile outputs back with the separable trapezoidal
 *           partition of unity, weight 1/k for a token kept by k tiles
 *           (TDP docs, "What it is" and "Shared negative (reference)
 *           positions").
 *
 * All tiles run on the calling GPU; what the multi-GPU form sums with one
 * all_reduce is accumulated in place here, with no GPU-to-GPU traffic.  A
 * rank plan runs one rank's round-robin share instead and writes that
 * rank's full-size partial sum, the input of the all_reduce.
 * Around it: plan-quality figures (decoded area, seams, round-robin
 * imbalance), a streaming blend that takes one tile at a time, and the blend
 * of decoded pixel tiles for a tiled VAE decode.
 *
 * Conventions
 *   - Every function returns TDP_OK (0) or a negative status; the message of
 *     the last failure on the calling thread is in tdp_last_error().
 *   - The library owns only the host plan.  Every device buffer is allocated
 *     and freed by the caller; the library never allocates device memory.
 *   - The device operations only enqueue work on `stream` (a hipStream_t,
 *     NULL = the null stream) and return without synchronizing.  All
 *     arguments are validated before anything is enqueued, so an error
 *     leaves every output untouched.
 *   - Results are deterministic: every output element has one writer and
 *     sums run in a fixed order; there are no atomics.
 *
 * Token and position layout (caller's tensors)
 *   latent    (B, N + Nc, C) row-major, dtype in_dtype; N = F*H*W generated
 *             tokens in patchified order n = (f*H + h)*W + w, followed by Nc
 *             conditioning tokens (TDP docs, "Shared negative (reference)
 *             positions": conditioning tokens are appended).
 *   pos       (B, 3, N + Nc, 2) float32: per token and axis (time, height,
 *             width) a [start, end) interval.
 *
 * Tile-major buffers (outputs of extract, input of blend)
 *   Tile t owns a fixed slot of capacity_t = gen_t + Nc rows per batch
 *   element; tile_count[t] = gen_t + kept_t rows of it are used: the gen_t
 *   generated tokens in tile-local row-major order, then the kept
 *   conditioning tokens in ascending original order.  Slot offsets are
 *   reported by tdp_plan_tile():
 *     tile_lat  + lat_offset   : (B, capacity_t, C)      dtype in_dtype
 *     tile_pos  + pos_offset   : (B, 3, capacity_t, 2)   float32
 *     tile_index+ index_offset : (capacity_t)            int32 source token
 *   Rows at and past tile_count[t] are not written.  A rank plan holds only
 *   its own tiles, in uniform slots, and indexes tile_count by slot
 *   (tdp_plan_create_rank).
 */
#ifndef TDP_H
#define TDP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define TDP_OK 0
#define TDP_EINVAL (-1) /* null pointer, bad count, bad dtype or flag       */
#define TDP_EGUARD (-2) /* overlap > dim/(n+1), or overlap on a 1-tile axis */
#define TDP_ESHAPE (-3) /* sizes out of the supported range                 */
#define TDP_EHIP (-4)   /* a HIP call or kernel launch failed               */

/* ---- dtypes and flags ---------------------------------------------------- */
#define TDP_F32 0
#define TDP_BF16 1

/* Shift each tile's positions so its generated tokens start at zero on every
 * axis (TDP docs, "Position normalization"; on by default upstream). */
#define TDP_NORMALIZE_POSITIONS 0x1u
/* Skip the overlap guard.  Plans built with it can be queried (intervals,
 * windows: used to study stacked windows) but tdp_extract and tdp_blend
 * refuse them with TDP_EGUARD. */
#define TDP_UNGUARDED 0x2u

#define TDP_MAX_TILES_PER_AXIS 32
#define TDP_MAX_WIDTH 4096
#define TDP_MAX_BATCH 1024
#define TDP_MAX_AXIS (1 << 26) /* cells per axis */
#define TDP_MAX_ROWS (1 << 29) /* tokens + conditioning per batch element (below) */

/* One axis of the tiling: a tile COUNT and an overlap in latent grid cells
 * (TDP docs, "API": DimensionTilingConfig(num_tiles, overlap)). */
typedef struct {
  int32_t num_tiles;
  int32_t overlap;
} tdp_axis_tiling;

typedef struct {
  int32_t batch;        /* 1 <= B <= TDP_MAX_BATCH                            */
  int32_t channels;     /* C >= 1; C * sizeof(in_dtype) a multiple of 16 B,   */
                        /* at most 1024 B                                     */
  int32_t frames;       /* 1 <= F <= TDP_MAX_AXIS latent grid                 */
  int32_t height;       /* 1 <= H <= TDP_MAX_AXIS                             */
  int32_t width;        /* 1 <= W <= TDP_MAX_WIDTH                            */
  int32_t num_cond;     /* Nc >= 0 conditioning tokens after the N generated; */
                        /* F*H*W + Nc < TDP_MAX_ROWS                          */
  tdp_axis_tiling axis[3]; /* frames, height, width (TDP docs, "API":       */
                           /* TileCountConfig)                                */
  int32_t in_dtype;     /* latent / tile dtype: TDP_F32 or TDP_BF16           */
  int32_t out_dtype;    /* blended output dtype: TDP_F32 or TDP_BF16 (RNE)    */
  uint32_t flags;       /* TDP_NORMALIZE_POSITIONS | TDP_UNGUARDED            */
} tdp_config;

typedef struct tdp_plan tdp_plan; /* opaque host object owned by the library */

typedef struct {
  int32_t index;         /* t = (i_f * n_h + i_h) * n_w + i_w                 */
  int32_t grid[3];       /* (i_f, i_h, i_w)                                   */
  int32_t origin[3];     /* first latent cell on each axis                    */
  int32_t shape[3];      /* cells on each axis                                */
  int32_t gen_tokens;    /* shape[0] * shape[1] * shape[2]                    */
  int32_t capacity;      /* gen_tokens + num_cond: slot rows per batch elem.  */
  int64_t lat_offset;    /* element offset of the slot in tile_lat/tile_out   */
  int64_t pos_offset;    /* float offset of the slot in tile_pos              */
  int64_t index_offset;  /* int32 offset of the slot in tile_index            */
                         /* (the three offsets are -1 for a tile that a rank  */
                         /* plan does not hold)                               */
} tdp_tile_info;

typedef struct {
  int32_t num_slots;        /* tiles the plan holds: T, or a rank's share;    */
                            /* entries of tile_count                          */
  int64_t tile_lat_elems;   /* elements of tile_lat (and tile_out)            */
  int64_t tile_pos_floats;  /* floats of tile_pos                             */
  int64_t tile_index_ints;  /* int32 entries of tile_index                    */
  int64_t cond_row_ints;    /* int32 entries of cond_row: T * Nc              */
  int64_t cond_k_ints;      /* int32 entries of cond_k: Nc                    */
  int64_t out_elems;        /* elements of out: B * (N + Nc) * C              */
  int64_t workspace_bytes;  /* device workspace of tdp_extract (0 if Nc == 0) */
} tdp_sizes;

/* ---- plan (host only; no GPU needed) ------------------------------------ */

/* Build a plan: split every axis with split_by_count, build the trapezoidal
 * windows and enumerate the tiles (mold #673, "Scope"; TDP docs, "API").
 *   split  a_i = floor(i * (dim - o) / n) for i = 0..n, tile i = [a_i,
 *          a_{i+1} + o); neighbours share exactly o cells, the last tile
 *          ends at dim.
 *   guard  o * (n + 1) <= dim (mold #673, "A bug found while porting":
 *          tile_size >= 2 * overlap); a 1-tile axis needs o == 0.
 *          Violations return TDP_EGUARD with a message naming the axis and
 *          the largest allowed overlap, unless TDP_UNGUARDED is set.
 *   also   n >= 1, o >= 0 (TDP_EINVAL); n <= dim - o, i.e. strides of at
 *          least one cell, and n <= TDP_MAX_TILES_PER_AXIS (TDP_ESHAPE).
 * On success *out receives a plan to release with tdp_plan_destroy. */
int tdp_plan_create(const tdp_config* cfg, tdp_plan** out);
void tdp_plan_destroy(tdp_plan* plan);

/* Number of tiles T = n_f * n_h * n_w: the product of the per-axis tile
 * counts of the TileCountConfig (TDP docs, "API"); 16 for the 4 x 4 split
 * that "What it is" runs on 4 GPUs.  TDP_EINVAL for a null argument. */
int tdp_plan_num_tiles(const tdp_plan* plan, int32_t* num_tiles);

/* The n intervals [starts[i], ends[i]) of one axis (0 frames, 1 height,
 * 2 width) as split_by_count lays them out (mold #673, "Scope"; the closed
 * form is tdp_plan_create's); both arrays hold at least n entries.
 * TDP_EINVAL for a null argument or an axis outside 0..2. */
int tdp_plan_intervals(const tdp_plan* plan, int axis, int32_t* starts, int32_t* ends);

/* The 1-D trapezoidal window of tile i on one axis, one fp32 per cell of
 * the interval (w has room for ends[i] - starts[i] floats): (j+1)/(o+1) on
 * the first o cells when a left neighbour exists, mirrored on the last o
 * cells when a right neighbour exists, 1 elsewhere, the product where both
 * apply (mold #673, "A bug found while porting"; TDP docs, "What it is").
 * Each value is the correctly rounded fp32 of the exact ratio. */
int tdp_plan_window(const tdp_plan* plan, int axis, int32_t i, float* w);

/* Tiles of one axis that contain cell x, ascending: tiles[0..*count), with
 * *count 1 or 2 (at most two overlap under the guard, which keeps every tile
 * at least twice the overlap: mold #673, "A bug found while porting").  This
 * is the lookup the kernels run for every latent row.  Guarded plans only. */
int tdp_plan_cell_tiles(const tdp_plan* plan, int axis, int32_t x, int32_t* tiles, int32_t* count);

/* Geometry and slot offsets of tile t, t = (i_f * n_h + i_h) * n_w + i_w:
 * the tile as one rank would run it (TDP docs, "What it is": each GPU
 * denoises its own tiles; mold #673, "Scope": tile enumeration), and where
 * tdp_extract puts its rows.  TDP_EINVAL for a null argument or t outside
 * [0, T). */
int tdp_plan_tile(const tdp_plan* plan, int32_t t, tdp_tile_info* info);

/* Sizes of every buffer the caller allocates for tdp_extract / tdp_blend:
 * the tile-major buffers hold each tile's latent slice, positions and kept
 * conditioning tokens (TDP docs, "Position normalization" and "Shared
 * negative (reference) positions"), plus the selection tables and the
 * workspace.  TDP_EINVAL for a null argument. */
int tdp_plan_sizes(const tdp_plan* plan, tdp_sizes* sizes);

/* Round-robin owner of tile t among `world` ranks: t mod world (TDP docs,
 * "What it is").  On one GPU every tile is local. */
int tdp_plan_tile_rank(const tdp_plan* plan, int32_t t, int32_t world, int32_t* rank);

/* ---- rank share (host only) ---------------------------------------------- */

/* The share of rank `rank` in a round-robin schedule of the plan's tiles over
 * `world` ranks (TDP docs, "What it is": tile t runs on rank t mod world,
 * every rank adds its tiles' weighted outputs into a full-size buffer and
 * one all_reduce sums the buffers).  The plan holds tiles rank, rank + world,
 * rank + 2*world, ...; local slot j = t / world.
 *   tdp_extract  writes the held tiles only: slot j of tile_lat, tile_pos
 *                and tile_index, and tile_count[j].  cond_row stays (T, Nc)
 *                for every tile, since k counts the tiles of all ranks.
 *   tdp_blend    writes the rank's partial sum over the whole output:
 *                sum over held tiles of W_t * y_t on generated rows and of
 *                (1/k) * y_t on conditioning rows, in ascending t; rows that
 *                no held tile covers are 0.  Summed over the ranks (in fp32,
 *                out_dtype TDP_F32), the partials give the whole plan's blend
 *                up to the order of the rank sum.
 *   tdp_blend_tile / tdp_blend_finish take whole plans only (TDP_EINVAL).
 * Slots are uniform: max over tiles of gen_tokens, plus num_cond, rows per
 * batch element; tdp_plan_tile gives each held tile's offsets.  A rank with
 * no tiles (rank >= T) holds none: its extract writes cond_row only and its
 * blend writes zeros.  world == 1 gives the whole plan.  Errors: TDP_EINVAL
 * for world < 1 or rank outside [0, world), otherwise as tdp_plan_create. */
int tdp_plan_create_rank(const tdp_config* cfg, int32_t world, int32_t rank, tdp_plan** out);

/* The plan's round-robin world and rank (1 and 0 for a whole plan) and the
 * number of tiles it holds (tiles dealt round-robin to ranks: TDP docs,
 * "What it is"). */
int tdp_plan_local_tiles(const tdp_plan* plan, int32_t* world, int32_t* rank, int32_t* count);

/* ---- plan quality (host only) -------------------------------------------- */

/* Cost figures of a tiling (DistVAE docs, "Choosing a tile window":
 * sections "The two axes cost differently", "Clipping unbalances a grid,
 * not the tile count" and "The tile count caps the GPU count").  A tile's
 * work is its cell count; tiles go to ranks round-robin, t mod world. */
typedef struct {
  int64_t total_cells;     /* sum over tiles of their cells (decoded work)    */
  int64_t grid_cells;      /* product of the axis lengths                     */
  int64_t largest_cells;   /* cells of the largest tile                       */
  int64_t seams;           /* pairs of tiles whose grid indices differ by one */
                           /* on exactly one axis                             */
  int64_t max_rank_cells;  /* cells of the heaviest rank                      */
  double area_ratio;       /* total_cells / grid_cells                        */
  double largest_fraction; /* largest_cells / grid_cells (activations held)   */
  double imbalance;        /* max_rank_cells / (total_cells / world) - 1;     */
                           /* idle ranks (world > tiles) count in the split   */
} tdp_quality;

/* Cost figures of a tiling (DistVAE docs, "Choosing a tile window": "The
 * two axes cost differently" for decoded area and seams, "Clipping
 * unbalances a grid, not the tile count" for the load imbalance of an even
 * tile count per rank, "The tile count caps the GPU count" for idle ranks).
 * Figures of any tiling given as per-axis intervals: ndim axes (1..8) of
 * lengths dims[d], counts[d] >= 1 intervals each, listed axis after axis in
 * starts/ends (sum of counts entries, 0 <= start < end <= dims[d]); tiles
 * are their Cartesian product in row-major order (at most 2^20 tiles).
 * rank_cells: NULL or `world` int64 entries, the cells of each rank.
 * Returns TDP_EINVAL for null or malformed arguments or world < 1. */
int tdp_tiling_quality(int32_t ndim, const int32_t* dims, const int32_t* counts, const int32_t* starts,
                       const int32_t* ends, int32_t world, tdp_quality* out, int64_t* rank_cells);

/* The same figures for a plan's generated-token tiles (frames, height,
 * width), e.g. to choose tile counts and overlaps before running (same
 * passages as tdp_tiling_quality). */
int tdp_plan_quality(const tdp_plan* plan, int32_t world, tdp_quality* out, int64_t* rank_cells);

/* ---- device operations (enqueue on `stream`) ----------------------------- */

/* Gather all tiles, every latent row read once.  Without conditioning
 * tokens this is one launch; with them an extent launch first leaves each
 * tile's partial extents and cleared look-back flags in `workspace`, and a
 * second launch selects and copies the conditioning tokens along with the
 * generated rows (tdp_set_lookback_polls).
 *   in   latent (B, N+Nc, C) in_dtype; pos (B, 3, N+Nc, 2) float32.
 *   out  tile_lat, tile_pos, tile_index: tile-major slots (layout above).
 *        tile_count (one per slot: T, or a rank's share) int32:
 *          gen_t + kept_t.
 *        cond_row (T * Nc) int32: row of conditioning token c inside tile
 *          t's slot, or -1 when t does not keep it.
 *        cond_k (Nc) int32: k, the number of tiles that keep token c (the
 *          non-negative entries of column c of cond_row); the blend weighs
 *          the token by 1/k (TDP docs, "Shared negative (reference)
 *          positions").  cond_row and cond_k may be NULL when Nc == 0.
 *   workspace  device scratch of tdp_sizes.workspace_bytes bytes, 16-byte
 *        aligned (NULL allowed when that is 0).  Caller-owned; its contents
 *        between calls mean nothing, and calls that share it must not
 *        overlap.
 * Positions: the tile's offset on axis d for batch element b is the minimum
 * start over its generated tokens; with TDP_NORMALIZE_POSITIONS it is
 * subtracted from both ends of every row the tile holds (one fp32
 * subtraction each), otherwise positions are copied (TDP docs, "Position
 * normalization").
 * Selection: tile t keeps conditioning token c when, for some batch
 * element, c's interval overlaps the tile's extent [min start, max end) on
 * all three axes (half-open: touching or empty intervals do not overlap) or
 * c's time start is negative (TDP docs, "Shared negative (reference)
 * positions"); tested on positions before normalization.  Positions must be
 * finite.
 * All pointers are device pointers except `plan`; latent/tile_lat 16-byte
 * aligned, pos/tile_pos 8-byte aligned; buffers must not overlap and hold
 * the sizes tdp_plan_sizes() reports (the library cannot check sizes).
 * Returns TDP_EGUARD for unguarded plans, TDP_EINVAL for null or misaligned
 * pointers, TDP_EHIP on launch failure.  TDP_ESHAPE, nothing enqueued, when
 * the plan is too large for HIP's launches: every device call of a plan
 * (extract, blend and their halves and steps) first adds up the work-items
 * of all the workgroups its launches use and refuses a sum above 2^32 - 1,
 * the 32-bit work-item count of one launch (only plans of hundreds of
 * millions of rows reach it; split the batch or the latent). */
int tdp_extract(const tdp_plan* plan, const void* latent, const float* pos,
                void* tile_lat, float* tile_pos, int32_t* tile_index,
                int32_t* tile_count, int32_t* cond_row, int32_t* cond_k,
                void* workspace, void* stream);

/* Conditioning selection (Nc > 0; the keep rule of TDP docs, "Shared
 * negative (reference) positions"), the second launch of tdp_extract: one
 * workgroup per (tile, chunk of 64 tokens) tests its chunk and finds the
 * tile's kept tokens before it: those of the 16 chunks before it from
 * their tokens, those of earlier chunks from the flags their workgroups
 * publish (look-back).  A flag still unpublished after `polls` reads is not
 * waited for: the workgroup counts that chunk from its tokens itself, so
 * the result never depends on the order in which workgroups start and no
 * wait is unbounded.  The default is 256 reads; 0 counts every unpublished
 * chunk at once.  Results are the same for every value.  Process-wide;
 * applies to every call that runs the selection (tdp_extract,
 * tdp_extract_noalloc, tdp_extract_positions, tdp_pipeline_step) enqueued
 * afterwards.
 * TDP_EINVAL for polls < 0. */
int tdp_set_lookback_polls(int32_t polls);

/* Largest workspace tdp_extract_noalloc serves (1 MiB: the look-back flags
 * take 4 bytes per tile and 64 conditioning tokens, so T * Nc up to about
 * 16 million; tdp_sizes gives a plan's figure). */
#define TDP_STATIC_SCRATCH_BYTES (1 << 20)

/* tdp_extract without the workspace argument, for callers that cannot
 * allocate device memory: work recorded under stream capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The selection tables go to a
 * static device array of TDP_STATIC_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends; its address is
 * looked up once per device, on the first call with that device current.
 * No allocation, and no clearing by the host: the extent launch clears
 * the look-back flags before the selection reads them.  Arguments, layouts,
 * ownership, results and errors as tdp_extract; in addition TDP_EINVAL
 * (nothing enqueued) when the plan's tdp_sizes.workspace_bytes exceed
 * TDP_STATIC_SCRATCH_BYTES, and TDP_EHIP when the array's address cannot be
 * found.  All calls on one GPU share the array, which keeps the last call's
 * contents: calls that may run at the same time on one GPU (two streams, or
 * threads without ordering) race and give wrong tables; calls in order on
 * one stream are safe. */
int tdp_extract_noalloc(const tdp_plan* plan, const void* latent, const float* pos,
                        void* tile_lat, float* tile_pos, int32_t* tile_index,
                        int32_t* tile_count, int32_t* cond_row, int32_t* cond_k,
                        void* stream);

/* Blend tile outputs (tile-major slots with tile_lat's layout and dtype,
 * rows as tdp_extract placed them) into out (B, N+Nc, C) out_dtype:
 *   generated token:    sum over covering tiles t, ascending, of
 *                       (wF*wH)*wW * y_t  (separable trapezoid),
 *   conditioning token: (1/k) * sum over the tiles that keep it, ascending
 *                       (rows from cond_row, k = cond_k[c]); 0 when k == 0,
 * fp32 accumulation, no normalization pass (mold #673, "A bug found while
 * porting"), bf16 output rounded to nearest even.  cond_row and cond_k are
 * tdp_extract's outputs for the same plan (NULL allowed when Nc == 0).
 * Device pointers except `plan`; tile_out/out 16-byte aligned, cond_row and
 * cond_k 4-byte aligned. */
int tdp_blend(const tdp_plan* plan, const void* tile_out, const int32_t* cond_row,
              const int32_t* cond_k, void* out, void* stream);

/* One step of a pipelined loop, for callers that have the extract of one
 * latent and the blend of an earlier latent's tile outputs ready together
 * (latents in flight one after another, each tiled, its tiles denoised and
 * their outputs blended back: TDP docs, "What it is").  Enqueues what
 * tdp_extract(plan, latent, ..., workspace) followed by tdp_blend(plan,
 * tile_out, blend_cond_row, blend_cond_k, out) would, with bit-identical
 * results.  For whole plans without conditioning tokens both run as one
 * launch, the extract's workgroups first, so the blend's fill the GPU while
 * the extract's drain (a rank's share too: its tiles' extract and its
 * partial buffer); plans with conditioning tokens take two launches (the
 * extents with the blend, then the selection with the positions and the
 * latent rows), a rank's share too.
 * The two halves may run at the same time, so the blend's buffers must be
 * none of the extract's: TDP_EINVAL, nothing enqueued, when tile_out,
 * blend_cond_row or blend_cond_k overlaps a buffer the extract writes, or
 * out overlaps a buffer the extract reads or writes (extents from
 * tdp_plan_sizes).  Other arguments, alignments and errors as the two
 * calls; one plan serves both halves. */
int tdp_pipeline_step(const tdp_plan* plan, const void* latent, const float* pos,
                      void* tile_lat, float* tile_pos, int32_t* tile_index,
                      int32_t* tile_count, int32_t* cond_row, int32_t* cond_k,
                      void* workspace, const void* tile_out,
                      const int32_t* blend_cond_row, const int32_t* blend_cond_k,
                      void* out, void* stream);

/* The extract in two halves, for callers whose positions stay the same
 * over many latents (the positions grid of a denoising stage).  Each tile's
 * shift is its generated tokens' minimum start (TDP docs, "Position
 * normalization") and a conditioning token's keep test reads only its
 * interval and the tile's (TDP docs, "Shared negative (reference)
 * positions"), so everything but the latent rows is a function of the
 * positions alone.
 *
 * tdp_extract_positions writes what tdp_extract writes except tile_lat:
 * tile_pos, tile_index, tile_count and, when Nc > 0, cond_row and cond_k,
 * bit-identical to tdp_extract on the same plan and positions.  Arguments,
 * layouts, workspace and errors as tdp_extract without latent and
 * tile_lat. */
int tdp_extract_positions(const tdp_plan* plan, const float* pos, float* tile_pos,
                          int32_t* tile_index, int32_t* tile_count, int32_t* cond_row,
                          int32_t* cond_k, void* workspace, void* stream);

/* tdp_extract_latent writes tile_lat from latent (B, N+Nc, C) in_dtype:
 * every held tile's generated rows (its slice of the grid, TDP docs, "What
 * it is") and its kept conditioning rows at the slot rows cond_row gives.
 * cond_row (T, Nc) int32 must come from tdp_extract_positions or
 * tdp_extract on the same plan and positions (NULL allowed when Nc == 0);
 * with it, tile_lat is bit-identical to tdp_extract's (an entry outside
 * [0, capacity) of its tile is skipped, so no row lands outside the tile's
 * slot).  One launch, no
 * workspace, no waiting between workgroups.  Device pointers except plan;
 * latent and tile_lat 16-byte aligned, cond_row 4-byte aligned; TDP_EINVAL
 * for a null or misaligned pointer (nothing enqueued), TDP_EHIP when the
 * launch fails. */
int tdp_extract_latent(const tdp_plan* plan, const void* latent, const int32_t* cond_row,
                       void* tile_lat, void* stream);

/* One step of a pipelined loop over latents that share one positions set
 * (latents in flight one after another, each tiled and blended back: TDP
 * docs, "What it is"):
 * tdp_extract_latent(plan, latent, cond_row, tile_lat) and tdp_blend(plan,
 * tile_out, blend_cond_row, blend_cond_k, out), bit-identical to the two
 * calls.  One launch, the gather's workgroups first (rank plans too: the
 * held tiles' rows, then the partial buffer).  cond_row and
 * blend_cond_row may be the same buffer (both halves only read them).
 * TDP_EINVAL, nothing enqueued, when tile_lat overlaps tile_out,
 * blend_cond_row, blend_cond_k or out, or out overlaps latent or cond_row
 * (extents from tdp_plan_sizes).  Other arguments, alignments and errors as
 * the two calls. */
int tdp_pipeline_latent_step(const tdp_plan* plan, const void* latent, const int32_t* cond_row,
                             void* tile_lat, const void* tile_out,
                             const int32_t* blend_cond_row, const int32_t* blend_cond_k,
                             void* out, void* stream);

/* Streaming blend, for schedules that produce one tile output at a time
 * (TDP docs, "What it is": a rank runs its tiles in turn and their blended
 * outputs are accumulated in place).  Adds tile t's outputs into the fp32
 * accumulator acc (B, N+Nc, C): generated rows weighted (wF*wH)*wW, kept
 * conditioning rows weighted 1/k.  tile_out is tile t's slot alone,
 * (B, capacity_t, C) in_dtype with the rows tdp_extract placed there
 * (tdp_tile_info.capacity, .gen_tokens), so it may live in its own buffer.
 * A voxel's first covering tile and a token's first keeping tile (smallest
 * index) overwrite acc instead of adding, so acc needs no clearing; tokens
 * no tile keeps are set to 0 at t = 0.  Call for t = 0, 1, ..., T-1 in this
 * order on one stream: acc then holds tdp_blend's fp32 sums bit for bit.
 * Any other order gives wrong sums.  Calls that share acc must not overlap.
 * tile_out/acc 16-byte aligned device pointers; cond_row and cond_k as for
 * tdp_blend.
 * Returns TDP_EINVAL for a bad tile index or pointer, or a rank plan;
 * TDP_ESHAPE (nothing enqueued) when this launch or tdp_blend_finish's
 * would exceed 2^32 - 1 work-items, so a streaming sequence is refused at
 * its first call; TDP_EHIP when the launch fails. */
int tdp_blend_tile(const tdp_plan* plan, int32_t t, const void* tile_out, const int32_t* cond_row,
                   const int32_t* cond_k, float* acc, void* stream);

/* The last step of the streaming blend (the in-place sum of TDP docs, "What
 * it is", rounded once): round the accumulator (B, N+Nc, C) fp32 to the
 * plan's out_dtype into out
 * (round to nearest even for bf16; a copy for fp32, nothing when out == acc).
 * After tdp_blend_tile for every tile in order, out equals tdp_blend's
 * output bit for bit.  16-byte aligned device pointers.  TDP_EINVAL for a
 * null or misaligned pointer or a rank plan, TDP_ESHAPE as tdp_blend_tile,
 * TDP_EHIP when the launch fails. */
int tdp_blend_finish(const tdp_plan* plan, const float* acc, void* out, void* stream);

/* ---- spatial blend of decoded pixel tiles --------------------------------- */

/* The VAE decode of a large frame is tiled too (mold #673, "Scope"; DistVAE
 * docs, "Choosing a tile window"): latent tile [a, b) on an axis decodes to
 * pixels [scale*a, scale*b), so neighbouring pixel tiles overlap by
 * scale*overlap pixels and are recombined with the same trapezoids in pixel
 * units (ramps over the overlapping pixels; TDP docs, "What it is").  Height
 * and width are tiled; frames are not. */
typedef struct tdp_pixel_plan tdp_pixel_plan;

typedef struct {
  int32_t batch;           /* B >= 1                                            */
  int32_t channels;        /* C >= 1 decoded channels (3 for RGB)               */
  int32_t frames;          /* decoded frames, >= 1 (not tiled)                  */
  int32_t height, width;   /* latent cells H, W (<= TDP_MAX_AXIS)               */
  int32_t scale[2];        /* pixels per latent cell on height and width; the   */
                           /* width scale times the element size is a multiple  */
                           /* of 16 bytes                                       */
  tdp_axis_tiling axis[2]; /* latent tiling of height and width (guarded)       */
  int32_t in_dtype;        /* decoded tiles: TDP_F32 or TDP_BF16                */
  int32_t out_dtype;       /* blended frame: TDP_F32 or TDP_BF16 (RNE)          */
} tdp_pixel_config;

typedef struct {
  int32_t index;           /* t = i_h * n_w + i_w                              */
  int32_t grid[2];         /* (i_h, i_w)                                       */
  int32_t origin[2];       /* first pixel row and column                       */
  int32_t shape[2];        /* pixel rows and columns                           */
  int64_t offset;          /* element offset of the tile in the tile buffer    */
  int64_t elems;           /* B * C * frames * rows * columns                  */
} tdp_pixel_tile;

/* Validate and build (host only).  TDP_EINVAL for a null argument, a bad
 * dtype or a scale below one; TDP_EGUARD as tdp_plan_create; TDP_ESHAPE when
 * the width scale does not fill 16-byte vectors or sizes leave int32 range
 * (B*C*frames*H*scale_h rows). */
int tdp_pixel_plan_create(const tdp_pixel_config* cfg, tdp_pixel_plan** out);
void tdp_pixel_plan_destroy(tdp_pixel_plan* plan);
/* Tile t's place: tiles are packed back to back in index order (row-major
 * over height and width, as the latent tiles: mold #673, "Scope"), each a
 * (B, C, frames, rows, columns) array of in_dtype. */
int tdp_pixel_plan_tile(const tdp_pixel_plan* plan, int32_t t, tdp_pixel_tile* out);
/* Elements of the tile buffer and of the output (B, C, frames, H*scale_h,
 * W*scale_w), the decoded image the tiles come from (mold #673, "Scope");
 * tile count. */
int tdp_pixel_plan_sizes(const tdp_pixel_plan* plan, int64_t* tile_elems, int64_t* out_elems,
                         int32_t* num_tiles);

/* out = sum over the tiles covering each pixel, ascending t, of
 * (wH * wW) * tile, fp32 accumulation from zero, rounded once to out_dtype
 * (the trapezoids of the latent blend in pixel units, so the weights still
 * sum to one: DistVAE docs, "Choosing a tile window"; mold #673, "Scope").
 * Device pointers, 16-byte aligned; tiles holds every tile as packed above.
 * TDP_EINVAL for a null or misaligned pointer, TDP_ESHAPE (nothing
 * enqueued) when the launch would exceed 2^32 - 1 work-items, TDP_EHIP when
 * it fails. */
int tdp_pixel_blend(const tdp_pixel_plan* plan, const void* tiles, void* out, void* stream);

/* ---- errors ------------------------------------------------------------ */
/* Errors are reported, never produced silently, and a guard violation names
 * the axis and the largest overlap it allows (mold #673, "A bug found while
 * porting": the guard overlap <= dim / (n + 1)).  tdp_status_string names a
 * status code (a static string; "unknown status" for other values). */
const char* tdp_status_string(int status);
/* The message of the last failure on the calling thread (thread-local,
 * never NULL; "" before the first failure), naming the axis and limit of a
 * guard violation as above (mold #673, "A bug found while porting"). */
const char* tdp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TDP_H */
