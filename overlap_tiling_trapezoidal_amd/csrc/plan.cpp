// Host planner: split_by_count, overlap guard, trapezoidal windows, tile
// enumeration and buffer sizes.  Pure host code; it needs no GPU.
//
// Sources: LTX-2 docs, "Tiled Data Parallelism (TDP)", sections "What it is"
// and "API"; mold issue #673, sections "Scope" and "A bug found while
// porting".
#include <limits.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>

#include "plan_internal.h"

namespace tdp {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int dtype_bytes(int32_t dtype) {
  switch (dtype) {
    case TDP_F32: return 4;
    case TDP_BF16: return 2;
    default: return 0;
  }
}

static const char* kAxisName[3] = {"frames", "height", "width"};

// Validate one axis.  The split itself (a_i = floor(i*(dim-o)/n), tile i =
// [a_i, a_{i+1} + o)) is the closed form in plan_internal.h, shared with the
// kernels: neighbours overlap by exactly o cells and the last tile ends at dim.
int build_axis(int d, int32_t dim, tdp_axis_tiling t, bool guarded, AxisSplit* ax) {
  const char* name = kAxisName[d];
  if (t.num_tiles < 1) return fail(TDP_EINVAL, "%s: num_tiles must be >= 1 (got %d)", name, t.num_tiles);
  if (t.overlap < 0) return fail(TDP_EINVAL, "%s: overlap must be >= 0 (got %d)", name, t.overlap);
  if (t.num_tiles > TDP_MAX_TILES_PER_AXIS)
    return fail(TDP_ESHAPE, "%s: %d tiles exceed the limit of %d per axis", name, t.num_tiles,
                TDP_MAX_TILES_PER_AXIS);
  if (t.num_tiles == 1 && t.overlap != 0)
    return fail(TDP_EGUARD, "%s: an untiled axis (1 tile) must request overlap 0 (got %d)", name, t.overlap);
  const int64_t free_len = (int64_t)dim - t.overlap;
  if (free_len < t.num_tiles)
    return fail(TDP_ESHAPE,
                "%s: %d tiles with overlap %d on %d cells leave a stride below one cell; "
                "use at most %lld tiles or a smaller overlap",
                name, t.num_tiles, t.overlap, dim, (long long)(free_len > 0 ? free_len : 0));
  if (guarded && (int64_t)t.overlap * (t.num_tiles + 1) > dim)
    return fail(TDP_EGUARD,
                "%s: overlap %d exceeds dim/(n+1) = %d/%d, so three windows would stack; "
                "reduce overlap on %s to <= %d or use fewer tiles",
                name, t.overlap, dim, t.num_tiles + 1, name, dim / (t.num_tiles + 1));
  if (dim > TDP_MAX_AXIS)
    return fail(TDP_ESHAPE, "%s: %d cells exceed the limit of %d per axis", name, dim, TDP_MAX_AXIS);
  ax->dim = dim;
  ax->n = t.num_tiles;
  ax->o = t.overlap;
  ax->by_n = make_fastdiv((uint32_t)t.num_tiles);
  ax->size_min = (int32_t)(free_len / t.num_tiles) + t.overlap;
  ax->by_size[0] = make_fastdiv((uint32_t)ax->size_min);
  ax->by_size[1] = make_fastdiv((uint32_t)ax->size_min + 1);
  ax->by_s = make_fastdiv((uint32_t)free_len);
  for (int i = 0; i < ax->n; ++i) {
    const int sz = split_size(*ax, i);
    if (sz != ax->size_min && sz != ax->size_min + 1)
      return fail(TDP_ESHAPE, "%s: internal error: tile %d has size %d outside {%d, %d}", name, i, sz,
                  ax->size_min, ax->size_min + 1);
  }
  return TDP_OK;
}

}  // namespace tdp

using namespace tdp;

// A whole plan (world == 1) or the share of one rank of a round-robin
// schedule over `world` ranks.
static int create_plan(const tdp_config* cfg, int32_t world, int32_t rank, tdp_plan** out) {
  const tdp_config c = *cfg;
  if (c.batch < 1 || c.channels < 1 || c.frames < 1 || c.height < 1 || c.width < 1)
    return fail(TDP_EINVAL, "batch, channels, frames, height and width must all be >= 1");
  if (c.num_cond < 0) return fail(TDP_EINVAL, "num_cond must be >= 0 (got %d)", c.num_cond);
  if (c.batch > TDP_MAX_BATCH) return fail(TDP_ESHAPE, "batch %d exceeds %d", c.batch, TDP_MAX_BATCH);
  const int ein = dtype_bytes(c.in_dtype), eout = dtype_bytes(c.out_dtype);
  if (!ein) return fail(TDP_EINVAL, "in_dtype must be TDP_F32 or TDP_BF16 (got %d)", c.in_dtype);
  if (!eout) return fail(TDP_EINVAL, "out_dtype must be TDP_F32 or TDP_BF16 (got %d)", c.out_dtype);
  if (c.flags & ~(TDP_NORMALIZE_POSITIONS | TDP_UNGUARDED))
    return fail(TDP_EINVAL, "unknown flag bits 0x%x", c.flags & ~(TDP_NORMALIZE_POSITIONS | TDP_UNGUARDED));
  const int64_t row_bytes = (int64_t)c.channels * ein;
  if (row_bytes % 16 != 0 || row_bytes > 1024)
    return fail(TDP_ESHAPE,
                "channels * element size must be a multiple of 16 bytes and at most 1024 bytes (got %lld)",
                (long long)row_bytes);
  if (c.width > TDP_MAX_WIDTH) return fail(TDP_ESHAPE, "width %d exceeds %d", c.width, TDP_MAX_WIDTH);
  const int64_t N = (int64_t)c.frames * c.height * c.width;
  const int64_t rows = N + c.num_cond;
  if ((int64_t)c.batch * rows > INT32_MAX || N > INT32_MAX)
    return fail(TDP_ESHAPE, "batch * (tokens + conditioning) = %lld exceeds the int32 range",
                (long long)((int64_t)c.batch * rows));
  if (rows >= TDP_MAX_ROWS)
    return fail(TDP_ESHAPE, "tokens + conditioning = %lld per batch element exceed the limit of %d",
                (long long)rows, TDP_MAX_ROWS);

  const bool guarded = !(c.flags & TDP_UNGUARDED);
  PlanDev dev;
  memset(&dev, 0, sizeof dev);
  const int32_t dims[3] = {c.frames, c.height, c.width};
  for (int d = 0; d < 3; ++d) {
    const int st = build_axis(d, dims[d], c.axis[d], guarded, &dev.ax[d]);
    if (st != TDP_OK) return st;
  }
  dev.B = c.batch;
  dev.C = c.channels;
  dev.F = c.frames;
  dev.H = c.height;
  dev.W = c.width;
  dev.N = (int32_t)N;
  dev.Nc = c.num_cond;
  dev.T = dev.ax[0].n * dev.ax[1].n * dev.ax[2].n;
  dev.rows = (int32_t)rows;
  dev.vin = (int32_t)(row_bytes / 16);
  dev.in_dtype = c.in_dtype;
  dev.out_dtype = c.out_dtype;
  dev.normalize = (c.flags & TDP_NORMALIZE_POSITIONS) ? 1 : 0;

  int64_t max_gen = 0;
  for (int i = 0; i < dev.ax[0].n; ++i)
    for (int j = 0; j < dev.ax[1].n; ++j)
      for (int k = 0; k < dev.ax[2].n; ++k) {
        const int64_t g =
            (int64_t)split_size(dev.ax[0], i) * split_size(dev.ax[1], j) * split_size(dev.ax[2], k);
        if (g > max_gen) max_gen = g;
      }

  // Tile slots.  Whole plan: capacities packed back to back, (sum of gen)
  // + T * Nc.  Rank plan: its tiles t = rank, rank + world, ... in uniform
  // slots of max gen + Nc rows.
  dev.world = world;
  dev.rank = rank;
  dev.by_world = make_fastdiv((uint32_t)world);
  dev.T_local = rank < dev.T ? (int32_t)(((int64_t)dev.T - rank + world - 1) / world) : 0;
  int64_t total_index;
  if (world == 1) {
    dev.slot_cap = 0;
    total_index = (int64_t)split_total(dev.ax[0]) * split_total(dev.ax[1]) * split_total(dev.ax[2]) +
                  (int64_t)dev.T * c.num_cond;
  } else {
    if (max_gen + c.num_cond > INT32_MAX)
      return fail(TDP_ESHAPE, "tile capacity of %lld rows exceeds the int32 range",
                  (long long)(max_gen + c.num_cond));
    dev.slot_cap = (int32_t)(max_gen + c.num_cond);
    total_index = (int64_t)dev.T_local * dev.slot_cap;
  }
  if (total_index * c.batch > INT32_MAX)
    return fail(TDP_ESHAPE, "tile buffers of %lld rows exceed the int32 range",
                (long long)(total_index * c.batch));

  dev.rpp = kThreads / dev.vin;
  dev.lpr = (dev.vin + 1) / 2;  // vin <= 64, so lpr <= 32 and a wave holds at least two rows
  dev.rwv = 64 / dev.lpr;
  dev.lat_rows = dev.rwv;
  dev.lat_chunks = (dev.W + dev.lat_rows - 1) / dev.lat_rows;
  dev.blend_rows = dev.rwv;
  dev.blend_chunks = (dev.W + dev.blend_rows - 1) / dev.blend_rows;
  dev.gen_units = dev.B * dev.F * dev.H * dev.blend_chunks;  // <= B * N < 2^31
  dev.by_vin = make_fastdiv((uint32_t)dev.vin);
  dev.by_lpr = make_fastdiv((uint32_t)dev.lpr);
  dev.by_H = make_fastdiv((uint32_t)dev.H);
  dev.by_FH = make_fastdiv((uint32_t)(dev.F * dev.H));
  dev.by_lat_chunks = make_fastdiv((uint32_t)dev.lat_chunks);
  dev.by_blend_chunks = make_fastdiv((uint32_t)dev.blend_chunks);

  // Bounding box of the held tiles (rank plans launch the latent copy over
  // it only; the blend writes zeros outside it without reading anything).
  int lo[3] = {INT_MAX, INT_MAX, INT_MAX}, hi[3] = {0, 0, 0};
  for (int64_t t = rank; t < dev.T; t += world) {
    int g[3];
    tile_grid(dev, (int)t, g[0], g[1], g[2]);
    for (int d = 0; d < 3; ++d) {
      const int a = split_start(dev.ax[d], g[d]);
      if (a < lo[d]) lo[d] = a;
      if (a + split_size(dev.ax[d], g[d]) > hi[d]) hi[d] = a + split_size(dev.ax[d], g[d]);
    }
  }
  if (dev.T_local > 0) {
    dev.box_f0 = lo[0];
    dev.box_nf = hi[0] - lo[0];
    dev.box_h0 = lo[1];
    dev.box_nh = hi[1] - lo[1];
    dev.box_w0 = lo[2];
    dev.box_nw = hi[2] - lo[2];
    dev.box_c0 = lo[2] / dev.lat_rows;
    dev.box_nc = (hi[2] + dev.lat_rows - 1) / dev.lat_rows - dev.box_c0;
  }
  // Position workgroups per (tile, batch element, axis) plane.  Every part
  // re-reads the rest of the plane for its minimum start, and those
  // re-reads are kept below 3/4 of the latent bytes the plan reads so that
  // on large latents they do not compete with the latent copy.  Two paths
  // (the launch picks one, with the occupancy cap):
  //  - one pass: a part holds its tokens in registers (at most kThreads *
  //    kPosOwnRows) while the minimum is reduced, so the plan uses the
  //    fewest parts that fit (4K-class latent: extract 21.1 -> 20.0 us);
  //  - two passes (minimum, then the part's copy from L2): parts of at
  //    most 1024 rows shorten the copy chain, which the smaller latents
  //    gain from (full-res 6.8 us against 7.1 us one-pass).
  // Measured: 4 parts beat 2 and 8 on the 4K-class latent.
  {
    const int64_t cells = world == 1 ? N : (int64_t)dev.box_nf * dev.box_nh * dev.box_nw;
    const int64_t latent_bytes = (int64_t)c.batch * cells * row_bytes;
    const int64_t plane_bytes = (int64_t)dev.T_local * c.batch * 3 * max_gen * 8;
    auto parts_for = [&](int64_t hold) {
      int64_t parts = (max_gen + hold - 1) / hold;
      if (plane_bytes > 0 && parts * plane_bytes * 4 > latent_bytes * 3) parts = latent_bytes * 3 / (plane_bytes * 4);
      if (parts < 1) parts = 1;
      if (parts > kMaxExtParts) parts = kMaxExtParts;
      return (int32_t)parts;
    };
    dev.pos_parts = parts_for(1024);
    dev.pos_parts_one = dev.normalize ? parts_for((int64_t)kThreads * kPosOwnRows) : dev.pos_parts;
  }
  // Workspace of the conditioning selection (every tile is tested, rank
  // plans included, since k counts the tiles of all ranks).
  if (c.num_cond > 0) {
    dev.n_chunks = (c.num_cond + kCondChunk - 1) / kCondChunk;
    // extent parts: about kExtPartBytes of positions (B * 3 planes of 8-byte
    // pairs per row) each, at least one row per part
    const int64_t row_bytes_pos = (int64_t)c.batch * 3 * 8;
    int64_t rows = kExtPartBytes / row_bytes_pos;
    if (rows < 1) rows = 1;
    int64_t parts = (max_gen + rows - 1) / rows;
    if (parts > kMaxExtParts) parts = kMaxExtParts;
    dev.ext_parts = (int32_t)parts;
    dev.ext_rows = (int32_t)((max_gen + parts - 1) / parts);
  }
  dev.lat_units = world == 1 ? dev.B * dev.F * dev.H * dev.lat_chunks : dev.B * dev.box_nf * dev.box_nh * dev.box_nc;
  // a rank's blend computes its box units (the extract's) and zero-fills the
  // rest of every line of its full-size partial buffer, one workgroup a line
  if (world > 1) dev.gen_units = dev.lat_units;
  dev.zero_lines = world > 1 ? dev.B * dev.F * dev.H : 0;
  dev.by_box_h = make_fastdiv((uint32_t)(dev.box_nh > 0 ? dev.box_nh : 1));
  dev.by_box_fh = make_fastdiv((uint32_t)(dev.box_nf * dev.box_nh > 0 ? dev.box_nf * dev.box_nh : 1));
  dev.by_box_c = make_fastdiv((uint32_t)(dev.box_nc > 0 ? dev.box_nc : 1));

  tdp_plan* p = new (std::nothrow) tdp_plan;
  if (!p) return fail(TDP_EINVAL, "out of host memory");
  p->cfg = c;
  p->dev = dev;
  p->guarded = guarded;
  p->total_index = total_index;
  *out = p;
  return TDP_OK;
}

extern "C" {

int tdp_plan_create(const tdp_config* cfg, tdp_plan** out) {
  if (!cfg || !out) return fail(TDP_EINVAL, "tdp_plan_create: null argument");
  *out = nullptr;
  return create_plan(cfg, 1, 0, out);
}

int tdp_plan_create_rank(const tdp_config* cfg, int32_t world, int32_t rank, tdp_plan** out) {
  if (!cfg || !out) return fail(TDP_EINVAL, "tdp_plan_create_rank: null argument");
  *out = nullptr;
  if (world < 1) return fail(TDP_EINVAL, "world must be >= 1 (got %d)", world);
  if (rank < 0 || rank >= world) return fail(TDP_EINVAL, "rank %d out of range [0, %d)", rank, world);
  return create_plan(cfg, world, rank, out);
}

int tdp_plan_local_tiles(const tdp_plan* plan, int32_t* world, int32_t* rank, int32_t* count) {
  if (!plan || !world || !rank || !count) return fail(TDP_EINVAL, "tdp_plan_local_tiles: null argument");
  *world = plan->dev.world;
  *rank = plan->dev.rank;
  *count = plan->dev.T_local;
  return TDP_OK;
}

void tdp_plan_destroy(tdp_plan* plan) { delete plan; }

int tdp_plan_num_tiles(const tdp_plan* plan, int32_t* num_tiles) {
  if (!plan || !num_tiles) return fail(TDP_EINVAL, "tdp_plan_num_tiles: null argument");
  *num_tiles = plan->dev.T;
  return TDP_OK;
}

int tdp_plan_intervals(const tdp_plan* plan, int axis, int32_t* starts, int32_t* ends) {
  if (!plan || !starts || !ends) return fail(TDP_EINVAL, "tdp_plan_intervals: null argument");
  if (axis < 0 || axis > 2) return fail(TDP_EINVAL, "axis must be 0, 1 or 2 (got %d)", axis);
  const AxisSplit& ax = plan->dev.ax[axis];
  for (int i = 0; i < ax.n; ++i) {
    starts[i] = split_start(ax, i);
    ends[i] = split_start(ax, i) + split_size(ax, i);
  }
  return TDP_OK;
}

int tdp_plan_window(const tdp_plan* plan, int axis, int32_t i, float* w) {
  if (!plan || !w) return fail(TDP_EINVAL, "tdp_plan_window: null argument");
  if (axis < 0 || axis > 2) return fail(TDP_EINVAL, "axis must be 0, 1 or 2 (got %d)", axis);
  const AxisSplit& ax = plan->dev.ax[axis];
  if (i < 0 || i >= ax.n) return fail(TDP_EINVAL, "tile index %d out of range [0, %d)", i, ax.n);
  const int size = split_size(ax, i), o = ax.o;
  for (int j = 0; j < size; ++j) {
    // Exact ratios are formed in double (numerator and denominator are
    // small integers, so each ratio is one rounding) and the product of the
    // two ramps, when both apply, is rounded once more to float.
    double v = 1.0;
    if (i > 0 && j < o) v *= (double)(j + 1) / (double)(o + 1);
    if (i < ax.n - 1 && j >= size - o) v *= (double)(size - j) / (double)(o + 1);
    w[j] = (float)v;
  }
  return TDP_OK;
}

int tdp_plan_cell_tiles(const tdp_plan* plan, int axis, int32_t x, int32_t* tiles, int32_t* count) {
  if (!plan || !tiles || !count) return fail(TDP_EINVAL, "tdp_plan_cell_tiles: null argument");
  if (axis < 0 || axis > 2) return fail(TDP_EINVAL, "axis must be 0, 1 or 2 (got %d)", axis);
  if (!plan->guarded) return fail(TDP_EGUARD, "tdp_plan_cell_tiles: plan was built with TDP_UNGUARDED");
  const AxisSplit& ax = plan->dev.ax[axis];
  if (x < 0 || x >= ax.dim) return fail(TDP_EINVAL, "cell %d out of range [0, %d)", x, ax.dim);
  const Covers c = split_covers(ax, x);
  tiles[0] = c.t0;
  tiles[1] = c.t1;
  *count = c.n;
  return TDP_OK;
}

int tdp_plan_tile(const tdp_plan* plan, int32_t t, tdp_tile_info* info) {
  if (!plan || !info) return fail(TDP_EINVAL, "tdp_plan_tile: null argument");
  const PlanDev& p = plan->dev;
  if (t < 0 || t >= p.T) return fail(TDP_EINVAL, "tile index %d out of range [0, %d)", t, p.T);
  int i, j, k;
  tile_grid(p, t, i, j, k);
  const TileSlot s = tile_slot(p, i, j, k);
  info->index = t;
  info->grid[0] = i;
  info->grid[1] = j;
  info->grid[2] = k;
  const int g[3] = {i, j, k};
  for (int d = 0; d < 3; ++d) {
    info->origin[d] = split_start(p.ax[d], g[d]);
    info->shape[d] = split_size(p.ax[d], g[d]);
  }
  info->gen_tokens = s.gen;
  info->capacity = s.cap;
  const bool held = tile_is_local(p, t);
  info->lat_offset = held ? s.row_base * p.C : -1;
  info->pos_offset = held ? s.row_base * 6 : -1;
  info->index_offset = held ? s.index_base : -1;
  return TDP_OK;
}

int tdp_plan_sizes(const tdp_plan* plan, tdp_sizes* sizes) {
  if (!plan || !sizes) return fail(TDP_EINVAL, "tdp_plan_sizes: null argument");
  const PlanDev& p = plan->dev;
  sizes->num_slots = p.T_local;
  sizes->tile_lat_elems = plan->total_index * p.B * p.C;
  sizes->tile_pos_floats = plan->total_index * p.B * 6;
  sizes->tile_index_ints = plan->total_index;
  sizes->cond_row_ints = (int64_t)p.T * p.Nc;
  sizes->cond_k_ints = p.Nc;
  sizes->out_elems = (int64_t)p.B * p.rows * p.C;
  sizes->workspace_bytes = ws_layout(p).bytes;
  return TDP_OK;
}

int tdp_plan_tile_rank(const tdp_plan* plan, int32_t t, int32_t world, int32_t* rank) {
  if (!plan || !rank) return fail(TDP_EINVAL, "tdp_plan_tile_rank: null argument");
  if (t < 0 || t >= plan->dev.T) return fail(TDP_EINVAL, "tile index %d out of range [0, %d)", t, plan->dev.T);
  if (world < 1) return fail(TDP_EINVAL, "world must be >= 1 (got %d)", world);
  *rank = t % world;
  return TDP_OK;
}

const char* tdp_status_string(int status) {
  switch (status) {
    case TDP_OK: return "TDP_OK";
    case TDP_EINVAL: return "TDP_EINVAL: invalid argument";
    case TDP_EGUARD: return "TDP_EGUARD: overlap guard violated (overlap > dim/(n+1))";
    case TDP_ESHAPE: return "TDP_ESHAPE: size out of the supported range";
    case TDP_EHIP: return "TDP_EHIP: HIP runtime error";
    default: return "unknown status";
  }
}

const char* tdp_last_error(void) { return g_last_error; }

}  // extern "C"
