// Internal plan representation shared by the host planner and the kernels.
//
// The split of an axis is a closed form (mold issue #673, "A bug found
// while porting", and TDP docs, "API": n tiles per axis overlapping by o
// cells): with s = dim - o,
//   start a_i = floor(i * s / n)           i = 0..n   (a_n = s)
//   tile  i   = [a_i, a_{i+1} + o)
//   size      = a_{i+1} + o - a_i
//   prefix    = a_i + i * o                 (sizes of tiles 0..i-1)
// so kernels and host compute every interval quantity from (dim, n, o) with
// the same functions below, instead of reading tables.
#pragma once

#include <stdint.h>

#include "tdp.h"

#if defined(__HIPCC__) || defined(__HIP__)
#include <hip/hip_runtime.h>
#define TDP_HD __host__ __device__ inline
#else
#define TDP_HD inline
#endif

namespace tdp {

// Unsigned division by an invariant d >= 1 for numerators up to 2^31, by
// multiplication (Granlund & Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994): with l = ceil(log2 d) and
// m = floor(2^32 * (2^l - d) / d) + 1, q = (mulhi(m, x) + x) >> l.
struct FastDiv {
  uint32_t m;
  uint32_t l;
};
TDP_HD FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  FastDiv f;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  f.l = l;
  return f;
}
TDP_HD uint32_t fastdiv(uint32_t x, const FastDiv& f) {
  const uint32_t hi = (uint32_t)(((uint64_t)f.m * x) >> 32);
  return (hi + x) >> f.l;
}

struct AxisSplit {
  int32_t dim;         // cells on the axis (<= TDP_MAX_AXIS, so products stay at most 2^31)
  int32_t n;           // tiles on the axis
  int32_t o;           // overlap in cells
  int32_t size_min;    // floor(s / n) + o: every tile size is size_min or size_min + 1
  FastDiv by_n;        // division by n
  FastDiv by_s;        // division by s = dim - o
  FastDiv by_size[2];  // division by size_min and size_min + 1
};

// i * s <= n * dim <= 32 * 2^26 = 2^31: unsigned, and within fastdiv's range.
TDP_HD int split_start(const AxisSplit& a, int i) {
  return (int)fastdiv((uint32_t)i * (uint32_t)(a.dim - a.o), a.by_n);
}
TDP_HD int split_size(const AxisSplit& a, int i) { return split_start(a, i + 1) + a.o - split_start(a, i); }
TDP_HD int split_prefix(const AxisSplit& a, int i) { return split_start(a, i) + i * a.o; }
TDP_HD int split_total(const AxisSplit& a) { return a.dim + (a.n - 1) * a.o; }

// Division by the size of a tile on this axis (x < 2^31).
TDP_HD uint32_t div_by_size(const AxisSplit& a, uint32_t x, int size) {
  return fastdiv(x, size == a.size_min ? a.by_size[0] : a.by_size[1]);
}

// The last tile that contains cell x: the largest i with a_i <= x.
// a_i <= x  <=>  i * s < (x + 1) * n  <=>  i <= ((x + 1) * n - 1) / s.
TDP_HD int split_last_cover(const AxisSplit& a, int x) {
  const int i = (int)fastdiv((uint32_t)(x + 1) * (uint32_t)a.n - 1u, a.by_s);  // <= 2^31 - 1
  return i < a.n - 1 ? i : a.n - 1;
}

// Tiles containing cell x, ascending (at most two when o*(n+1) <= dim):
// the last cover i always contains x; tile i-1 also does iff x < a_i + o.
struct Covers {
  int n;       // 1 or 2
  int t0, t1;  // tile indices, t0 < t1 when n == 2
  int a0, a1;  // their starts
  int s0, s1;  // their sizes
};
TDP_HD Covers split_covers(const AxisSplit& a, int x) {
  Covers c;
  const int i = split_last_cover(a, x);
  const int ai = split_start(a, i);
  const int si = split_start(a, i + 1) + a.o - ai;
  if (i > 0 && x < ai + a.o) {
    const int ap = split_start(a, i - 1);
    c.n = 2;
    c.t0 = i - 1;
    c.a0 = ap;
    c.s0 = ai + a.o - ap;
    c.t1 = i;
    c.a1 = ai;
    c.s1 = si;
  } else {
    c.n = 1;
    c.t0 = c.t1 = i;
    c.a0 = c.a1 = ai;
    c.s0 = c.s1 = si;
  }
  return c;
}

// Launch shape shared by the host planner and the kernels.
constexpr int kThreads = 256;   // threads per workgroup
constexpr int kPosOwnRows = 16;  // position rows per thread one extract position workgroup holds
// Conditioning-token selection (plans with Nc > 0): an extent launch ahead
// of the extract launch reduces partial extents of each tile (parts of about
// kExtPartBytes of positions, every workgroup small, since one compute unit
// reads only a few tens of GB/s); in the extract launch each wave then tests
// one chunk of kCondChunk tokens against one tile and finds the tile's kept
// tokens before its chunk by look-back over the earlier chunks' flags.
constexpr int kCondChunk = 64;                 // one token per lane of a wave
constexpr int kExtPartBytes = 48 * 1024;       // position bytes one extent workgroup reads
constexpr int kMaxExtParts = 64;              // extent parts per tile at most

// Everything a kernel needs about a plan; passed by value (kernel argument).
struct PlanDev {
  AxisSplit ax[3];
  int32_t B, C, F, H, W;
  int32_t N;          // F * H * W generated tokens
  int32_t Nc;         // appended conditioning tokens
  int32_t T;          // number of tiles
  int32_t rows;       // N + Nc rows per batch element of latent / pos / out
  int32_t vin;        // 16-byte vectors per latent row
  int32_t in_dtype;
  int32_t out_dtype;
  int32_t normalize;  // subtract the per-tile offsets
  int32_t pos_parts;      // position workgroups per (tile, batch element, axis), two-pass path
  int32_t pos_parts_one;  // the same for the one-pass path (parts held in registers)
  // Launch geometry and invariant divisors (multiply-shift), from the host:
  int32_t rpp;        // rows per workgroup pass, one vector per lane: kThreads / vin
  // Generated rows of extract and blend: each lane moves two vectors of one
  // row, q and lpr + q, so lpr = ceil(vin / 2) lanes share a row and a wave
  // holds rwv = 64 / lpr rows.  The unit of work is one wave's rows of one
  // (b, f, h) line; a workgroup takes kThreads / 64 consecutive units.
  int32_t lpr, rwv;
  int32_t lat_rows, lat_chunks;      // extract: rows per wave unit (rwv), units per line
  int32_t blend_rows, blend_chunks;  // blend: rows per wave unit (rwv), units per line
  int32_t lat_units, gen_units;      // wave units of extract and of blend (whole latent, or a rank's box)
  int32_t zero_lines;                // rank plans: B * F * H lines whose rows outside the box the blend zeroes
  FastDiv by_vin, by_lpr, by_H, by_FH, by_lat_chunks, by_blend_chunks;
  // Round-robin share (TDP docs, "What it is": tile t runs on rank t mod
  // world).  world == 1 is the whole plan.  A rank plan holds the tiles with
  // t mod world == rank, local index t / world, in uniform slots of
  // slot_cap rows per batch element.
  int32_t world, rank;
  int32_t T_local;    // tiles of this plan's rank (T when world == 1)
  int32_t slot_cap;   // rank plans: largest tile's gen + Nc
  FastDiv by_world;
  // Rank plans: bounding box of the held tiles, [f0, f0+nf) x [h0, h0+nh)
  // x [w0, w0+nw) cells; on width also as extract chunks [c0, c0+nc) (all
  // zero without tiles).
  int32_t box_f0, box_nf, box_h0, box_nh, box_c0, box_nc;
  int32_t box_w0, box_nw;  // the same box on width, in cells
  FastDiv by_box_h, by_box_fh, by_box_c;
  // Conditioning selection (Nc > 0): chunks of kCondChunk tokens, extent
  // parts of ext_rows rows per tile (WsLayout places their tables).
  int32_t n_chunks, ext_parts, ext_rows;
};

// Workspace of the conditioning selection: byte offsets of its tables, each
// 256-byte aligned (every size is 0 when Nc == 0):
//   part  (T, ext_parts, B, 3) float2  [min start, max end) over one part of a tile's rows
//   flags (T, n_chunks) uint32  look-back word of each (tile, chunk): 0 until
//         published, then a status bit and the chunk's kept count or the
//         tile's kept count up to and including the chunk
// Derived from the plan in closed form, so kernels need no extra arguments.
struct WsLayout {
  int64_t part, flags, bytes;
};
TDP_HD int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }
TDP_HD WsLayout ws_layout(const PlanDev& p) {
  WsLayout w;
  w.part = 0;
  w.flags = align256((int64_t)p.T * p.ext_parts * p.B * 3 * 8);
  w.bytes = p.Nc > 0 ? w.flags + align256((int64_t)p.T * p.n_chunks * 4) : 0;
  return w;
}

// Tile t -> per-axis tile index (row-major, width fastest).
TDP_HD void tile_grid(const PlanDev& p, int t, int& i, int& j, int& k) {
  const int nh = p.ax[1].n, nw = p.ax[2].n;
  k = t % nw;
  j = (t / nw) % nh;
  i = t / (nw * nh);
}

// Generated tokens held by all tiles that precede tile (i, j, k) in
// row-major order: sum of sf*sh*sw over lexicographically smaller triples.
TDP_HD int64_t gen_before(const PlanDev& p, int i, int j, int k) {
  const int64_t SH = split_total(p.ax[1]), SW = split_total(p.ax[2]);
  return (int64_t)split_prefix(p.ax[0], i) * SH * SW +
         (int64_t)split_size(p.ax[0], i) *
             ((int64_t)split_prefix(p.ax[1], j) * SW + (int64_t)split_size(p.ax[1], j) * split_prefix(p.ax[2], k));
}

struct TileSlot {
  int64_t index_base;  // first tile_index entry (rows of one batch element)
  int64_t row_base;    // first row of the slot in tile_lat (B * capacity rows)
  int32_t gen;         // generated tokens
  int32_t cap;         // gen + Nc
};

// Whole plan: tiles packed back to back in index order.
TDP_HD TileSlot tile_slot_whole(const PlanDev& p, int i, int j, int k) {
  const int t = (i * p.ax[1].n + j) * p.ax[2].n + k;
  TileSlot s;
  s.gen = split_size(p.ax[0], i) * split_size(p.ax[1], j) * split_size(p.ax[2], k);
  s.cap = s.gen + p.Nc;
  s.index_base = gen_before(p, i, j, k) + (int64_t)t * p.Nc;
  s.row_base = s.index_base * p.B;
  return s;
}

TDP_HD bool tile_is_local(const PlanDev& p, int t) {
  return (int)((uint32_t)t - fastdiv((uint32_t)t, p.by_world) * (uint32_t)p.world) == p.rank;
}

// Rank plan: local tile t / world in a slot of slot_cap rows per batch
// element (meaningful for the rank's own tiles only).
TDP_HD TileSlot tile_slot_rank(const PlanDev& p, int i, int j, int k) {
  const int t = (i * p.ax[1].n + j) * p.ax[2].n + k;
  TileSlot s;
  s.gen = split_size(p.ax[0], i) * split_size(p.ax[1], j) * split_size(p.ax[2], k);
  s.cap = s.gen + p.Nc;
  s.index_base = (int64_t)fastdiv((uint32_t)t, p.by_world) * p.slot_cap;
  s.row_base = s.index_base * p.B;
  return s;
}

TDP_HD TileSlot tile_slot(const PlanDev& p, int i, int j, int k) {
  return p.world > 1 ? tile_slot_rank(p, i, j, k) : tile_slot_whole(p, i, j, k);
}

}  // namespace tdp

// The opaque handle of the public API.
struct tdp_plan {
  tdp_config cfg;
  tdp::PlanDev dev;
  bool guarded;
  int64_t total_index;  // tile_index entries: sum of the slots' capacities
};

namespace tdp {
// Validate axis d (0 frames, 1 height, 2 width) of length dim and fill *ax.
int build_axis(int d, int32_t dim, tdp_axis_tiling t, bool guarded, AxisSplit* ax);
void set_error(const char* fmt, ...);
int fail(int status, const char* fmt, ...);
int dtype_bytes(int32_t dtype);
}  // namespace tdp
