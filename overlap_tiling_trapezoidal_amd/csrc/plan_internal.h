// Internal plan representation shared by the host planner and the kernels.
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

constexpr int kMaxTiles = TDP_MAX_TILES_PER_AXIS;

// One axis of the split: n intervals [start[i], start[i] + size[i]).
struct AxisDev {
  int32_t dim;
  int32_t n;
  int32_t o;
  int32_t start[kMaxTiles];
  int32_t size[kMaxTiles];
  int32_t pre[kMaxTiles + 1];  // pre[i] = size[0] + ... + size[i-1]
};

// Everything a kernel needs about a plan; passed by value (kernel argument).
struct PlanDev {
  AxisDev ax[3];
  int32_t B, C, F, H, W;
  int32_t N;          // F * H * W generated tokens
  int32_t Nc;         // appended conditioning tokens
  int32_t T;          // number of tiles
  int32_t rows;       // N + Nc rows per batch element of latent / pos / out
  int32_t vin;        // 16-byte vectors per latent row
  int32_t in_dtype;
  int32_t out_dtype;
  int32_t normalize;  // subtract the per-tile offsets
  int32_t chunks;     // extent partials per (tile, batch element)
};

// Tile t -> per-axis tile index.
TDP_HD void tile_grid(const PlanDev& p, int t, int& i, int& j, int& k) {
  const int nh = p.ax[1].n, nw = p.ax[2].n;
  k = t % nw;
  j = (t / nw) % nh;
  i = t / (nw * nh);
}

// Generated tokens held by all tiles that precede tile (i, j, k) in
// row-major order: sum of sf*sh*sw over lexicographically smaller triples.
TDP_HD int64_t gen_before(const PlanDev& p, int i, int j, int k) {
  const int64_t SH = p.ax[1].pre[p.ax[1].n], SW = p.ax[2].pre[p.ax[2].n];
  return (int64_t)p.ax[0].pre[i] * SH * SW +
         (int64_t)p.ax[0].size[i] * ((int64_t)p.ax[1].pre[j] * SW + (int64_t)p.ax[1].size[j] * p.ax[2].pre[k]);
}

struct TileSlot {
  int64_t index_base;  // first tile_index entry (rows of one batch element)
  int64_t row_base;    // first row of the slot in tile_lat (B * capacity rows)
  int32_t gen;         // generated tokens
  int32_t cap;         // gen + Nc
};

TDP_HD TileSlot tile_slot(const PlanDev& p, int i, int j, int k) {
  const int t = (i * p.ax[1].n + j) * p.ax[2].n + k;
  TileSlot s;
  s.gen = p.ax[0].size[i] * p.ax[1].size[j] * p.ax[2].size[k];
  s.cap = s.gen + p.Nc;
  s.index_base = gen_before(p, i, j, k) + (int64_t)t * p.Nc;
  s.row_base = s.index_base * p.B;
  return s;
}

}  // namespace tdp

// The opaque handle of the public API.
struct tdp_plan {
  tdp_config cfg;
  tdp::PlanDev dev;
  bool guarded;
  int64_t total_index;  // sum over tiles of capacity
};

namespace tdp {
void set_error(const char* fmt, ...);
int fail(int status, const char* fmt, ...);
int dtype_bytes(int32_t dtype);
}  // namespace tdp
