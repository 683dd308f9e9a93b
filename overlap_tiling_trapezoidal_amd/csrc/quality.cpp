// Cost figures of a tiling: decoded area, largest tile, seams and the
// round-robin load per rank (DistVAE docs, "Choosing a tile window":
// sections "The two axes cost differently", "Clipping unbalances a grid,
// not the tile count" and "The tile count caps the GPU count").
//
// Host code only.  A tile's work is its cell count.  Tiles are the
// Cartesian product of the per-axis intervals in row-major order (last axis
// fastest) and tile t runs on rank t mod world (TDP docs, "What it is").
#include <stdint.h>
#include <string.h>

#include <vector>

#include "plan_internal.h"

using namespace tdp;

namespace {

constexpr int kMaxDims = 8;
constexpr int64_t kMaxQualityTiles = int64_t(1) << 20;

int quality(int ndim, const int32_t* dims, const int32_t* counts, const int32_t* starts, const int32_t* ends,
            int32_t world, tdp_quality* out, int64_t* rank_cells) {
  // per-axis interval lengths
  std::vector<std::vector<int64_t>> len(ndim);
  int64_t tiles = 1, grid = 1, off = 0;
  for (int d = 0; d < ndim; ++d) {
    for (int i = 0; i < counts[d]; ++i, ++off) {
      const int64_t a = starts[off], b = ends[off];
      if (a < 0 || b <= a || b > dims[d])
        return fail(TDP_EINVAL, "tdp_tiling_quality: axis %d interval %d = [%lld, %lld) is not inside [0, %d)", d,
                    i, (long long)a, (long long)b, dims[d]);
      len[d].push_back(b - a);
    }
    tiles *= counts[d];
    grid *= dims[d];
  }
  // Work per tile in row-major order; rank loads round-robin.
  std::vector<int64_t> rank(world, 0);
  int64_t total = 0, largest = 0;
  int idx[kMaxDims] = {0};
  for (int64_t t = 0; t < tiles; ++t) {
    int64_t cells = 1;
    for (int d = 0; d < ndim; ++d) cells *= len[d][idx[d]];
    total += cells;
    if (cells > largest) largest = cells;
    rank[t % world] += cells;
    for (int d = ndim - 1; d >= 0; --d) {  // advance the row-major index
      if (++idx[d] < counts[d]) break;
      idx[d] = 0;
    }
  }
  // Neighbour pairs along axis d: (counts[d] - 1) per line of the other axes.
  int64_t seams = 0;
  for (int d = 0; d < ndim; ++d) seams += (tiles / counts[d]) * (counts[d] - 1);
  int64_t max_rank = 0;
  for (int r = 0; r < world; ++r)
    if (rank[r] > max_rank) max_rank = rank[r];
  tdp_quality q;
  memset(&q, 0, sizeof q);
  q.total_cells = total;
  q.grid_cells = grid;
  q.largest_cells = largest;
  q.seams = seams;
  q.max_rank_cells = max_rank;
  q.area_ratio = (double)total / (double)grid;
  q.largest_fraction = (double)largest / (double)grid;
  q.imbalance = (double)max_rank * (double)world / (double)total - 1.0;
  *out = q;
  if (rank_cells)
    for (int r = 0; r < world; ++r) rank_cells[r] = rank[r];
  return TDP_OK;
}

}  // namespace

extern "C" {

int tdp_tiling_quality(int32_t ndim, const int32_t* dims, const int32_t* counts, const int32_t* starts,
                       const int32_t* ends, int32_t world, tdp_quality* out, int64_t* rank_cells) {
  if (!dims || !counts || !starts || !ends || !out) return fail(TDP_EINVAL, "tdp_tiling_quality: null argument");
  if (ndim < 1 || ndim > kMaxDims)
    return fail(TDP_EINVAL, "tdp_tiling_quality: ndim must be in [1, %d] (got %d)", kMaxDims, ndim);
  if (world < 1) return fail(TDP_EINVAL, "tdp_tiling_quality: world must be >= 1 (got %d)", world);
  int64_t tiles = 1;
  for (int d = 0; d < ndim; ++d) {
    if (dims[d] < 1) return fail(TDP_EINVAL, "tdp_tiling_quality: axis %d has length %d", d, dims[d]);
    if (counts[d] < 1 || counts[d] > kMaxQualityTiles)
      return fail(TDP_EINVAL, "tdp_tiling_quality: axis %d has %d intervals", d, counts[d]);
    tiles *= counts[d];
    if (tiles > kMaxQualityTiles)
      return fail(TDP_EINVAL, "tdp_tiling_quality: more than %lld tiles", (long long)kMaxQualityTiles);
  }
  return quality(ndim, dims, counts, starts, ends, world, out, rank_cells);
}

int tdp_plan_quality(const tdp_plan* plan, int32_t world, tdp_quality* out, int64_t* rank_cells) {
  if (!plan || !out) return fail(TDP_EINVAL, "tdp_plan_quality: null argument");
  if (world < 1) return fail(TDP_EINVAL, "tdp_plan_quality: world must be >= 1 (got %d)", world);
  const PlanDev& p = plan->dev;
  const int32_t dims[3] = {p.F, p.H, p.W};
  const int32_t counts[3] = {p.ax[0].n, p.ax[1].n, p.ax[2].n};
  std::vector<int32_t> starts, ends;
  for (int d = 0; d < 3; ++d)
    for (int i = 0; i < p.ax[d].n; ++i) {
      starts.push_back(split_start(p.ax[d], i));
      ends.push_back(split_start(p.ax[d], i) + split_size(p.ax[d], i));
    }
  return quality(3, dims, counts, starts.data(), ends.data(), world, out, rank_cells);
}

}  // extern "C"
