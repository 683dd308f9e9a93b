// Host planner of the pixel-tile blend: validates a tdp_pixel_config and
// lays the decoded tiles out back to back in tile order (mold issue #673,
// "Scope": the VAE decode is tiled spatially; DistVAE docs, "Choosing a
// tile window": tiles and overlaps per spatial axis).  Plain C++, no GPU
// code, so it builds with a host compiler too.
#include <stdint.h>
#include <string.h>

#include <new>

#include "pixel_internal.h"

using namespace tdp;

extern "C" {

int tdp_pixel_plan_create(const tdp_pixel_config* cfg, tdp_pixel_plan** out) {
  if (!cfg || !out) return fail(TDP_EINVAL, "tdp_pixel_plan_create: null argument");
  *out = nullptr;
  const tdp_pixel_config c = *cfg;
  if (c.batch < 1 || c.channels < 1 || c.frames < 1)
    return fail(TDP_EINVAL, "batch, channels and frames must be >= 1 (got %d, %d, %d)", c.batch, c.channels,
                c.frames);
  if (c.height < 1 || c.width < 1) return fail(TDP_EINVAL, "latent height and width must be >= 1");
  if (c.scale[0] < 1 || c.scale[1] < 1)
    return fail(TDP_EINVAL, "scale must be >= 1 pixel per cell (got %d, %d)", c.scale[0], c.scale[1]);
  const int ein = dtype_bytes(c.in_dtype), eout = dtype_bytes(c.out_dtype);
  if (!ein || !eout) return fail(TDP_EINVAL, "dtypes must be TDP_F32 or TDP_BF16");
  PixelDev d;
  memset(&d, 0, sizeof d);
  const int32_t dims[2] = {c.height, c.width};
  for (int a = 0; a < 2; ++a) {
    const int st = build_axis(1 + a, dims[a], c.axis[a], true, &d.ax[a]);
    if (st != TDP_OK) return st;
  }
  const int vec = 16 / ein;
  if (c.scale[1] % vec != 0)
    return fail(TDP_ESHAPE,
                "width scale %d: pixel tiles must start and end on 16-byte vectors, so it must be a multiple of "
                "%d for this input dtype",
                c.scale[1], vec);
  const int64_t hp = (int64_t)c.height * c.scale[0], wp = (int64_t)c.width * c.scale[1];
  const int64_t rows = (int64_t)c.batch * c.channels * c.frames * hp;
  if (hp > INT32_MAX || wp > INT32_MAX || rows > INT32_MAX)
    return fail(TDP_ESHAPE, "%lld output rows of %lld pixels exceed the int32 range", (long long)rows,
                (long long)wp);
  for (int a = 0; a < 2; ++a) {
    d.s[a] = c.scale[a];
    d.o[a] = c.axis[a].overlap * c.scale[a];
    d.by_s[a] = make_fastdiv((uint32_t)c.scale[a]);
  }
  d.B = c.batch;
  d.C = c.channels;
  d.Fo = c.frames;
  d.Hp = (int32_t)hp;
  d.Wp = (int32_t)wp;
  d.rows = (int32_t)rows;
  d.in_dtype = c.in_dtype;
  d.out_dtype = c.out_dtype;
  d.by_hp = make_fastdiv((uint32_t)hp);
  tdp_pixel_plan* p = new (std::nothrow) tdp_pixel_plan;
  if (!p) return fail(TDP_EINVAL, "out of host memory");
  p->cfg = c;
  p->dev = d;
  p->tile_elems = (int64_t)c.batch * c.channels * c.frames * c.scale[0] * c.scale[1] *
                  ((int64_t)split_total(d.ax[0]) * split_total(d.ax[1]));
  p->out_elems = rows * wp;
  *out = p;
  return TDP_OK;
}

void tdp_pixel_plan_destroy(tdp_pixel_plan* plan) { delete plan; }

int tdp_pixel_plan_tile(const tdp_pixel_plan* plan, int32_t t, tdp_pixel_tile* out) {
  if (!plan || !out) return fail(TDP_EINVAL, "tdp_pixel_plan_tile: null argument");
  const PixelDev& d = plan->dev;
  const int T = d.ax[0].n * d.ax[1].n;
  if (t < 0 || t >= T) return fail(TDP_EINVAL, "tile index %d out of range [0, %d)", t, T);
  const int i = t / d.ax[1].n, j = t % d.ax[1].n;
  tdp_pixel_tile r;
  r.index = t;
  r.grid[0] = i;
  r.grid[1] = j;
  r.origin[0] = d.s[0] * split_start(d.ax[0], i);
  r.origin[1] = d.s[1] * split_start(d.ax[1], j);
  r.shape[0] = d.s[0] * split_size(d.ax[0], i);
  r.shape[1] = d.s[1] * split_size(d.ax[1], j);
  r.offset = pixel_tile_offset(d, i, j);
  r.elems = (int64_t)d.B * d.C * d.Fo * r.shape[0] * r.shape[1];
  *out = r;
  return TDP_OK;
}

int tdp_pixel_plan_sizes(const tdp_pixel_plan* plan, int64_t* tile_elems, int64_t* out_elems, int32_t* num_tiles) {
  if (!plan || !tile_elems || !out_elems || !num_tiles) return fail(TDP_EINVAL, "tdp_pixel_plan_sizes: null argument");
  *tile_elems = plan->tile_elems;
  *out_elems = plan->out_elems;
  *num_tiles = plan->dev.ax[0].n * plan->dev.ax[1].n;
  return TDP_OK;
}

}  // extern "C"
