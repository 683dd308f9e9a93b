// Pixel-tile plan shared by the host planner (pixel_plan.cpp) and the
// blend kernel (pixel.hip).
//
// Latent tile [a, b) on an axis decodes to pixels [s*a, s*b) (mold issue
// #673, "Scope"; DistVAE docs, "Choosing a tile window"), so the pixel
// tiling is the latent split of plan_internal.h scaled by s.
#pragma once

#include <stdint.h>

#include "plan_internal.h"

namespace tdp {

struct PixelDev {
  AxisSplit ax[2];   // latent split of height and width
  int32_t s[2];      // pixels per cell
  int32_t o[2];      // pixel overlaps s * overlap
  int32_t B, C, Fo;
  int32_t Hp, Wp;    // output pixel rows and columns
  int32_t rows;      // B * C * Fo * Hp output rows
  int32_t in_dtype, out_dtype;
  FastDiv by_s[2];   // pixel -> cell
  FastDiv by_hp;     // output row -> (b, c, f)
};

// Element offset of tile (i, j): B*C*Fo*s_h*s_w times the latent cells of
// the tiles before it in row-major order.
TDP_HD int64_t pixel_tile_offset(const PixelDev& p, int i, int j) {
  const int64_t cells = (int64_t)split_prefix(p.ax[0], i) * split_total(p.ax[1]) +
                        (int64_t)split_size(p.ax[0], i) * split_prefix(p.ax[1], j);
  return (int64_t)p.B * p.C * p.Fo * p.s[0] * p.s[1] * cells;
}

}  // namespace tdp

struct tdp_pixel_plan {
  tdp_pixel_config cfg;
  tdp::PixelDev dev;
  int64_t tile_elems, out_elems;
};
