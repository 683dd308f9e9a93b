// Spatial blend of decoded pixel tiles on gfx950.
//
// Sources: mold issue #673, "Scope" (the VAE decode of a large frame is
// tiled spatially as well); DistVAE docs, "Choosing a tile window" (tiles
// and overlaps are set per spatial axis); LTX-2 docs, "Tiled Data
// Parallelism (TDP)", "What it is" (overlaps are blended with trapezoidal
// masks that sum to one).
//
// Latent tile [a, b) on an axis decodes to pixels [s*a, s*b), so the pixel
// tiling is the latent split scaled by s and neighbours overlap by s*o
// pixels; the windows are the latent trapezoids in pixel units.  Frames
// are not tiled.  Tiles (B, C, frames, rows, cols) are packed back to back
// in tile order; the output is (B, C, frames, H*s_h, W*s_w).
//
// The kernel is bound by HBM bandwidth (a fan-in of at most four tile
// reads per output element).  A workgroup owns a strip of 64 * E output
// columns (E = elements per 16-byte vector) and kPixRows output rows; each
// lane computes its columns' width covers and weights once and reuses them
// for every row, each wave takes consecutive rows, and a row's loads (up to
// two height and two width covers) are all issued before it is summed.
// Issuing the loads of all of a wave's rows first raises the registers to
// 117 and was slower (4 workgroups per CU); this form keeps 69.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "pixel_internal.h"

namespace tdp {
namespace {

constexpr int kBlock = 256;
constexpr int kPixRows = 16;  // output rows per workgroup (4 consecutive per wave)

template <int IN, int OUT>
__global__ __launch_bounds__(kBlock) void pixel_blend_kernel(const PixelDev p, const u32x4* __restrict__ tiles,
                                                             void* __restrict__ out, int n_strips) {
  constexpr int E = InVec<IN>::E;
  const int strip = blockIdx.x % n_strips;
  const int group = blockIdx.x / n_strips;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  // Columns x .. x+E-1 of this lane share their covers: s_w is a multiple
  // of E, so tile edges fall on vector boundaries.
  const int x = (strip * 64 + lane) * E;
  const bool col_ok = x < p.Wp;
  const int xc = col_ok ? x : 0;
  const Covers cw = split_covers(p.ax[1], (int)fastdiv((uint32_t)xc, p.by_s[1]));
  const int pw0 = p.s[1] * cw.s0, pw1 = p.s[1] * cw.s1;
  const int lx0 = xc - p.s[1] * cw.a0, lx1 = xc - p.s[1] * cw.a1;
  const bool two_w = cw.n > 1;
  const bool wave_two = __any(two_w);  // else every lane of the wave has one width cover
  float w0[E], w1[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    w0[e] = ramp(p.ax[1].n, p.o[1], cw.t0, lx0 + e, pw0);
    w1[e] = two_w ? ramp(p.ax[1].n, p.o[1], cw.t1, lx1 + e, pw1) : 0.0f;
  }

  constexpr int kPerWave = kPixRows / 4;
  for (int k = 0; k < kPerWave; ++k) {
    const int r = group * kPixRows + wave * kPerWave + k;  // wave-uniform
    if (r >= p.rows) break;
    const int bcf = (int)fastdiv((uint32_t)r, p.by_hp);
    const int y = r - bcf * p.Hp;
    const Covers ch = split_covers(p.ax[0], (int)fastdiv((uint32_t)y, p.by_s[0]));
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    // ascending tile index: (i0, j0), (i0, j1), (i1, j0), (i1, j1); both
    // height covers' loads are issued before either is summed
    u32x4 v[2][2];
    float wy[2];
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      if (hi >= ch.n) break;  // wave-uniform
      const int i = hi ? ch.t1 : ch.t0;
      const int ph = p.s[0] * (hi ? ch.s1 : ch.s0);
      const int ly = y - p.s[0] * (hi ? ch.a1 : ch.a0);
      wy[hi] = ramp(p.ax[0].n, p.o[0], i, ly, ph);
      const int64_t row0 = (int64_t)bcf * ph + ly;
      const int j1 = two_w ? cw.t1 : cw.t0;
      const int64_t e0 = pixel_tile_offset(p, i, cw.t0) + row0 * pw0 + lx0;
      const int64_t e1 = pixel_tile_offset(p, i, j1) + row0 * (two_w ? pw1 : pw0) + (two_w ? lx1 : lx0);
      v[hi][0] = ld_nt(tiles + e0 / E);
      v[hi][1] = wave_two ? ld_nt(tiles + e1 / E) : v[hi][0];
    }
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      if (hi >= ch.n) break;
      float a0[E], a1[E];
      InVec<IN>::unpack(v[hi][0], a0);
      InVec<IN>::unpack(v[hi][1], a1);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        acc[e] = fmaf(wy[hi] * w0[e], a0[e], acc[e]);
        acc[e] = two_w ? fmaf(wy[hi] * w1[e], a1[e], acc[e]) : acc[e];
      }
    }
    if (col_ok) store_out<OUT, E>(out, (int64_t)r * p.Wp + x, acc);
  }
}

template <int IN, int OUT>
hipError_t launch_pixel(const PixelDev& p, const void* tiles, void* out, hipStream_t s) {
  constexpr int E = InVec<IN>::E;
  const int n_strips = (p.Wp + 64 * E - 1) / (64 * E);
  const int64_t groups = ((int64_t)p.rows + kPixRows - 1) / kPixRows;
  hipLaunchKernelGGL((pixel_blend_kernel<IN, OUT>), dim3((unsigned)(groups * n_strips)), dim3(kBlock), 0, s, p,
                     reinterpret_cast<const u32x4*>(tiles), out, n_strips);
  return hipGetLastError();
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

}  // namespace
}  // namespace tdp

using namespace tdp;

extern "C" {

int tdp_pixel_blend(const tdp_pixel_plan* plan, const void* tiles, void* out, void* stream) {
  if (!plan) return fail(TDP_EINVAL, "tdp_pixel_blend: null plan");
  if (!tiles || !out) return fail(TDP_EINVAL, "tdp_pixel_blend: null device pointer");
  if (!aligned16(tiles) || !aligned16(out)) return fail(TDP_EINVAL, "tdp_pixel_blend: tiles and out must be 16-byte aligned");
  const PixelDev& p = plan->dev;
  // one launch: (groups of kPixRows rows) x (strips of 64 vectors) workgroups,
  // whose work-items a HIP launch counts in 32 bits
  const int64_t E = p.in_dtype == TDP_BF16 ? 8 : 4;
  const int64_t items = ((int64_t)p.rows + kPixRows - 1) / kPixRows * ((p.Wp + 64 * E - 1) / (64 * E)) * kBlock;
  if (items > 0xffffffffLL)
    return fail(TDP_ESHAPE, "tdp_pixel_blend: %lld work-items, more than one HIP launch holds (split the batch "
                            "or the frames over several plans)", (long long)items);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (p.in_dtype == TDP_BF16)
    e = p.out_dtype == TDP_BF16 ? launch_pixel<TDP_BF16, TDP_BF16>(p, tiles, out, s)
                                : launch_pixel<TDP_BF16, TDP_F32>(p, tiles, out, s);
  else
    e = p.out_dtype == TDP_BF16 ? launch_pixel<TDP_F32, TDP_BF16>(p, tiles, out, s)
                                : launch_pixel<TDP_F32, TDP_F32>(p, tiles, out, s);
  if (e != hipSuccess) return fail(TDP_EHIP, "tdp_pixel_blend: kernel launch failed: %s", hipGetErrorString(e));
  return TDP_OK;
}

}  // extern "C"
