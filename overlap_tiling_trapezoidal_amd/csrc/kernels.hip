// gfx950 kernels for the tiled hot path: extract (extents, conditioning
// selection, gather) and blend (owner-computes weighted sum).
//
// Sources: LTX-2 docs, "Tiled Data Parallelism (TDP)", sections "What it is",
// "Position normalization" and "Shared negative (reference) positions";
// mold issue #673, "A bug found while porting" (blend has no normalization
// pass).
//
// Data movement is the whole cost: every kernel is bound by HBM bandwidth.
// Latent rows move as 16-byte vectors (one global_load/store_dwordx4 per
// lane), V lanes per row, 256 / V rows per 256-thread workgroup pass.
// Nothing is a contraction, so no MFMA is used.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "plan_internal.h"

namespace tdp {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kGatherUnroll = 8;   // latent rows in flight per thread (extract)
constexpr int kCondRowsPerBlock = 64;
constexpr int kMaxCombos = 4;      // <= 2 covering tiles on frames x 2 on height
constexpr int kNoTile = 0xFF;

// ---------------------------------------------------------------------------
// Axis helpers
// ---------------------------------------------------------------------------

// Tiles of one axis that contain cell x, ascending; at most two under the
// overlap guard.  Returns how many were found.
__device__ inline int axis_covers(const AxisDev& ax, int x, int* ti, int* tl) {
  int c = 0;
  for (int i = 0; i < ax.n; ++i) {
    const int l = x - ax.start[i];
    if (l >= 0 && l < ax.size[i] && c < 2) {
      ti[c] = i;
      tl[c] = l;
      ++c;
    }
  }
  return c;
}

// 1-D trapezoid of tile i at local cell l: (l+1)/(o+1) on a left ramp,
// (size-l)/(o+1) on a right ramp, 1 elsewhere.  IEEE division (the build
// keeps fp32 division correctly rounded), so each value equals the host
// plan's window bit for bit.
__device__ inline float axis_weight(const AxisDev& ax, int i, int l) {
  float w = 1.0f;
  const float den = (float)(ax.o + 1);
  if (i > 0 && l < ax.o) w = (float)(l + 1) / den;
  if (i < ax.n - 1 && l >= ax.size[i] - ax.o) w *= (float)(ax.size[i] - l) / den;
  return w;
}

__device__ inline int pack_covers(int c, const int* ti) {
  const int a = c > 0 ? ti[0] : kNoTile;
  const int b = c > 1 ? ti[1] : kNoTile;
  return a | (b << 8);
}

// ---------------------------------------------------------------------------
// Reductions
// ---------------------------------------------------------------------------

__device__ inline float wave_min(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Offset (minimum start) and extent end (maximum end) of tile t, batch b,
// axis d, from the per-chunk partials written by extents_kernel.
__device__ inline float2 tile_extent(const PlanDev& p, const float* __restrict__ part, int t, int b, int d) {
  const float* q = part + ((int64_t)(t * p.B + b) * p.chunks) * 6 + d * 2;
  float lo = INFINITY, hi = -INFINITY;
  for (int c = 0; c < p.chunks; ++c) {
    lo = fminf(lo, q[c * 6]);
    hi = fmaxf(hi, q[c * 6 + 1]);
  }
  return make_float2(lo, hi);
}

// ---------------------------------------------------------------------------
// bf16 / f32 vectors
// ---------------------------------------------------------------------------

__device__ inline uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Unpack one 16-byte input vector into E floats.
template <int IN>  // IN = TDP_BF16 or TDP_F32
struct InVec;
template <>
struct InVec<TDP_BF16> {
  static constexpr int E = 8;
  __device__ static inline void unpack(const uint4& v, float* x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct InVec<TDP_F32> {
  static constexpr int E = 4;
  __device__ static inline void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
};

// Store E accumulated floats as the output dtype at element offset `e`.
template <int OUT, int E>
__device__ inline void store_out(void* out, int64_t e, const float* acc);
template <>
__device__ inline void store_out<TDP_BF16, 8>(void* out, int64_t e, const float* a) {
  uint4 v;
  v.x = bf16_rne(a[0]) | (bf16_rne(a[1]) << 16);
  v.y = bf16_rne(a[2]) | (bf16_rne(a[3]) << 16);
  v.z = bf16_rne(a[4]) | (bf16_rne(a[5]) << 16);
  v.w = bf16_rne(a[6]) | (bf16_rne(a[7]) << 16);
  *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + e) = v;
}
template <>
__device__ inline void store_out<TDP_BF16, 4>(void* out, int64_t e, const float* a) {
  uint2 v;
  v.x = bf16_rne(a[0]) | (bf16_rne(a[1]) << 16);
  v.y = bf16_rne(a[2]) | (bf16_rne(a[3]) << 16);
  *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + e) = v;
}
template <>
__device__ inline void store_out<TDP_F32, 8>(void* out, int64_t e, const float* a) {
  float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + e);
  o[0] = make_float4(a[0], a[1], a[2], a[3]);
  o[1] = make_float4(a[4], a[5], a[6], a[7]);
}
template <>
__device__ inline void store_out<TDP_F32, 4>(void* out, int64_t e, const float* a) {
  *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + e) = make_float4(a[0], a[1], a[2], a[3]);
}

// ---------------------------------------------------------------------------
// Kernel 1: per-chunk extents of every tile's generated positions.
// grid (chunks, B, T).  Writes part[(t, b, chunk)] = 3 x {min start, max end}.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void extents_kernel(const PlanDev p, const float2* __restrict__ pos,
                                                         float* __restrict__ part) {
  const int ch = blockIdx.x, b = blockIdx.y, t = blockIdx.z;
  int i, j, k;
  tile_grid(p, t, i, j, k);
  const int f0 = p.ax[0].start[i], h0 = p.ax[1].start[j], w0 = p.ax[2].start[k];
  const int sh = p.ax[1].size[j], sw = p.ax[2].size[k];
  const int lines = p.ax[0].size[i] * sh;
  const int per = (lines + p.chunks - 1) / p.chunks;
  const int l0 = min(lines, ch * per), l1 = min(lines, l0 + per);
  const int count = (l1 - l0) * sw;

  float lo[3] = {INFINITY, INFINITY, INFINITY};
  float hi[3] = {-INFINITY, -INFINITY, -INFINITY};
  const float2* pb = pos + (int64_t)b * 3 * p.rows;
  for (int e = threadIdx.x; e < count; e += kBlock) {
    const int line = l0 + e / sw;
    const int w = w0 + e % sw;
    const int f = f0 + line / sh, h = h0 + line % sh;
    const int64_t n = ((int64_t)f * p.H + h) * p.W + w;
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const float2 v = pb[(int64_t)d * p.rows + n];
      lo[d] = fminf(lo[d], v.x);
      hi[d] = fmaxf(hi[d], v.y);
    }
  }
  __shared__ float red[kWaves][6];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    const float a = wave_min(lo[d]);
    const float c = wave_max(hi[d]);
    if (lane == 0) {
      red[wave][2 * d] = a;
      red[wave][2 * d + 1] = c;
    }
  }
  __syncthreads();
  if (threadIdx.x < 6) {
    const int m = threadIdx.x;
    float v = red[0][m];
    for (int wv = 1; wv < kWaves; ++wv) v = (m & 1) ? fmaxf(v, red[wv][m]) : fminf(v, red[wv][m]);
    part[((int64_t)(t * p.B + b) * p.chunks + ch) * 6 + m] = v;
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: conditioning-token selection, one workgroup per tile.
// Keeps token c when, for some batch element, its [start, end) overlaps
// the tile's extent on all three axes, or its time start is negative;
// compacts the kept tokens in ascending order (wave ballot + prefix).
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void select_kernel(const PlanDev p, const float2* __restrict__ pos,
                                                        const float* __restrict__ part,
                                                        int32_t* __restrict__ tile_index,
                                                        int32_t* __restrict__ tile_count,
                                                        int32_t* __restrict__ cond_row) {
  extern __shared__ float ext[];  // [B][3][2]: extent start, end
  __shared__ int wave_tot[kWaves];
  const int t = blockIdx.x;
  int i, j, k;
  tile_grid(p, t, i, j, k);
  const TileSlot s = tile_slot(p, i, j, k);
  for (int e = threadIdx.x; e < p.B * 3; e += kBlock) {
    const float2 x = tile_extent(p, part, t, e / 3, e % 3);
    ext[2 * e] = x.x;
    ext[2 * e + 1] = x.y;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int running = 0;
  for (int c0 = 0; c0 < p.Nc; c0 += kBlock) {
    const int c = c0 + threadIdx.x;
    bool keep = false;
    if (c < p.Nc) {
      for (int b = 0; b < p.B && !keep; ++b) {
        const float2* pc = pos + (int64_t)b * 3 * p.rows + p.N + c;
        const float2 x0 = pc[0], x1 = pc[p.rows], x2 = pc[2 * (int64_t)p.rows];
        const float* e = ext + b * 6;
        const bool inside = x0.x < e[1] && x0.y > e[0] && x1.x < e[3] && x1.y > e[2] && x2.x < e[5] && x2.y > e[4];
        keep = inside || x0.x < 0.0f;
      }
    }
    const uint64_t m = __ballot(keep);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __popcll(m);
    __syncthreads();
    int base = running;
    for (int wv = 0; wv < wave; ++wv) base += wave_tot[wv];
    int total = 0;
    for (int wv = 0; wv < kWaves; ++wv) total += wave_tot[wv];
    if (c < p.Nc) {
      const int slot_row = s.gen + base + before;
      cond_row[(int64_t)t * p.Nc + c] = keep ? slot_row : -1;
      if (keep) tile_index[s.index_base + slot_row] = p.N + c;
    }
    running += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) tile_count[t] = s.gen + running;
}

// ---------------------------------------------------------------------------
// Kernel 3: gather.  Three kinds of workgroups in one launch:
//   [0, n_line)                 one (b, f, h) line of the latent: read every
//                               latent row once and write it to each tile
//                               that covers it, with shifted positions and
//                               the source index;
//   [n_line, n_line + n_cond)   kept conditioning rows of one tile;
//   [.., + n_k)                 k = number of tiles keeping each token.
// ---------------------------------------------------------------------------

struct LineTables {
  int ncombo;
  int64_t row[kMaxCombos][kMaxTiles];    // tile_lat row of cell w = row + w
  int64_t pos2[kMaxCombos][kMaxTiles];   // tile_pos float2 of axis 0, cell w
  int64_t idx[kMaxCombos][kMaxTiles];    // tile_index entry of cell w
  int32_t cap[kMaxCombos][kMaxTiles];
  float off[kMaxCombos][kMaxTiles][3];
};

__global__ __launch_bounds__(kBlock) void gather_kernel(const PlanDev p, const uint4* __restrict__ latent,
                                                        const float2* __restrict__ pos,
                                                        const float* __restrict__ part,
                                                        uint4* __restrict__ tile_lat,
                                                        float2* __restrict__ tile_pos,
                                                        int32_t* __restrict__ tile_index,
                                                        int32_t* __restrict__ tile_count,
                                                        const int32_t* __restrict__ cond_row,
                                                        int32_t* __restrict__ cond_k, int n_line, int n_cond) {
  extern __shared__ int wcov[];  // [W] packed covering width tiles
  __shared__ LineTables tb;
  const int bid = blockIdx.x;
  const int V = p.vin;
  const int rpp = kBlock / V;  // rows per pass
  const int r = threadIdx.x / V, vv = threadIdx.x - (threadIdx.x / V) * V;
  const bool lane_on = r < rpp;

  if (bid < n_line) {
    if (bid == 0 && p.Nc == 0) {
      for (int t = threadIdx.x; t < p.T; t += kBlock) {
        int i, j, k;
        tile_grid(p, t, i, j, k);
        tile_count[t] = p.ax[0].size[i] * p.ax[1].size[j] * p.ax[2].size[k];
      }
    }
    const int b = bid / (p.F * p.H);
    const int fh = bid - b * (p.F * p.H);
    const int f = fh / p.H, h = fh - (fh / p.H) * p.H;
    int fi[2], fl[2], hi[2], hl[2];
    const int nf = axis_covers(p.ax[0], f, fi, fl);
    const int nh = axis_covers(p.ax[1], h, hi, hl);
    const int nw = p.ax[2].n;
    for (int w = threadIdx.x; w < p.W; w += kBlock) {
      int ti[2], tl[2];
      const int c = axis_covers(p.ax[2], w, ti, tl);
      wcov[w] = pack_covers(c, ti);
    }
    for (int e = threadIdx.x; e < nf * nh * nw; e += kBlock) {
      const int combo = e / nw, iw = e - (e / nw) * nw;
      const int cf = combo / nh, chh = combo - (combo / nh) * nh;
      const int i = fi[cf], j = hi[chh];
      const TileSlot s = tile_slot(p, i, j, iw);
      const int64_t local = (int64_t)(fl[cf] * p.ax[1].size[j] + hl[chh]) * p.ax[2].size[iw] - p.ax[2].start[iw];
      tb.row[combo][iw] = s.row_base + (int64_t)b * s.cap + local;
      tb.pos2[combo][iw] = 3 * s.row_base + (int64_t)b * 3 * s.cap + local;
      tb.idx[combo][iw] = s.index_base + local;
      tb.cap[combo][iw] = s.cap;
      const int t = (i * p.ax[1].n + j) * nw + iw;
#pragma unroll
      for (int d = 0; d < 3; ++d) tb.off[combo][iw][d] = p.normalize ? tile_extent(p, part, t, b, d).x : 0.0f;
    }
    if (threadIdx.x == 0) tb.ncombo = nf * nh;
    __syncthreads();
    const int ncombo = tb.ncombo;
    const int64_t src0 = (int64_t)b * p.rows + ((int64_t)f * p.H + h) * p.W;

    // latent rows
    for (int wb = 0; wb < p.W; wb += rpp * kGatherUnroll) {
      uint4 v[kGatherUnroll];
      int w[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        w[u] = wb + u * rpp + r;
        if (lane_on && w[u] < p.W) v[u] = latent[(src0 + w[u]) * V + vv];
      }
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        if (!(lane_on && w[u] < p.W)) continue;
        const int cov = wcov[w[u]];
        for (int q = 0; q < 2; ++q) {
          const int iw = (cov >> (8 * q)) & 0xFF;
          if (iw == kNoTile) break;
          for (int cb = 0; cb < ncombo; ++cb) tile_lat[(tb.row[cb][iw] + w[u]) * V + vv] = v[u];
        }
      }
    }
    // positions and source indices
    const int64_t nline = ((int64_t)f * p.H + h) * p.W;
    for (int e = threadIdx.x; e < 3 * p.W; e += kBlock) {
      const int d = e / p.W, w = e - (e / p.W) * p.W;
      const float2 pv = pos[((int64_t)b * 3 + d) * p.rows + nline + w];
      const int cov = wcov[w];
      for (int q = 0; q < 2; ++q) {
        const int iw = (cov >> (8 * q)) & 0xFF;
        if (iw == kNoTile) break;
        for (int cb = 0; cb < ncombo; ++cb) {
          const float o = tb.off[cb][iw][d];
          tile_pos[tb.pos2[cb][iw] + (int64_t)d * tb.cap[cb][iw] + w] = make_float2(pv.x - o, pv.y - o);
          if (b == 0 && d == 0) tile_index[tb.idx[cb][iw] + w] = (int32_t)(nline + w);
        }
      }
    }
    return;
  }

  if (bid < n_line + n_cond) {
    // kept conditioning rows of one tile
    const int per_tile = (p.Nc + kCondRowsPerBlock - 1) / kCondRowsPerBlock;
    const int cid = bid - n_line;
    const int t = cid / per_tile;
    const int j0 = (cid - t * per_tile) * kCondRowsPerBlock;
    int i, j, k;
    tile_grid(p, t, i, j, k);
    const TileSlot s = tile_slot(p, i, j, k);
    const int kept = tile_count[t] - s.gen;
    if (j0 >= kept) return;
    const int nrows = min(kCondRowsPerBlock, kept - j0);
    float* off = reinterpret_cast<float*>(wcov);  // [B][3]
    for (int e = threadIdx.x; e < p.B * 3; e += kBlock)
      off[e] = p.normalize ? tile_extent(p, part, t, e / 3, e % 3).x : 0.0f;
    __syncthreads();
    const int32_t* srcidx = tile_index + s.index_base + s.gen + j0;
    // latent: rows (b, jj) flattened
    const int total = p.B * nrows;
    for (int e = r; e < total; e += rpp) {
      if (!lane_on) break;
      const int b = e / nrows, jj = e - (e / nrows) * nrows;
      const int64_t src = (int64_t)b * p.rows + srcidx[jj];
      const int64_t dst = s.row_base + (int64_t)b * s.cap + s.gen + j0 + jj;
      tile_lat[dst * V + vv] = latent[src * V + vv];
    }
    for (int e = threadIdx.x; e < total * 3; e += kBlock) {
      const int jj = e % nrows, bd = e / nrows;  // bd = b*3 + d
      const int b = bd / 3, d = bd - (bd / 3) * 3;
      const float2 pv = pos[(int64_t)bd * p.rows + srcidx[jj]];
      const float o = off[b * 3 + d];
      tile_pos[3 * s.row_base + ((int64_t)b * 3 + d) * s.cap + s.gen + j0 + jj] = make_float2(pv.x - o, pv.y - o);
    }
    return;
  }

  // k per conditioning token
  const int c = (bid - n_line - n_cond) * kBlock + threadIdx.x;
  if (c < p.Nc) {
    int kc = 0;
    for (int t = 0; t < p.T; ++t) kc += cond_row[(int64_t)t * p.Nc + c] >= 0;
    cond_k[c] = kc;
  }
}

// ---------------------------------------------------------------------------
// Kernel 4: blend.  Owner computes: each output row sums its covering tiles
// in ascending tile order, fp32 accumulation, one store.
//   [0, n_line)   one (b, f, h) line of generated tokens;
//   [n_line, ..)  kCondRowsPerBlock conditioning rows of one batch element.
// ---------------------------------------------------------------------------

struct BlendTables {
  int ncombo;
  float wfh[kMaxCombos];                 // frames x height weight of the combo
  int64_t row[kMaxCombos][kMaxTiles];    // tile_out row of cell w = row + w
};

template <int IN, int OUT, int NCM>
__global__ __launch_bounds__(kBlock) void blend_kernel(const PlanDev p, const uint4* __restrict__ tile_out,
                                                       const int32_t* __restrict__ cond_row,
                                                       const int32_t* __restrict__ cond_k, void* __restrict__ out,
                                                       int n_line) {
  constexpr int E = InVec<IN>::E;
  // Rows in flight per lane: keeps (rows x covering tiles) loads near 16.
  constexpr int U = NCM >= 4 ? 2 : 4;
  extern __shared__ int smem[];  // wcov[W] then wgt[W] (float2)
  __shared__ BlendTables tb;
  const int bid = blockIdx.x;
  const int V = p.vin;
  const int rpp = kBlock / V;
  const int r = threadIdx.x / V, vv = threadIdx.x - (threadIdx.x / V) * V;
  const bool lane_on = r < rpp;

  if (bid < n_line) {
    int* wcov = smem;
    float2* wgt = reinterpret_cast<float2*>(smem + ((p.W + 1) & ~1));
    const int b = bid / (p.F * p.H);
    const int fh = bid - b * (p.F * p.H);
    const int f = fh / p.H, h = fh - (fh / p.H) * p.H;
    int fi[2], fl[2], hi[2], hl[2];
    const int nf = axis_covers(p.ax[0], f, fi, fl);
    const int nh = axis_covers(p.ax[1], h, hi, hl);
    const int nw = p.ax[2].n;
    for (int w = threadIdx.x; w < p.W; w += kBlock) {
      int ti[2], tl[2];
      const int c = axis_covers(p.ax[2], w, ti, tl);
      wcov[w] = pack_covers(c, ti);
      wgt[w] = make_float2(c > 0 ? axis_weight(p.ax[2], ti[0], tl[0]) : 0.0f,
                           c > 1 ? axis_weight(p.ax[2], ti[1], tl[1]) : 0.0f);
    }
    for (int e = threadIdx.x; e < nf * nh * nw; e += kBlock) {
      const int combo = e / nw, iw = e - (e / nw) * nw;
      const int cf = combo / nh, chh = combo - (combo / nh) * nh;
      const int i = fi[cf], j = hi[chh];
      const TileSlot s = tile_slot(p, i, j, iw);
      const int64_t local = (int64_t)(fl[cf] * p.ax[1].size[j] + hl[chh]) * p.ax[2].size[iw] - p.ax[2].start[iw];
      tb.row[combo][iw] = s.row_base + (int64_t)b * s.cap + local;
      if (iw == 0) tb.wfh[combo] = axis_weight(p.ax[0], i, fl[cf]) * axis_weight(p.ax[1], j, hl[chh]);
    }
    if (threadIdx.x == 0) tb.ncombo = nf * nh;
    __syncthreads();
    const int ncombo = tb.ncombo;
    const int64_t dst0 = (int64_t)b * p.rows + ((int64_t)f * p.H + h) * p.W;
    for (int wb = 0; wb < p.W; wb += rpp * U) {
      // All loads of U rows first, then the arithmetic in ascending tile
      // order: combos ascend in (i_f, i_h), width covers in i_w.
      uint4 y[U][2 * NCM];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int w = wb + u * rpp + r;
        if (!(lane_on && w < p.W)) continue;
        const int cov = wcov[w];
#pragma unroll
        for (int cb = 0; cb < NCM; ++cb) {
          if (cb >= ncombo) break;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int iw = (cov >> (8 * q)) & 0xFF;
            if (iw != kNoTile) y[u][2 * cb + q] = tile_out[(tb.row[cb][iw] + w) * V + vv];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int w = wb + u * rpp + r;
        if (!(lane_on && w < p.W)) continue;
        const int cov = wcov[w];
        const float2 ww = wgt[w];
        float acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int cb = 0; cb < NCM; ++cb) {
          if (cb >= ncombo) break;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int iw = (cov >> (8 * q)) & 0xFF;
            if (iw == kNoTile) continue;
            const float wt = tb.wfh[cb] * (q == 0 ? ww.x : ww.y);
            float x[E];
            InVec<IN>::unpack(y[u][2 * cb + q], x);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(wt, x[e], acc[e]);
          }
        }
        store_out<OUT, E>(out, ((dst0 + w) * V + vv) * (int64_t)E, acc);
      }
    }
    return;
  }

  // conditioning rows: (1/k) * sum over the tiles that keep the token
  const int per_b = (p.Nc + kCondRowsPerBlock - 1) / kCondRowsPerBlock;
  const int cid = bid - n_line;
  const int b = cid / per_b;
  const int c0 = (cid - b * per_b) * kCondRowsPerBlock;
  const int nrows = min(kCondRowsPerBlock, p.Nc - c0);
  for (int jj = r; jj < nrows; jj += rpp) {
    if (!lane_on) break;
    const int c = c0 + jj;
    const int kc = cond_k[c];
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    if (kc > 0) {
      const float inv = 1.0f / (float)kc;
      for (int t = 0; t < p.T; ++t) {
        const int row = cond_row[(int64_t)t * p.Nc + c];
        if (row < 0) continue;
        int i, j, k;
        tile_grid(p, t, i, j, k);
        const TileSlot s = tile_slot(p, i, j, k);
        if (row >= s.cap) continue;  // not a row tdp_extract could have written
        const uint4 yv = tile_out[(s.row_base + (int64_t)b * s.cap + row) * V + vv];
        float x[E];
        InVec<IN>::unpack(yv, x);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(inv, x[e], acc[e]);
      }
    }
    store_out<OUT, E>(out, (((int64_t)b * p.rows + p.N + c) * V + vv) * (int64_t)E, acc);
  }
}

template <int IN, int OUT>
hipError_t launch_blend(const PlanDev& p, const void* tile_out, const int32_t* cond_row, const int32_t* cond_k,
                        void* out, hipStream_t s) {
  const int n_line = p.B * p.F * p.H;
  const int n_cond = p.Nc > 0 ? p.B * ((p.Nc + kCondRowsPerBlock - 1) / kCondRowsPerBlock) : 0;
  const size_t lds = (size_t)((p.W + 1) & ~1) * sizeof(int) + (size_t)p.W * sizeof(float2);
  const int ncm = (p.ax[0].n > 1 ? 2 : 1) * (p.ax[1].n > 1 ? 2 : 1);
  const dim3 grid(n_line + n_cond), block(kBlock);
  const uint4* y = reinterpret_cast<const uint4*>(tile_out);
  if (ncm == 1)
    hipLaunchKernelGGL((blend_kernel<IN, OUT, 1>), grid, block, lds, s, p, y, cond_row, cond_k, out, n_line);
  else if (ncm == 2)
    hipLaunchKernelGGL((blend_kernel<IN, OUT, 2>), grid, block, lds, s, p, y, cond_row, cond_k, out, n_line);
  else
    hipLaunchKernelGGL((blend_kernel<IN, OUT, 4>), grid, block, lds, s, p, y, cond_row, cond_k, out, n_line);
  return hipGetLastError();
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

}  // namespace
}  // namespace tdp

using namespace tdp;

extern "C" {

int tdp_extract(const tdp_plan* plan, const void* latent, const float* pos, void* tile_lat, float* tile_pos,
                int32_t* tile_index, int32_t* tile_count, int32_t* cond_row, int32_t* cond_k, void* workspace,
                void* stream) {
  if (!plan) return fail(TDP_EINVAL, "tdp_extract: null plan");
  if (!plan->guarded) return fail(TDP_EGUARD, "tdp_extract: plan was built with TDP_UNGUARDED");
  const PlanDev& p = plan->dev;
  if (!latent || !pos || !tile_lat || !tile_pos || !tile_index || !tile_count)
    return fail(TDP_EINVAL, "tdp_extract: null device pointer");
  if (p.Nc > 0 && (!cond_row || !cond_k))
    return fail(TDP_EINVAL, "tdp_extract: cond_row and cond_k are required when num_cond > 0");
  const bool need_ext = p.normalize || p.Nc > 0;
  if (need_ext && !workspace) return fail(TDP_EINVAL, "tdp_extract: null workspace");
  if (!aligned(latent, 16) || !aligned(tile_lat, 16))
    return fail(TDP_EINVAL, "tdp_extract: latent and tile_lat must be 16-byte aligned");
  if (!aligned(pos, 8) || !aligned(tile_pos, 8) || !aligned(workspace, 4) || !aligned(tile_index, 4) ||
      !aligned(tile_count, 4) || !aligned(cond_row, 4) || !aligned(cond_k, 4))
    return fail(TDP_EINVAL, "tdp_extract: pos/tile_pos need 8-byte and int/float buffers 4-byte alignment");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float2* pos2 = reinterpret_cast<const float2*>(pos);
  float* part = reinterpret_cast<float*>(workspace);
  if (need_ext) {
    hipLaunchKernelGGL(extents_kernel, dim3(p.chunks, p.B, p.T), dim3(kBlock), 0, s, p, pos2, part);
  }
  if (p.Nc > 0) {
    hipLaunchKernelGGL(select_kernel, dim3(p.T), dim3(kBlock), (size_t)p.B * 6 * sizeof(float), s, p, pos2, part,
                       tile_index, tile_count, cond_row);
  }
  const int n_line = p.B * p.F * p.H;
  const int n_cond = p.Nc > 0 ? p.T * ((p.Nc + kCondRowsPerBlock - 1) / kCondRowsPerBlock) : 0;
  const int n_k = p.Nc > 0 ? (p.Nc + kBlock - 1) / kBlock : 0;
  size_t lds = (size_t)p.W * sizeof(int);
  const size_t lds_cond = (size_t)p.B * 3 * sizeof(float);
  if (lds_cond > lds) lds = lds_cond;
  hipLaunchKernelGGL(gather_kernel, dim3(n_line + n_cond + n_k), dim3(kBlock), lds, s, p,
                     reinterpret_cast<const uint4*>(latent), pos2, part, reinterpret_cast<uint4*>(tile_lat),
                     reinterpret_cast<float2*>(tile_pos), tile_index, tile_count, cond_row, cond_k, n_line, n_cond);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TDP_EHIP, "tdp_extract: kernel launch failed: %s", hipGetErrorString(e));
  return TDP_OK;
}

int tdp_blend(const tdp_plan* plan, const void* tile_out, const int32_t* cond_row, const int32_t* cond_k, void* out,
              void* stream) {
  if (!plan) return fail(TDP_EINVAL, "tdp_blend: null plan");
  if (!plan->guarded) return fail(TDP_EGUARD, "tdp_blend: plan was built with TDP_UNGUARDED");
  const PlanDev& p = plan->dev;
  if (!tile_out || !out) return fail(TDP_EINVAL, "tdp_blend: null device pointer");
  if (p.Nc > 0 && (!cond_row || !cond_k))
    return fail(TDP_EINVAL, "tdp_blend: cond_row and cond_k are required when num_cond > 0");
  if (!aligned(tile_out, 16) || !aligned(out, 16))
    return fail(TDP_EINVAL, "tdp_blend: tile_out and out must be 16-byte aligned");
  if (!aligned(cond_row, 4) || !aligned(cond_k, 4)) return fail(TDP_EINVAL, "tdp_blend: misaligned int buffers");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (p.in_dtype == TDP_BF16 && p.out_dtype == TDP_BF16)
    e = launch_blend<TDP_BF16, TDP_BF16>(p, tile_out, cond_row, cond_k, out, s);
  else if (p.in_dtype == TDP_BF16 && p.out_dtype == TDP_F32)
    e = launch_blend<TDP_BF16, TDP_F32>(p, tile_out, cond_row, cond_k, out, s);
  else if (p.in_dtype == TDP_F32 && p.out_dtype == TDP_F32)
    e = launch_blend<TDP_F32, TDP_F32>(p, tile_out, cond_row, cond_k, out, s);
  else
    e = launch_blend<TDP_F32, TDP_BF16>(p, tile_out, cond_row, cond_k, out, s);
  if (e != hipSuccess) return fail(TDP_EHIP, "tdp_blend: kernel launch failed: %s", hipGetErrorString(e));
  return TDP_OK;
}

}  // extern "C"
