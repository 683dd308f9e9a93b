// gfx950 kernels for the tiled hot path: extract and blend.
//
// Sources: LTX-2 docs, "Tiled Data Parallelism (TDP)", sections "What it is",
// "Position normalization" and "Shared negative (reference) positions";
// mold issue #673, "A bug found while porting" (the blend has no
// normalization pass).
//
// Both operations are bound by HBM bandwidth: nothing is a contraction, so
// no MFMA is used.  Latent rows move as 16-byte vectors (global_load /
// global_store_dwordx4).  Generated rows go two vectors per lane, so
// ceil(V / 2) lanes share a row and each wave instruction covers 16 *
// ceil(V / 2) contiguous bytes of every row it touches (a full 128-byte
// line at C = 128 bf16).  The unit of work is one wave's rows of one
// (batch, frame, row) line; tile rows come in closed form from the lane's
// width covers and the line's frame x height combos, with no tables.
// Hot loops are straight-line: every load is unconditional (out-of-range
// lanes re-read a valid row and discard it), so the compiler keeps all of a
// thread's loads in flight instead of waiting before each one.
//
// extract is one launch with three kinds of workgroups, in grid order:
//   selection  (tile, chunk of conditioning tokens): the tile's extents on
//              every (batch, axis), keep test, ordered compaction, copy of
//              the kept rows;
//   positions  (tile, batch, axis, part): the plane's minimum start,
//              reduced by the workgroup itself, then the shifted positions
//              and source indices of one part of the tile;
//   latent     four wave units of (batch, frame, row) line rows each: every
//              latent row is read once and written to each tile that
//              covers it.
// The first two kinds are few and long; dispatched first, they run under
// the latent copy, and no workgroup ever waits on another.  blend is one
// launch too: conditioning workgroups first, then workgroups of four wave
// units that gather each output row from its covering tile rows (owner
// computes: no atomics, fixed order).
// A rank plan (one rank's round-robin share) runs the same kernels,
// instantiated with R = true: they touch only the tiles the rank holds and
// blend writes the rank's full-size partial sum.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "plan_internal.h"

namespace tdp {
namespace {

constexpr int kBlock = kThreads;
constexpr int kWaves = kBlock / 64;
constexpr int kPosUnroll = 8;      // position rows in flight per thread (copy pass)
constexpr int kMinUnroll = 12;     // starts in flight per thread (minimum-start pass)
constexpr int kOwnRows = kPosOwnRows;  // own position rows a thread holds through the minimum pass
constexpr int kSelLoads = 24;      // position loads in flight per thread in the extent launch
constexpr int kCopyBatch = 8;      // kept conditioning vectors in flight per thread
constexpr int kGatherTiles = 4;    // most held tiles per conditioning workgroup of the latent gather
constexpr int kLookbackPolls = 256;  // reads of an unpublished flag before a wave counts that chunk itself
constexpr int kDirectChunks = 16;    // earlier chunks a selection workgroup counts from their tokens
constexpr int kCondRowsPerBlock = 64;  // conditioning tokens per workgroup (streaming, large plans)
constexpr int kCondTokens = 16;        // conditioning tokens per blend workgroup
constexpr int kCondTiles = 256;        // plans up to this many tiles cache cond_row and slots in LDS
constexpr int kCondBatch = 8;          // tile rows in flight per lane
constexpr int kXcds = 8;           // accelerator dies; workgroups are dealt to them round-robin

// ---------------------------------------------------------------------------
// Axis helpers (closed-form split from plan_internal.h; no tables)
// ---------------------------------------------------------------------------

// R: the plan holds one rank's round-robin share (uniform slots, local
// index t / world); otherwise every tile, packed.  A compile-time switch, so
// the whole-plan kernels carry none of the share's checks.
template <bool R>
__device__ inline TileSlot slot_of(const PlanDev& p, int i, int j, int k) {
  if constexpr (R)
    return tile_slot_rank(p, i, j, k);
  else
    return tile_slot_whole(p, i, j, k);
}

template <bool R>
__device__ inline bool held(const PlanDev& p, int t) {
  if constexpr (R)
    return tile_is_local(p, t);
  else
    return true;
}

struct TileBox {
  int f0, h0, w0, sf, sh, sw;
  TileSlot s;
};

template <bool R>
__device__ inline TileBox tile_box(const PlanDev& p, int t) {
  int i, j, k;
  tile_grid(p, t, i, j, k);
  TileBox tb;
  tb.f0 = split_start(p.ax[0], i);
  tb.h0 = split_start(p.ax[1], j);
  tb.w0 = split_start(p.ax[2], k);
  tb.sf = split_size(p.ax[0], i);
  tb.sh = split_size(p.ax[1], j);
  tb.sw = split_size(p.ax[2], k);
  tb.s = slot_of<R>(p, i, j, k);
  return tb;
}

// Frame x height covers of one (f, h) line: up to four (tile pair, local
// cell) combos in ascending (i_f, i_h) order.
struct LineCombos {
  int n;                   // number of combos: 1, 2 or 4
  int nh;                  // height covers
  Covers cf, ch;
  __device__ inline void init(const PlanDev& p, int f, int h) {
    cf = split_covers(p.ax[0], f);
    ch = split_covers(p.ax[1], h);
    nh = ch.n;
    n = cf.n * ch.n;
  }
  // combo -> (i, lf, sf, j, lh, sh)
  __device__ inline void get(int combo, int f, int h, int& i, int& lf, int& sf, int& j, int& lh, int& sh) const {
    const int a = nh == 2 ? combo >> 1 : combo, c = nh == 2 ? combo & 1 : 0;
    i = a ? cf.t1 : cf.t0;
    lf = f - (a ? cf.a1 : cf.a0);
    sf = a ? cf.s1 : cf.s0;
    j = c ? ch.t1 : ch.t0;
    lh = h - (c ? ch.a1 : ch.a0);
    sh = c ? ch.s1 : ch.s0;
  }
};

// Rows of one (f, h) line in the tiles of one frame x height combo (i, j).
// In tile t = tbase + k (width tile k, start a_k, size sw_k), batch element
// b, the row of width cell w is
//   whole plan: base + sfsh * (B * PW_k + b * sw_k) + Nc * (B * k + b)
//                    + L * sw_k + (w - a_k),   PW_k = a_k + k * o (cells of
//               width tiles before k), base = B * (rows of every tile before
//               (i, j, 0), i.e. gen_before(i, j, 0) + tbase * Nc);
//   rank plan:  (t / world) * slot_cap * B + b * (sfsh * sw_k + Nc)
//                    + L * sw_k + (w - a_k),
// the slot layout of tile_slot_whole / tile_slot_rank written out by width
// tile.  The plan keeps every tile row below 2^31, so rows are int32.
struct ComboRows {
  int base;   // whole plan: rows of the tiles before (i, j, 0), all batch elements
  int tbase;  // (i * nH + j) * nW
  int sfsh;   // sf * sh: width rows per tile row of this combo's tiles
  int L;      // lf * sh + lh: the line's row within a width-row of the tile
};
template <bool R>
__device__ inline ComboRows combo_rows(const PlanDev& p, int i, int lf, int sf, int j, int lh, int sh) {
  ComboRows c;
  c.tbase = (i * p.ax[1].n + j) * p.ax[2].n;
  c.sfsh = sf * sh;
  c.L = lf * sh + lh;
  c.base = R ? 0
             : p.B * ((split_prefix(p.ax[0], i) * split_total(p.ax[1]) + sf * split_prefix(p.ax[1], j)) *
                          split_total(p.ax[2]) +
                      p.Nc * c.tbase);
  return c;
}
// Row of width cell w in width tile k (start a, size s) of combo c.
template <bool R>
__device__ inline int cover_row(const PlanDev& p, const ComboRows& c, int b, int k, int a, int s, int w) {
  if constexpr (R)
    return (int)fastdiv((uint32_t)(c.tbase + k), p.by_world) * p.slot_cap * p.B + b * (c.sfsh * s + p.Nc) +
           c.L * s + (w - a);
  else
    return c.base + c.sfsh * (p.B * (a + k * p.ax[2].o) + b * s) + p.Nc * (p.B * k + b) + c.L * s + (w - a);
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

// Block-wide (min of a, max of b), returned to every thread.  `red` is
// kWaves float2 of shared memory.
__device__ inline float2 block_minmax(float a, float b, float2* red) {
  a = wave_min(a);
  b = wave_max(b);
  __syncthreads();  // earlier readers of red are done
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(a, b);
  __syncthreads();
  float2 r = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    r.x = fminf(r.x, red[w].x);
    r.y = fmaxf(r.y, red[w].y);
  }
  return r;
}

// ---------------------------------------------------------------------------
// extract
// ---------------------------------------------------------------------------

struct ExtractArgs {
  const u32x4* latent;   // (B, rows, V) vectors
  const f32x2* pos;      // (B, 3, rows) [start, end)
  u32x4* tile_lat;
  f32x2* tile_pos;
  int32_t* tile_index;
  int32_t* tile_count;
  int32_t* cond_row;     // (T, Nc)
  int32_t* cond_k;       // (Nc)
  char* ws;              // workspace: extent partials and look-back flags (Nc > 0), else null
  int n_ext, n_sel, n_pos, pos_parts;
  int copy_latent;       // 0: positions, index, counts and selection only (no latent rows)
  int pos_one_pass;      // position workgroups hold their part in registers (one pass)
  int lookback_polls;    // reads of an unpublished flag before a wave counts that chunk itself
};

// Tables of the conditioning selection in the workspace (layout in WsLayout).
__device__ inline const float2* ws_part(const PlanDev& p, const ExtractArgs& a) {
  return reinterpret_cast<const float2*>(a.ws + ws_layout(p).part);
}
__device__ inline float2* ws_part_w(const PlanDev& p, const ExtractArgs& a) {
  return reinterpret_cast<float2*>(a.ws + ws_layout(p).part);
}
__device__ inline uint32_t* ws_flags(const PlanDev& p, const ExtractArgs& a) {
  return reinterpret_cast<uint32_t*>(a.ws + ws_layout(p).flags);
}

// Source token (within one batch element) of generated row r of a tile:
// r = (lf * sh + lh) * sw + x.
__device__ inline int tile_row_source(const PlanDev& p, const TileBox& tb, int r) {
  const int line = (int)div_by_size(p.ax[2], (uint32_t)r, tb.sw);
  const int x = r - line * tb.sw;
  const int lf = (int)div_by_size(p.ax[1], (uint32_t)line, tb.sh);
  const int lh = line - lf * tb.sh;
  return ((tb.f0 + lf) * p.H + (tb.h0 + lh)) * p.W + tb.w0 + x;
}

struct ExtractShared {
  float2 red[kWaves];
};

// Token n of a position plane (n < 2^29, which the plan enforces): a 32-bit
// byte offset lets the load take a scalar base plus one vector register.
__device__ inline f32x2 ld_plane(const f32x2* plane, int n) {
  return *reinterpret_cast<const f32x2*>(reinterpret_cast<const char*>(plane) + ((uint32_t)n << 3));
}

// Minimum start over a tile's generated tokens of one position plane, the
// offset that normalization subtracts.  Only the start of each interval is
// loaded (4 bytes), so many rows fit in flight per thread, which keeps the
// number of dependent passes over a large tile small.  Rows past the end
// re-read row 0: a repeat does not change a minimum.
__device__ float tile_plane_min_start(const PlanDev& p, const TileBox& tb, const f32x2* __restrict__ src,
                                      float2* red) {
  const int gen = tb.s.gen;
  const float* starts = reinterpret_cast<const float*>(src);
  float lo = INFINITY;
  for (int r0 = 0; r0 < gen; r0 += kBlock * kMinUnroll) {
    float v[kMinUnroll];
#pragma unroll
    for (int u = 0; u < kMinUnroll; ++u) {
      const int r = r0 + u * kBlock + (int)threadIdx.x;
      const int n = tile_row_source(p, tb, r < gen ? r : 0);
      v[u] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(starts) + ((uint32_t)n << 3));
    }
#pragma unroll
    for (int u = 0; u < kMinUnroll; ++u) lo = fminf(lo, v[u]);
  }
  return block_minmax(lo, -INFINITY, red).x;
}

// ---- conditioning selection in the extract launch (Nc > 0) ----
//
// Look-back words (flags table, zeroed by the extent launch): 0 until
// published, then kFlagAgg with the chunk's own kept count, or kFlagPrefix
// with the tile's kept count over chunks 0..k.  Counts stay below 2^29.
// Words are read and written with device-scope atomics, so a wave on
// another accelerator die sees them.
constexpr uint32_t kFlagAgg = 1u << 30;
constexpr uint32_t kFlagPrefix = 1u << 31;
constexpr uint32_t kFlagCount = kFlagAgg - 1u;

__device__ inline void flag_publish(uint32_t* f, uint32_t v) {
  __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t flag_read(uint32_t* f) {
  return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline int wave_sum_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Position (from 0) of the set bit of m with j set bits below it (j < popcount(m)).
__device__ inline int nth_set_bit(uint64_t m, int j) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const uint64_t lo = m & ((1ull << w) - 1ull);
    const int cnt = __popcll(lo);
    const bool up = j >= cnt;
    j = up ? j - cnt : j;
    m = up ? m >> w : lo;
    pos += up ? w : 0;
  }
  return pos;
}

// The tile's extent, its parts combined, into ext[0 .. B*3) (whole
// workgroup; eight parts' loads in flight per thread).
__device__ void combine_extent(const PlanDev& p, const ExtractArgs& a, int t, float2* ext) {
  const int planes = p.B * 3;
  const float2* parts = ws_part(p, a) + (int64_t)t * p.ext_parts * planes;
  for (int e = threadIdx.x; e < planes; e += kBlock) {
    float2 m = make_float2(INFINITY, -INFINITY);
    for (int q0 = 0; q0 < p.ext_parts; q0 += 8) {
      float2 y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) y[u] = parts[(int64_t)min(q0 + u, p.ext_parts - 1) * planes + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        m.x = fminf(m.x, y[u].x);
        m.y = fmaxf(m.y, y[u].y);
      }
    }
    ext[e] = m;
  }
}

// Minimum start of tile t on plane bd = b * 3 + d, its parts combined
// (eight parts' loads in flight).
__device__ inline float tile_min_start(const PlanDev& p, const ExtractArgs& a, int t, int bd) {
  const int planes = p.B * 3;
  const float2* parts = ws_part(p, a) + (int64_t)t * p.ext_parts * planes + bd;
  float m = INFINITY;
  for (int q0 = 0; q0 < p.ext_parts; q0 += 8) {
    float y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) y[u] = parts[(int64_t)min(q0 + u, p.ext_parts - 1) * planes].x;
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fminf(m, y[u]);
  }
  return m;
}

// Positions of the token of lane l of chunk ch for batch elements b0 and
// b0 + 1 (an odd batch repeats the last: the keep test ORs over them).
struct TokenPos {
  f32x2 x[2][3];
};
__device__ inline TokenPos load_token_pos(const PlanDev& p, const f32x2* __restrict__ pos, int ch, int b0) {
  const int c = ch * kCondChunk + (int)(threadIdx.x & 63);
  const int cs = c < p.Nc ? c : 0;  // token 0 exists whenever this runs; masked by the test
  TokenPos tp;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const f32x2* pc = pos + (int64_t)min(b0 + kb, p.B - 1) * 3 * p.rows + p.N + cs;
    tp.x[kb][0] = pc[0];
    tp.x[kb][1] = pc[p.rows];
    tp.x[kb][2] = pc[2 * (int64_t)p.rows];
  }
  return tp;
}

// Keep bits of chunk ch (one wave) for the tile whose extent (B * 3 planes
// of [min start, max end)) is ext; lane l tests token ch * kCondChunk + l,
// its positions for batch elements 0 and 1 already in tp.  A token is kept
// when, for some batch element, its interval overlaps the extent on all
// three axes (half-open) or its time start is negative (TDP docs, "Shared
// negative (reference) positions"), on the positions as given.
__device__ uint64_t chunk_keep_mask(const PlanDev& p, const f32x2* __restrict__ pos, const float2* ext, int ch,
                                    TokenPos tp) {
  const int c = ch * kCondChunk + (int)(threadIdx.x & 63);
  bool keep = false;
  for (int b0 = 0; b0 < p.B; b0 += 2) {
    if (b0 > 0) tp = load_token_pos(p, pos, ch, b0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float2* e = ext + min(b0 + kb, p.B - 1) * 3;
      const f32x2* x = tp.x[kb];
      const bool inside = x[0].x < e[0].y && x[0].y > e[0].x && x[1].x < e[1].y && x[1].y > e[1].x &&
                          x[2].x < e[2].y && x[2].y > e[2].x;
      keep = keep || inside || x[0].x < 0.0f;
    }
  }
  return __ballot(keep && c < p.Nc);
}

// Kept tokens of the tile in chunks 0..ch-1 (ch >= 1; one wave), from those
// chunks' flags, the nearest 64 per read: aggregates add up to the first
// inclusive prefix.  A chunk whose word is still 0 after a.lookback_polls
// reads is counted here from its tokens, so no wave depends on the order in
// which workgroups start.
__device__ int lookback(const PlanDev& p, const ExtractArgs& a, uint32_t* flags, const float2* ext, int ch) {
  const int lane = threadIdx.x & 63;
  int before = 0, j = ch - 1, polls = 0;
  while (true) {
    const int jj = j - lane;
    const uint32_t f = jj >= 0 ? flag_read(flags + jj) : kFlagPrefix;  // before chunk 0: a prefix of 0
    const uint64_t pre = __ballot((f & kFlagPrefix) != 0);
    const uint64_t wait = __ballot(f == 0);
    const int first_pre = pre ? (int)__builtin_ctzll(pre) : 64;
    const int first_wait = wait ? (int)__builtin_ctzll(wait) : 64;
    const int n = min(first_pre + 1, first_wait);  // lanes [0, n) are counted now
    before += wave_sum_int(lane < n ? (int)(f & kFlagCount) : 0);
    if (first_pre < first_wait) return before;
    j -= n;  // chunk j is the first one not counted yet
    if (n > 0) polls = 0;
    if (n == 64) continue;
    if (++polls > a.lookback_polls) {  // chunk j has not published: count it here
      before += __popcll(chunk_keep_mask(p, a.pos, ext, j, load_token_pos(p, a.pos, j, 0)));
      --j;
      polls = 0;
    } else {
      __builtin_amdgcn_s_sleep(4);
    }
  }
}

// Kept row jj (< n) of batch element b and vector vv for flat index e of
// the (b, kept j, vector) copy order.
struct KeptVec {
  int b, jj, vv;
};
__device__ inline KeptVec kept_vec(const PlanDev& p, const FastDiv& by_n, int n, int e) {
  KeptVec k;
  const int row = (int)fastdiv((uint32_t)e, p.by_vin);
  k.vv = e - row * p.vin;
  k.b = (int)fastdiv((uint32_t)row, by_n);
  k.jj = row - k.b * n;
  return k;
}

struct CondShared {
  uint64_t mask;        // keep bits of the chunk
  int direct[kWaves];   // kept tokens of the chunks each wave counted
  int before;           // kept tokens of the tile before the chunk
};

// Selection workgroup (Nc > 0): chunk ch of the conditioning tokens
// against tile t.  Two regimes, by the number of chunks per tile (SMALL:
// each its own instantiation, so the large one carries none of the small
// one's registers):
//   small (at most kDirectChunks + 1 chunks): every earlier chunk of the
//     tile is counted here from its tokens, tested in the same pass as the
//     chunk's own, so no workgroup waits on another; and when the chunk's
//     rows of every batch element fit one round of loads (B * kCondChunk * V
//     <= kBlock * kCopyBatch), every token's latent vectors and positions
//     are loaded with the extent, before the test, and only the kept ones
//     stored: one round trip for the whole workgroup;
//   large: the earlier chunks' kept tokens come from their flags by
//     look-back (wave 0) and only the kept rows are loaded, after the test,
//     so each token's rows and positions are read about once per keeping
//     tile (re-testing or re-reading whole chunks would multiply the reads
//     by the window or by T).
// Then cond_row (every tile: k counts the tiles of all ranks), cond_k, and
// for a held tile the index entries, the rows, the shifted positions and,
// from the last chunk, the tile's count.
template <bool R, bool SMALL>
__device__ void extract_cond_chunk(const PlanDev& p, const ExtractArgs& a, CondShared& sm, float2* ext, int t,
                                   int ch) {
  constexpr int kPer = SMALL ? (kDirectChunks + 1 + kWaves - 1) / kWaves : 1;  // chunks per wave
  constexpr int kPosPer = (kCondChunk * 6 + kBlock - 1) / kBlock;   // position pairs per thread, B <= 2
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* flags = ws_flags(p, a) + (int64_t)t * p.n_chunks;
  constexpr bool publish = !SMALL;  // some workgroup reads flags
  const int j0 = SMALL ? 0 : ch;    // first chunk tested here
  const bool held_t = held<R>(p, t);
  const int V = p.vin;
  const int c0 = p.N + ch * kCondChunk;
  const int ntok = min(kCondChunk, p.Nc - ch * kCondChunk);
  // (b, token j, vector) of the whole chunk, token-minor over vectors
  const int all_vec = p.B * kCondChunk * V;
  const bool lat = a.copy_latent != 0;
  const bool early = lat && SMALL && held_t && all_vec <= kBlock * kCopyBatch && p.B <= 2;  // workgroup-uniform
  u32x4 v[kCopyBatch];
  f32x2 w[kPosPer];
  if (early) {
#pragma unroll
    for (int q = 0; q < kCopyBatch; ++q) {
      const int e = min(q * kBlock + tid, all_vec - 1);
      const int row = (int)fastdiv((uint32_t)e, p.by_vin), vv = e - row * V;
      const int b = row / kCondChunk, j = min(row - b * kCondChunk, ntok - 1);
      v[q] = ld_nt(a.latent + ((int64_t)b * p.rows + c0 + j) * V + vv);
    }
#pragma unroll
    for (int q = 0; q < kPosPer; ++q) {
      const int e = min(q * kBlock + tid, p.B * 3 * kCondChunk - 1);
      const int bd = e / kCondChunk, j = min(e - bd * kCondChunk, ntok - 1);
      w[q] = a.pos[(int64_t)bd * p.rows + c0 + j];
    }
  }
  // chunks j0..ch: wave w takes j0 + w, j0 + w + 4, ...; their positions
  // are in flight while the extent is combined
  TokenPos tp[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (j0 + wave + i * kWaves <= ch) tp[i] = load_token_pos(p, a.pos, j0 + wave + i * kWaves, 0);
  combine_extent(p, a, t, ext);
  __syncthreads();
  int direct = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = j0 + wave + i * kWaves;
    if (j <= ch) {  // wave-uniform
      const uint64_t m = chunk_keep_mask(p, a.pos, ext, j, tp[i]);
      if (j < ch) {
        direct += __popcll(m);
      } else if (lane == 0) {
        sm.mask = m;
        if (publish && j0 > 0) flag_publish(flags + ch, kFlagAgg | (uint32_t)__popcll(m));
      }
    }
  }
  if (lane == 0) sm.direct[wave] = direct;
  __syncthreads();
  const uint64_t mask = sm.mask;
  const int n = __popcll(mask);
  const TileBox tb = tile_box<R>(p, t);
  const bool copy = held_t && n > 0 && !early;  // the copy after the test
  const FastDiv by_n = make_fastdiv((uint32_t)(n > 0 ? n : 1));
  const int total = p.B * n * V;
  if (copy && lat) {
#pragma unroll
    for (int q = 0; q < kCopyBatch; ++q) {
      const KeptVec k = kept_vec(p, by_n, n, min(q * kBlock + tid, total - 1));
      v[q] = ld_nt(a.latent + ((int64_t)k.b * p.rows + c0 + nth_set_bit(mask, k.jj)) * V + k.vv);
    }
  }
  int before = sm.direct[0] + sm.direct[1] + sm.direct[2] + sm.direct[3];
  if (j0 > 0) {  // workgroup-uniform
    if (wave == 0) {
      before += lookback(p, a, flags, ext, j0);
      if (lane == 0) {
        flag_publish(flags + ch, kFlagPrefix | (uint32_t)(before + n));
        sm.before = before;
      }
    }
    __syncthreads();
    before = sm.before;
  } else if (publish && tid == 0) {
    flag_publish(flags + ch, kFlagPrefix | (uint32_t)(before + n));
  }
  const int first = tb.s.gen + before;  // slot row of the chunk's first kept token
  if (tid < kCondChunk) {
    const int c = ch * kCondChunk + tid;
    const bool keep = (mask >> tid) & 1ull;
    const int row = first + __popcll(mask & ((1ull << tid) - 1ull));
    if (c < p.Nc) a.cond_row[(int64_t)t * p.Nc + c] = keep ? row : -1;
    if (keep) atomicAdd(a.cond_k + c, 1);
    if (keep && held_t) a.tile_index[tb.s.index_base + row] = p.N + c;
  }
  if (held_t && ch == p.n_chunks - 1 && tid == 0)
    a.tile_count[R ? (int)fastdiv((uint32_t)t, p.by_world) : t] = first + n;
  if (early) {  // the kept ones of the vectors and positions already loaded
#pragma unroll
    for (int q = 0; q < kCopyBatch; ++q) {
      const int e = q * kBlock + tid;
      const int row = (int)fastdiv((uint32_t)e, p.by_vin), vv = e - row * V;
      const int b = row / kCondChunk, j = row - b * kCondChunk;
      if (e < all_vec && ((mask >> j) & 1ull)) {
        const int r = __popcll(mask & ((1ull << j) - 1ull));
        st_nt(a.tile_lat + (tb.s.row_base + (int64_t)b * tb.s.cap + first + r) * V + vv, v[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < kPosPer; ++q) {
      const int e = q * kBlock + tid;
      const int bd = e / kCondChunk, j = e - bd * kCondChunk;
      if (e < p.B * 3 * kCondChunk && ((mask >> j) & 1ull)) {
        const int r = __popcll(mask & ((1ull << j) - 1ull));
        const float o = p.normalize ? ext[bd].x : 0.0f;
        st_nt(a.tile_pos + 3 * tb.s.row_base + (int64_t)bd * tb.s.cap + first + r, w[q] - o);
      }
    }
    return;
  }
  if (!copy) return;
  for (int e0 = 0; lat && e0 < total; e0 += kBlock * kCopyBatch) {
    if (e0 > 0) {
#pragma unroll
      for (int q = 0; q < kCopyBatch; ++q) {
        const KeptVec k = kept_vec(p, by_n, n, min(e0 + q * kBlock + tid, total - 1));
        v[q] = ld_nt(a.latent + ((int64_t)k.b * p.rows + c0 + nth_set_bit(mask, k.jj)) * V + k.vv);
      }
    }
#pragma unroll
    for (int q = 0; q < kCopyBatch; ++q) {
      const int e = e0 + q * kBlock + tid;
      if (e < total) {
        const KeptVec k = kept_vec(p, by_n, n, e);
        st_nt(a.tile_lat + (tb.s.row_base + (int64_t)k.b * tb.s.cap + first + k.jj) * V + k.vv, v[q]);
      }
    }
  }
  const int ptotal = p.B * 3 * n;  // (plane b * 3 + d, kept j)
  for (int e0 = 0; e0 < ptotal; e0 += kBlock * kCopyBatch) {
    f32x2 y[kCopyBatch];
#pragma unroll
    for (int q = 0; q < kCopyBatch; ++q) {
      const int e = min(e0 + q * kBlock + tid, ptotal - 1);
      const int bd = (int)fastdiv((uint32_t)e, by_n), jj = e - bd * n;
      y[q] = a.pos[(int64_t)bd * p.rows + c0 + nth_set_bit(mask, jj)];
    }
#pragma unroll
    for (int q = 0; q < kCopyBatch; ++q) {
      const int e = e0 + q * kBlock + tid;
      if (e < ptotal) {
        const int bd = (int)fastdiv((uint32_t)e, by_n), jj = e - bd * n;
        const float o = p.normalize ? ext[bd].x : 0.0f;
        st_nt(a.tile_pos + 3 * tb.s.row_base + (int64_t)bd * tb.s.cap + first + jj, y[q] - o);
      }
    }
  }
}

// Positions workgroup: tile t, batch b, axis d, part `part` of the tile's
// generated rows: the shifted [start, end) pairs and the source indices.
// The shift is the tile's minimum start on this plane, which the workgroup
// reduces itself over the whole plane (the parts of a plane repeat that
// pass, so no workgroup waits on another); the copy pass then re-reads its
// own rows from L2.
// `slot` is the tile's local index (t itself for a whole plan).
template <bool R>
__device__ void extract_positions(const PlanDev& p, const ExtractArgs& a, ExtractShared& sm, int t, int slot,
                                  int b, int d, int part) {
  const TileBox tb = tile_box<R>(p, t);
  const int gen = tb.s.gen;
  const int per = (gen + a.pos_parts - 1) / a.pos_parts;
  const int r_begin = min(gen, part * per), r_end = min(gen, r_begin + per);
  if (part == 0 && b == 0 && d == 0 && p.Nc == 0 && threadIdx.x == 0) a.tile_count[slot] = gen;
  const f32x2* src = a.pos + ((int64_t)b * 3 + d) * p.rows;
  f32x2* dst = a.tile_pos + 3 * tb.s.row_base + ((int64_t)b * 3 + d) * tb.s.cap;
  int32_t* idx = a.tile_index + tb.s.index_base;
  const bool write_index = (b == 0 && d == 0);
  const int own = r_end - r_begin;
  if (a.pos_one_pass && own <= kBlock * kOwnRows) {
    // One pass: the part's own [start, end) pairs are loaded into registers
    // (their indices stored at once) together with the starts of the rest
    // of the plane, so the shifted pairs need no second round of loads.
    // Without normalization the shift is 0 and the rest is not read.
    // Slots past the part (a workgroup-uniform test) load nothing; within
    // the last slot, idle lanes re-read a valid row of the tile.
    const int rs = own > 0 ? r_begin : 0;
    f32x2 v[kOwnRows];
#pragma unroll
    for (int u = 0; u < kOwnRows; ++u) {
      v[u] = f32x2{INFINITY, INFINITY};
      if (u * kBlock < own) {
        const int r = r_begin + u * kBlock + (int)threadIdx.x;
        const int n = tile_row_source(p, tb, r < r_end ? r : rs);
        v[u] = ld_plane(src, n);
        if (write_index && r < r_end) st_nt(idx + r, (int32_t)n);
      }
    }
    // rows outside [r_begin, r_end): starts only; past the end, row 0 again
    // (a repeat does not change a minimum)
    const int rest = p.normalize ? gen - own : 0;
    const float* starts = reinterpret_cast<const float*>(src);
    float lo = INFINITY;
    for (int r0 = 0; r0 < rest; r0 += kBlock * kMinUnroll) {
      float m[kMinUnroll];
#pragma unroll
      for (int u = 0; u < kMinUnroll; ++u) {
        m[u] = INFINITY;
        if (r0 + u * kBlock < rest) {
          const int rr = r0 + u * kBlock + (int)threadIdx.x;
          const int r = rr < rest ? (rr < r_begin ? rr : rr + own) : 0;
          const int n = tile_row_source(p, tb, r);
          m[u] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(starts) + ((uint32_t)n << 3));
        }
      }
#pragma unroll
      for (int u = 0; u < kMinUnroll; ++u) lo = fminf(lo, m[u]);
    }
#pragma unroll
    for (int u = 0; u < kOwnRows; ++u) lo = fminf(lo, v[u].x);  // idle lanes hold a row of the tile or +inf
    const float off = p.normalize ? block_minmax(lo, -INFINITY, sm.red).x : 0.0f;  // uniform branch
#pragma unroll
    for (int u = 0; u < kOwnRows; ++u) {
      const int r = r_begin + u * kBlock + (int)threadIdx.x;
      if (r < r_end) st_nt(dst + r, v[u] - off);
    }
    return;
  }
  const float off = p.normalize ? tile_plane_min_start(p, tb, src, sm.red) : 0.0f;
  for (int r0 = r_begin; r0 < r_end; r0 += kBlock * kPosUnroll) {
    int n[kPosUnroll];
    f32x2 v[kPosUnroll];
#pragma unroll
    for (int u = 0; u < kPosUnroll; ++u) {
      const int r = r0 + u * kBlock + (int)threadIdx.x;
      n[u] = tile_row_source(p, tb, r < r_end ? r : r_begin);
      v[u] = ld_plane(src, n[u]);
    }
#pragma unroll
    for (int u = 0; u < kPosUnroll; ++u) {
      const int r = r0 + u * kBlock + (int)threadIdx.x;
      if (r < r_end) {
        st_nt(dst + r, v[u] - off);
        if (write_index) st_nt(idx + r, (int32_t)n[u]);
      }
    }
  }
}

// Positions workgroup with the shift `off` already known (Nc > 0: from the
// tile's extent parts): it only copies its part of the plane (shifted pairs
// and source indices).
template <bool R>
__device__ void extract_positions_copy(const PlanDev& p, const ExtractArgs& a, int t, int b, int d, int part,
                                       float off) {
  const TileBox tb = tile_box<R>(p, t);
  const int gen = tb.s.gen;
  const int per = (gen + a.pos_parts - 1) / a.pos_parts;
  const int r_begin = min(gen, part * per), r_end = min(gen, r_begin + per);
  const f32x2* src = a.pos + ((int64_t)b * 3 + d) * p.rows;
  f32x2* dst = a.tile_pos + 3 * tb.s.row_base + ((int64_t)b * 3 + d) * tb.s.cap;
  int32_t* idx = a.tile_index + tb.s.index_base;
  const bool write_index = (b == 0 && d == 0);
  for (int r0 = r_begin; r0 < r_end; r0 += kBlock * kPosUnroll) {
    int n[kPosUnroll];
    f32x2 v[kPosUnroll];
#pragma unroll
    for (int u = 0; u < kPosUnroll; ++u) {
      const int r = r0 + u * kBlock + (int)threadIdx.x;
      n[u] = tile_row_source(p, tb, r < r_end ? r : r_begin);
      v[u] = ld_plane(src, n[u]);
    }
#pragma unroll
    for (int u = 0; u < kPosUnroll; ++u) {
      const int r = r0 + u * kBlock + (int)threadIdx.x;
      if (r < r_end) {
        st_nt(dst + r, v[u] - off);
        if (write_index) st_nt(idx + r, (int32_t)n[u]);
      }
    }
  }
}

// Latent wave unit: rows [w0, w0 + rwv) of one (b, f, h) line, every row
// read once and written to each covering tile.  Lane (r, q) of the wave
// moves vectors q and lpr + q of row w0 + r, so each load and
// store instruction covers 16 * lpr contiguous bytes of every row it
// touches.  Tile rows come in closed form from the lane's width covers and
// the line's frame x height combos (wave-uniform), with no tables and no
// barrier; the loads are issued before any of that is computed.  A rank
// plan reads only the rows that one of its tiles covers.
template <bool R, int W = kWaves>
__device__ void extract_latent(const PlanDev& p, const ExtractArgs& a, int blk) {
  const int V = p.vin, LPR = p.lpr;
  const int rows = p.lat_rows;
  // this wave's unit: the waves of a workgroup take consecutive units
  const int unit = __builtin_amdgcn_readfirstlane(blk * W + (int)(threadIdx.x >> 6));
  if (unit >= p.lat_units) return;
  int b, f, h, w0;
  if constexpr (R) {  // units tile the held tiles' bounding box only
    const int line = (int)fastdiv((uint32_t)unit, p.by_box_c);
    w0 = (p.box_c0 + unit - line * p.box_nc) * rows;
    b = (int)fastdiv((uint32_t)line, p.by_box_fh);
    const int fh = line - b * (p.box_nf * p.box_nh);
    const int fb = (int)fastdiv((uint32_t)fh, p.by_box_h);
    f = p.box_f0 + fb;
    h = p.box_h0 + fh - fb * p.box_nh;
  } else {
    const int line = (int)fastdiv((uint32_t)unit, p.by_lat_chunks);
    w0 = (unit - line * p.lat_chunks) * rows;
    b = (int)fastdiv((uint32_t)line, p.by_FH);
    const int fh = line - b * (p.F * p.H);
    f = (int)fastdiv((uint32_t)fh, p.by_H);
    h = fh - f * p.H;
  }
  const int lane = threadIdx.x & 63;
  const int r = (int)fastdiv((uint32_t)lane, p.by_lpr), q = lane - r * LPR;
  const int wr = w0 + r;
  bool ok = r < p.rwv && wr < p.W;
  const int w = ok ? wr : w0;  // w0 < W: an unused lane re-reads a row of this line
  const int v1 = LPR + q;
  const bool ok1 = v1 < V;
  const int v1l = ok1 ? v1 : q;
  const u32x4* src = a.latent + ((int64_t)b * p.rows + ((int64_t)f * p.H + h) * p.W + w) * V;
  u32x4 x0, x1;
  if constexpr (!R) {
    x0 = ld_nt(src + q);
    x1 = ld_nt(src + v1l);
  }
  LineCombos lc;
  lc.init(p, f, h);
  const Covers cw = split_covers(p.ax[2], w);
  if constexpr (R) {
    bool any = false;
    for (int cb = 0; cb < lc.n; ++cb) {
      int i, lf, sf, j, lh, sh;
      lc.get(cb, f, h, i, lf, sf, j, lh, sh);
      const int tb = (i * p.ax[1].n + j) * p.ax[2].n;
      any = any || tile_is_local(p, tb + cw.t0) || (cw.n > 1 && tile_is_local(p, tb + cw.t1));
    }
    ok = ok && any;
    x0 = ok ? ld_nt(src + q) : u32x4{0u, 0u, 0u, 0u};
    x1 = ok ? ld_nt(src + v1l) : u32x4{0u, 0u, 0u, 0u};
  }
  for (int cb = 0; cb < lc.n; ++cb) {
    int i, lf, sf, j, lh, sh;
    lc.get(cb, f, h, i, lf, sf, j, lh, sh);
    const ComboRows c = combo_rows<R>(p, i, lf, sf, j, lh, sh);
    const bool s0 = ok && held<R>(p, c.tbase + cw.t0);
    const bool s1 = ok && cw.n > 1 && held<R>(p, c.tbase + cw.t1);
    // (a rank plan computes rows of the tiles it holds only)
    u32x4* d0 = a.tile_lat + (int64_t)(!R || s0 ? cover_row<R>(p, c, b, cw.t0, cw.a0, cw.s0, w) : 0) * V;
    u32x4* d1 = a.tile_lat + (int64_t)(!R || s1 ? cover_row<R>(p, c, b, cw.t1, cw.a1, cw.s1, w) : 0) * V;
    if (s0) st_nt(d0 + q, x0);
    if (s0 && ok1) st_nt(d0 + v1, x1);
    if (s1) st_nt(d1 + q, x0);
    if (s1 && ok1) st_nt(d1 + v1, x1);
  }
}

// Workgroups are dealt to the XCDs round-robin by index.  Index `bid` of
// `items * parts` workgroups -> (item, part) such that the parts of one item
// get indices equal mod kXcds and so share one L2; items past the last full
// group of kXcds keep the plain order.
__device__ inline void xcd_group(int bid, int items, int parts, int& item, int& part) {
  const int grouped = items / kXcds * kXcds * parts;
  if (bid < grouped) {
    part = (bid / kXcds) % parts;
    item = bid / (kXcds * parts) * kXcds + bid % kXcds;
  } else {
    part = (bid - grouped) % parts;
    item = grouped / parts + (bid - grouped) / parts;
  }
}

// ---------------------------------------------------------------------------
// Conditioning tokens: the extent launch (plans with Nc > 0)
// ---------------------------------------------------------------------------

// Extent launch (Nc > 0), ahead of the selection launch: workgroup (tile
// t, part q) reduces [min start, max end) over rows [q * ext_rows, (q + 1)
// * ext_rows) of tile t's generated tokens on every (batch, axis) plane, NP
// planes per pass with all of a pass's loads in flight and one exchange for
// all of them.  It also clears what the selection launch counts into: part
// 0 the tile's look-back flags, and the workgroups together cond_k.  Every
// tile is reduced, in rank plans too, since k counts the tiles of all
// ranks.  The generated latent rows go to the selection launch, where they
// stream while the selection's chains wait; in the pipeline step the
// extent parts share their launch with the blend instead
// (extent_blend_kernel).
template <int NP>
__device__ void extent_body(const PlanDev& p, const ExtractArgs& a, int bid) {
  __shared__ float2 red[kWaves][NP];
  int t, q;
  xcd_group(bid, p.T, p.ext_parts, t, q);  // the parts of a tile share an L2
  const TileBox tb = tile_box<false>(p, t);
  const int r_begin = min(tb.s.gen, q * p.ext_rows), r_end = min(tb.s.gen, r_begin + p.ext_rows);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int planes = p.B * 3;
  constexpr int RP = kSelLoads / NP;  // rows per thread per pass
  if (q == 0) {
    uint32_t* flags = ws_flags(p, a) + (int64_t)t * p.n_chunks;
    for (int i = tid; i < p.n_chunks; i += kBlock) flags[i] = 0u;
  }
  for (int c = bid * kBlock + tid; c < p.Nc; c += a.n_ext * kBlock) a.cond_k[c] = 0;
  float2* out = ws_part_w(p, a) + ((int64_t)t * p.ext_parts + q) * planes;
  // (a repeated row or plane leaves a minimum and a maximum as they are;
  // an empty part stores +inf and -inf, which the combine ignores)
  for (int e0 = 0; e0 < planes; e0 += NP) {
    float lo[NP], hi[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      lo[k] = INFINITY;
      hi[k] = -INFINITY;
    }
    for (int r0 = r_begin; r0 < r_end; r0 += kBlock * RP) {
      f32x2 v[RP][NP];
#pragma unroll
      for (int u = 0; u < RP; ++u) {
        const int r = r0 + u * kBlock + tid;
        const int n = tile_row_source(p, tb, r < r_end ? r : r_begin);
#pragma unroll
        for (int k = 0; k < NP; ++k) v[u][k] = ld_plane(a.pos + (int64_t)min(e0 + k, planes - 1) * p.rows, n);
      }
#pragma unroll
      for (int u = 0; u < RP; ++u)
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          lo[k] = fminf(lo[k], v[u][k].x);
          hi[k] = fmaxf(hi[k], v[u][k].y);
        }
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      lo[k] = wave_min(lo[k]);
      hi[k] = wave_max(hi[k]);
    }
    if (lane == 0)
#pragma unroll
      for (int k = 0; k < NP; ++k) red[wave][k] = make_float2(lo[k], hi[k]);
    __syncthreads();
    if (tid < NP && e0 + tid < planes) {
      float2 x = red[0][tid];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        x.x = fminf(x.x, red[w][tid].x);
        x.y = fmaxf(x.y, red[w][tid].y);
      }
      out[e0 + tid] = x;
    }
    __syncthreads();  // red is reused by the next pass
  }
}
template <int NP>
__global__ __launch_bounds__(kBlock) void extent_kernel(const PlanDev p, const ExtractArgs a) {
  extent_body<NP>(p, a, blockIdx.x);
}

// Every position workgroup of a launch: (tile, batch, axis, part) of `bid`.
struct PosWork {
  int t, slot, b, d, part;
};
template <bool R>
__device__ inline PosWork pos_work(const PlanDev& p, const ExtractArgs& a, int bid) {
  // every part of a plane reads the whole plane: keep them on one XCD
  PosWork w;
  int plane;
  xcd_group(bid, a.n_pos / a.pos_parts, a.pos_parts, plane, w.part);
  w.d = plane % 3;
  w.b = (plane / 3) % p.B;
  w.slot = plane / (3 * p.B);
  w.t = R ? p.rank + w.slot * p.world : w.slot;
  return w;
}

// Extract without conditioning tokens: one launch, two kinds of
// workgroups that share nothing:
//   [0, n_pos)                 positions per (tile, batch, axis, part);
//   [n_pos, + latent blocks)   generated latent rows per (line, chunk).
// Position workgroups are few and run a longer chain of dependent loads,
// so they come first and run under the latent copy.  Rank plans: the held
// tiles only.
template <bool R>
__global__ __launch_bounds__(kBlock) void extract_kernel(const PlanDev p, const ExtractArgs a) {
  __shared__ ExtractShared sm;
  const int bid = blockIdx.x;
  if (bid < a.n_pos) {
    const PosWork w = pos_work<R>(p, a, bid);
    extract_positions<R>(p, a, sm, w.t, w.slot, w.b, w.d, w.part);
    return;
  }
  extract_latent<R>(p, a, bid - a.n_pos);
}

// Extract with conditioning tokens, after the extent launch: one launch,
// three kinds of workgroups:
//   [0, n_sel)                 one per (tile, chunk of kCondChunk tokens),
//                              tile-major: selection and kept rows;
//   [n_sel, n_sel + n_pos)     positions per (tile, batch, axis, part),
//                              shifted by the tile's extent parts;
//   [.., + latent blocks)      generated latent rows per (line, chunk)
//                              (none in tdp_extract_positions' launch).
// Only wave 0 of a selection workgroup waits on others (the flags of the
// tile's earlier chunks), never without bound.  Rank plans: selection over
// every tile (k counts the tiles of all ranks), the rest for the held
// tiles.
template <bool R, bool SMALL>
__global__ __launch_bounds__(kBlock) void select_kernel(const PlanDev p, const ExtractArgs a) {
  const int bid = blockIdx.x;
  if (bid < a.n_sel) {
    extern __shared__ float2 ext_s[];  // dynamic: at least B * 3 (the launch asks for it)
    __shared__ CondShared cs;
    const int t = bid / p.n_chunks;
    extract_cond_chunk<R, SMALL>(p, a, cs, ext_s, t, bid - t * p.n_chunks);
    return;
  }
  if (bid - a.n_sel < a.n_pos) {
    const PosWork w = pos_work<R>(p, a, bid - a.n_sel);
    extract_positions_copy<R>(p, a, w.t, w.b, w.d, w.part,
                              p.normalize ? tile_min_start(p, a, w.t, w.b * 3 + w.d) : 0.0f);
    return;
  }
  extract_latent<R>(p, a, bid - a.n_sel - a.n_pos);
}

// ---------------------------------------------------------------------------
// latent gather from a selection already made (tdp_extract_latent)
// ---------------------------------------------------------------------------

// Held tiles per conditioning workgroup of the latent gather: kGatherTiles
// when that still leaves a workgroup per compute unit, else half as many
// (fewer tokens: more, shorter workgroups).
__host__ __device__ inline int gather_tiles(const PlanDev& p) {
  return p.n_chunks * ((p.T_local + kGatherTiles - 1) / kGatherTiles) >= 256 ? kGatherTiles : kGatherTiles / 2;
}

// Workgroup (chunk of kCondChunk conditioning tokens, group of gather_tiles
// held tiles): it loads the chunk's rows (every batch element) and the
// group's cond_row entries for those tokens in one round trip, then stores
// each row at the slot row of every tile in the group that keeps it.  A
// token kept by many tiles (a reference token is kept by all) is read once
// per group, not once per tile; the groups of a chunk run on one XCD, so
// its rows come from HBM about once.  cond_row comes from the selection of
// the same positions, so the rows land where tdp_extract puts them.
template <bool R>
__device__ void gather_cond_tokens(const PlanDev& p, const ExtractArgs& a, int bid) {
  __shared__ int row_s[kGatherTiles][kCondChunk];  // slot row per (tile of the group, token); -1: not kept
  __shared__ int64_t base_s[kGatherTiles];         // tile_lat row of slot row 0, batch 0
  __shared__ int cap_s[kGatherTiles];
  const int G = gather_tiles(p);
  const int n_groups = (p.T_local + G - 1) / G;
  int ch, grp;
  xcd_group(bid, p.n_chunks, n_groups, ch, grp);  // the groups of a chunk share an L2
  const int tid = threadIdx.x, V = p.vin;
  const int c0 = ch * kCondChunk;
  const int ntok = min(kCondChunk, p.Nc - c0);
  const int s0 = grp * G, ng = min(G, p.T_local - s0);
  const int all_vec = p.B * ntok * V;  // (b, token j, vector), vector fastest
  const FastDiv by_ntok = make_fastdiv((uint32_t)ntok);
  for (int e0 = 0; e0 < all_vec; e0 += kBlock * kCopyBatch) {
    u32x4 v[kCopyBatch];
#pragma unroll
    for (int q = 0; q < kCopyBatch; ++q) {
      const int e = min(e0 + q * kBlock + tid, all_vec - 1);
      const int row = (int)fastdiv((uint32_t)e, p.by_vin), vv = e - row * V;
      const int b = (int)fastdiv((uint32_t)row, by_ntok), j = row - b * ntok;
      v[q] = ld_nt(a.latent + ((int64_t)b * p.rows + p.N + c0 + j) * V + vv);
    }
    if (e0 == 0) {  // the group's entries, in flight with the first rows
      static_assert(kGatherTiles * kCondChunk <= kBlock, "one entry per thread");
      const int gs = tid / kCondChunk, j = tid - gs * kCondChunk;
      if (gs < ng) {
        const int slot = s0 + gs;
        const int t = R ? p.rank + slot * p.world : slot;
        row_s[gs][j] = j < ntok ? a.cond_row[(int64_t)t * p.Nc + c0 + j] : -1;
        if (j == 0) {
          const TileBox tb = tile_box<R>(p, t);
          base_s[gs] = tb.s.row_base;
          cap_s[gs] = tb.s.cap;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < kCopyBatch; ++q) {
      const int e = e0 + q * kBlock + tid;
      if (e < all_vec) {
        const int row = (int)fastdiv((uint32_t)e, p.by_vin), vv = e - row * V;
        const int b = (int)fastdiv((uint32_t)row, by_ntok), j = row - b * ntok;
        for (int gs = 0; gs < ng; ++gs) {
          const int r = row_s[gs][j];
          if ((uint32_t)r < (uint32_t)cap_s[gs])  // -1: not kept; nothing lands outside the slot
            st_nt(a.tile_lat + (base_s[gs] + (int64_t)b * cap_s[gs] + r) * V + vv, v[q]);
        }
      }
    }
  }
}

// Conditioning workgroups of the latent gather: (chunk, group of held tiles).
__host__ __device__ inline int gather_cond_blocks(const PlanDev& p) {
  const int G = gather_tiles(p);
  return p.Nc > 0 && p.T_local > 0 ? p.n_chunks * ((p.T_local + G - 1) / G) : 0;
}

// tdp_extract_latent: [0, n_cg) conditioning workgroups (chunk, group of
// held tiles; one round trip each, so first), then the generated latent rows
// per (line, chunk), as in the extract.
template <bool R>
__global__ __launch_bounds__(kBlock) void gather_kernel(const PlanDev p, const ExtractArgs a, int n_cg) {
  const int bid = blockIdx.x;
  if (bid < n_cg) {
    gather_cond_tokens<R>(p, a, bid);
    return;
  }
  extract_latent<R>(p, a, bid - n_cg);
}

// ---------------------------------------------------------------------------
// blend
// ---------------------------------------------------------------------------

// Terms of NC frame x height combos (cr, wfh) for the lane's row w and its
// NV vectors vs[], added into acc[k] in ascending tile order: combos ascend
// in (i_f, i_h), then the width covers.  TWO: some row of the wave has a
// second width cover; then every lane loads both covers (a missing second
// one re-reads the first row and is left out of the sum).  Without TWO only
// the first cover is loaded.  R (rank plan): a term of a tile the plan does
// not hold re-reads a vector of slot 0 (there is one: workgroups outside
// the held tiles' box never get here) and is left out.
template <int IN, int OUT, int NC, int NV, bool TWO, bool R>
__device__ inline void blend_terms(const PlanDev& p, const ComboRows* cr, const float* wfh, const Covers& cw,
                                   float wx, float wy, int b, int w, const int* vs,
                                   const u32x4* __restrict__ tile_out, float (&acc)[NV][InVec<IN>::E]) {
  constexpr int E = InVec<IN>::E;
  using IO = LaneIO<IN, OUT>;
  const int V = p.vin;
  u32x4 y0[NC][NV], y1[NC][NV];
  bool h0[NC], h1[NC];  // the term is held (always, for a whole plan)
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    h0[cb] = held<R>(p, cr[cb].tbase + cw.t0);
    const int64_t r0 = h0[cb] ? (int64_t)cover_row<R>(p, cr[cb], b, cw.t0, cw.a0, cw.s0, w) * V : 0;
#pragma unroll
    for (int k = 0; k < NV; ++k) y0[cb][k] = IO::load(tile_out, r0 + vs[k], vs[k], V);
    if (TWO) {
      h1[cb] = held<R>(p, cr[cb].tbase + cw.t1);
      const int64_t r1 = h1[cb] ? (int64_t)cover_row<R>(p, cr[cb], b, cw.t1, cw.a1, cw.s1, w) * V : 0;
#pragma unroll
      for (int k = 0; k < NV; ++k) y1[cb][k] = IO::load(tile_out, r1 + vs[k], vs[k], V);
    }
  }
  const bool has1 = cw.n > 1;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      const float wa = wfh[cb] * wx;
      float x0[E];
      InVec<IN>::unpack(y0[cb][k], x0);
      const bool use0 = h0[cb];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[k][e] = use0 ? fmaf(wa, x0[e], acc[k][e]) : acc[k][e];
      if (TWO) {
        const float wb = wfh[cb] * wy;
        float x1[E];
        InVec<IN>::unpack(y1[cb][k], x1);
        const bool use1 = has1 && h1[cb];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[k][e] = use1 ? fmaf(wb, x1[e], acc[k][e]) : acc[k][e];
      }
    }
  }
}

// Lane (r, q) owns row w = w0 + r of its wave's unit and its vectors q and
// lpr + q; it sums the row's covering tile rows in fp32 and rounds once.
// With up to two combos both vectors are in flight together; four combos (a
// tiled frame axis) take one vector at a time, so a lane never holds more
// than eight loads.
template <int IN, int OUT, int NC, bool TWO, bool R>
__device__ inline void blend_lane(const PlanDev& p, const LineCombos& lc, int f, int h, const Covers& cw, int b,
                                  int w, bool ok, int q, const u32x4* __restrict__ tile_out,
                                  void* __restrict__ out, int64_t dst_row) {
  constexpr int E = InVec<IN>::E;
  using IO = LaneIO<IN, OUT>;
  ComboRows cr[NC];
  float wfh[NC];
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    int i, lf, sf, j, lh, sh;
    lc.get(cb, f, h, i, lf, sf, j, lh, sh);
    cr[cb] = combo_rows<R>(p, i, lf, sf, j, lh, sh);
    wfh[cb] = ramp_weight(p.ax[0], i, lf, sf) * ramp_weight(p.ax[1], j, lh, sh);
  }
  const int v1 = p.lpr + q;
  const bool ok1 = v1 < p.vin;
  const int vs[2] = {q, ok1 ? v1 : q};
  const float wx = ramp_weight(p.ax[2], cw.t0, w - cw.a0, cw.s0);
  const float wy = TWO && cw.n > 1 ? ramp_weight(p.ax[2], cw.t1, w - cw.a1, cw.s1) : 0.0f;
  if constexpr (NC <= 2) {
    float acc[2][E];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[k][e] = 0.0f;
    blend_terms<IN, OUT, NC, 2, TWO, R>(p, cr, wfh, cw, wx, wy, b, w, vs, tile_out, acc);
    if (ok) IO::store(out, dst_row, q, p.vin, acc[0]);
    if (ok && ok1) IO::store(out, dst_row, v1, p.vin, acc[1]);
  } else {
#pragma unroll 1
    for (int k = 0; k < 2; ++k) {
      float acc[1][E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[0][e] = 0.0f;
      blend_terms<IN, OUT, NC, 1, TWO, R>(p, cr, wfh, cw, wx, wy, b, w, vs + k, tile_out, acc);
      if (ok && (k == 0 || ok1)) IO::store(out, dst_row, vs[k], p.vin, acc[0]);
    }
  }
}

// Rows [w0, w0 + rwv) of one (b, f, h) line, one wave, with exactly NC
// frame x height combos (wave-uniform row bases and weights); the wave takes
// the single-cover path unless one of its rows lies in two width tiles.
template <int IN, int OUT, int NC, bool R>
__device__ void blend_line(const PlanDev& p, const LineCombos& lc, int b, int f, int h, int w0,
                           const u32x4* __restrict__ tile_out, void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int r = (int)fastdiv((uint32_t)lane, p.by_lpr), q = lane - r * p.lpr;
  const int wr = w0 + r;
  const bool ok = r < p.rwv && wr < p.W;
  const int w = ok ? wr : w0;  // w0 < W
  const Covers cw = split_covers(p.ax[2], w);
  const int64_t dst_row = (int64_t)b * p.rows + ((int64_t)f * p.H + h) * p.W + w;
  // wave-uniform: most waves lie inside one width tile
  if (__any(ok && cw.n > 1))
    blend_lane<IN, OUT, NC, true, R>(p, lc, f, h, cw, b, w, ok, q, tile_out, out, dst_row);
  else
    blend_lane<IN, OUT, NC, false, R>(p, lc, f, h, cw, b, w, ok, q, tile_out, out, dst_row);
}

// Generated rows: one wave per unit of rwv rows of one (b, f, h) line, the
// waves of a workgroup on consecutive units, one pass each; many short
// workgroups let the dispatcher overlap the tail of one with the start of
// the next, and no lane idles at the end of a line unless W % rwv != 0.
// Conditioning rows: (1/k) * sum, ascending t, over the k tiles that keep
// the token (k = non-negative entries of its cond_row column; 0 when k = 0).
// Workgroup `cid` = (batch element, chunk of kCondTokens tokens).  The
// chunk's cond_row entries and every tile's slot go to LDS in one parallel
// pass; one thread per token then lists the tiles whose rows it sums, in
// ascending t, so each lane loads only those rows, kCondBatch at a time (one
// round for k <= 8; conditioned 4K-class workload: 15.8 -> 11.2 us, against
// loading every tile's row and masking).  A rank plan counts k over every
// tile but sums only the tiles it holds (capacity 0 for the others).
template <int IN, int OUT, bool R>
__device__ void blend_cond_cached(const PlanDev& p, const u32x4* __restrict__ tile_out,
                                  const int32_t* __restrict__ cond_row, const int32_t* __restrict__ cond_k,
                                  void* __restrict__ out, int cid) {
  constexpr int E = InVec<IN>::E;
  // LDS: rowtab[T][kCondTokens], cap[T], k[kCondTokens], n[kCondTokens],
  // list[kCondTokens][T] (slot rows of the terms, ascending t), base[T] (int64)
  extern __shared__ int cond_lds[];
  int* rowtab = cond_lds;
  int* cap = rowtab + p.T * kCondTokens;
  int* kcount = cap + p.T;
  int* nterms = kcount + kCondTokens;
  int* list = nterms + kCondTokens;
  int64_t* base = reinterpret_cast<int64_t*>(list + kCondTokens * p.T);
  base = reinterpret_cast<int64_t*>((reinterpret_cast<uintptr_t>(base) + 7) & ~uintptr_t(7));
  const int per_b = (p.Nc + kCondTokens - 1) / kCondTokens;
  const int b = cid / per_b;
  const int c0 = (cid - b * per_b) * kCondTokens;
  const int ntok = min(kCondTokens, p.Nc - c0);
  for (int t = threadIdx.x; t < p.T; t += kBlock) {
    int i, j, k;
    tile_grid(p, t, i, j, k);
    const TileSlot sl = slot_of<R>(p, i, j, k);
    cap[t] = held<R>(p, t) ? sl.cap : 0;
    base[t] = sl.row_base + (int64_t)b * sl.cap;
  }
  for (int e = threadIdx.x; e < p.T * kCondTokens; e += kBlock) {
    const int t = e / kCondTokens, jj = e - t * kCondTokens;
    rowtab[e] = jj < ntok ? cond_row[(int64_t)t * p.Nc + c0 + jj] : -1;
  }
  __syncthreads();
  // per token: k (tiles that keep it, from extract) and the terms summed
  // here (kept rows tdp_extract could have written), ascending t
  if (threadIdx.x < kCondTokens) {
    const int jj = threadIdx.x;
    int n = 0;
    for (int t = 0; t < p.T; ++t) {
      const int row = rowtab[t * kCondTokens + jj];
      if (row >= 0 && row < cap[t]) list[jj * p.T + n++] = t;
    }
    kcount[jj] = jj < ntok ? cond_k[c0 + jj] : 0;
    nterms[jj] = n;
  }
  __syncthreads();
  const int V = p.vin;
  const int r = (int)fastdiv(threadIdx.x, p.by_vin), vv = threadIdx.x - r * V;
  if (r >= p.rpp) return;
  if (R && p.T_local == 0) {  // a rank without tiles: zeros, and no slot 0 to re-read
    float z[E];
#pragma unroll
    for (int e = 0; e < E; ++e) z[e] = 0.0f;
    for (int jj = r; jj < ntok; jj += p.rpp)
      store_out<OUT, E>(out, (((int64_t)b * p.rows + p.N + c0 + jj) * V + vv) * (int64_t)E, z);
    return;
  }
  for (int jj = r; jj < ntok; jj += p.rpp) {
    const int kc = kcount[jj], n = nterms[jj];
    const float inv = kc > 0 ? 1.0f / (float)kc : 0.0f;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    const int* lj = list + jj * p.T;
    for (int q0 = 0; q0 < n; q0 += kCondBatch) {
      // only the terms: slots past the list re-read its last term, left out
      u32x4 y[kCondBatch];
#pragma unroll
      for (int q = 0; q < kCondBatch; ++q) {
        const int t = lj[min(q0 + q, n - 1)];
        y[q] = ld_nt(tile_out + (base[t] + rowtab[t * kCondTokens + jj]) * V + vv);
      }
#pragma unroll
      for (int q = 0; q < kCondBatch; ++q) {
        float x[E];
        InVec<IN>::unpack(y[q], x);
        const bool use = q0 + q < n;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = use ? fmaf(inv, x[e], acc[e]) : acc[e];
      }
    }
    store_out<OUT, E>(out, (((int64_t)b * p.rows + p.N + c0 + jj) * V + vv) * (int64_t)E, acc);
  }
}

// The same sum for plans with more than kCondTiles tiles, one tile at a time.
template <int IN, int OUT, bool R>
__device__ void blend_cond_direct(const PlanDev& p, const u32x4* __restrict__ tile_out,
                                  const int32_t* __restrict__ cond_row, const int32_t* __restrict__ cond_k,
                                  void* __restrict__ out, int cid) {
  constexpr int E = InVec<IN>::E;
  const int V = p.vin;
  const int r = (int)fastdiv(threadIdx.x, p.by_vin), vv = threadIdx.x - r * V;
  if (r >= p.rpp) return;
  const int per_b = (p.Nc + kCondTokens - 1) / kCondTokens;
  const int b = cid / per_b;
  const int c0 = (cid - b * per_b) * kCondTokens;
  const int ntok = min(kCondTokens, p.Nc - c0);
  for (int jj = r; jj < ntok; jj += p.rpp) {
    const int c = c0 + jj;
    const int kc = cond_k[c];
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    if (kc > 0) {
      const float inv = 1.0f / (float)kc;
      for (int t = 0; t < p.T; ++t) {
        const int row = cond_row[(int64_t)t * p.Nc + c];
        if (row < 0 || !held<R>(p, t)) continue;
        int i, j, k;
        tile_grid(p, t, i, j, k);
        const TileSlot sl = slot_of<R>(p, i, j, k);
        if (row >= sl.cap) continue;  // not a row tdp_extract could have written
        const u32x4 yv = ld_nt(tile_out + (sl.row_base + (int64_t)b * sl.cap + row) * V + vv);
        float x[E];
        InVec<IN>::unpack(yv, x);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(inv, x[e], acc[e]);
      }
    }
    store_out<OUT, E>(out, (((int64_t)b * p.rows + p.N + c) * V + vv) * (int64_t)E, acc);
  }
}

// Rank plans: zero-fill workgroup `zl` (a (b, f, h) line of the partial
// buffer) writes zeros on the line's rows that no box unit writes: rows
// outside the box's width chunks, or the whole line when it lies outside
// the box on frames or height.  Plain contiguous stores, 16 bytes where the
// output row allows (its bytes are always a multiple of 8).
template <int OUT>
__device__ void blend_zero_line(const PlanDev& p, void* __restrict__ out, int zl) {
  const int b = (int)fastdiv((uint32_t)zl, p.by_FH);
  const int fh = zl - b * (p.F * p.H);
  const int f = (int)fastdiv((uint32_t)fh, p.by_H), h = fh - f * p.H;
  const bool in_box = p.box_nc > 0 && f >= p.box_f0 && f < p.box_f0 + p.box_nf && h >= p.box_h0 &&
                      h < p.box_h0 + p.box_nh;
  const int w_lo = in_box ? p.box_c0 * p.blend_rows : p.W;       // [0, w_lo) and [w_hi, W) are zero
  const int w_hi = in_box ? min(p.W, (p.box_c0 + p.box_nc) * p.blend_rows) : p.W;
  const int64_t row_bytes = (int64_t)p.C * (OUT == TDP_BF16 ? 2 : 4);
  char* line = static_cast<char*>(out) + ((int64_t)b * p.rows + ((int64_t)f * p.H + h) * p.W) * row_bytes;
  const int seg[2][2] = {{0, w_lo}, {w_hi, p.W}};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (seg[k][1] <= seg[k][0]) continue;
    char* base = line + seg[k][0] * row_bytes;
    const int64_t bytes = (int64_t)(seg[k][1] - seg[k][0]) * row_bytes;
    if (row_bytes % 16 == 0) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int64_t i = threadIdx.x; i < bytes / 16; i += kBlock) st_nt(reinterpret_cast<u32x4*>(base) + i, z);
    } else {
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 z = {0u, 0u};
      for (int64_t i = threadIdx.x; i < bytes / 8; i += kBlock) st_nt(reinterpret_cast<u32x2*>(base) + i, z);
    }
  }
}

// F2: the frame axis is tiled, so a line can have four frame x height
// combos; only plans with a tiled frame axis carry that path (and its
// registers).
// Generated-row workgroup `gid` of a blend: each wave takes one unit (rows
// [w0, w0 + rwv) of one line), the waves of a workgroup consecutive units.
// A rank plan's units tile its held tiles' bounding box (as the extract's),
// and the workgroups after them zero-fill the rest of each line.
template <int IN, int OUT, bool R, bool F2, int W = kWaves>
__device__ void blend_gen(const PlanDev& p, const u32x4* __restrict__ tile_out, void* __restrict__ out, int gid) {
  static_assert(!R || W == kWaves, "a rank plan's zero-fill strides by a whole workgroup of kBlock threads");
  int line, w0, b, f, h;
  const int rows = p.blend_rows;
  if constexpr (R) {
    const int n_box = (p.gen_units + kWaves - 1) / kWaves;
    if (gid >= n_box) {
      blend_zero_line<OUT>(p, out, gid - n_box);
      return;
    }
    const int unit = __builtin_amdgcn_readfirstlane(gid * kWaves + (int)(threadIdx.x >> 6));
    if (unit >= p.gen_units) return;
    line = (int)fastdiv((uint32_t)unit, p.by_box_c);
    w0 = (p.box_c0 + unit - line * p.box_nc) * rows;
    b = (int)fastdiv((uint32_t)line, p.by_box_fh);
    const int fh = line - b * (p.box_nf * p.box_nh);
    const int fb = (int)fastdiv((uint32_t)fh, p.by_box_h);
    f = p.box_f0 + fb;
    h = p.box_h0 + fh - fb * p.box_nh;
  } else {
    const int unit = __builtin_amdgcn_readfirstlane(gid * W + (int)(threadIdx.x >> 6));
    if (unit >= p.gen_units) return;
    line = (int)fastdiv((uint32_t)unit, p.by_blend_chunks);
    w0 = (unit - line * p.blend_chunks) * rows;
    b = (int)fastdiv((uint32_t)line, p.by_FH);
    const int fh = line - b * (p.F * p.H);
    f = (int)fastdiv((uint32_t)fh, p.by_H);
    h = fh - f * p.H;
  }
  LineCombos lc;
  lc.init(p, f, h);
  if (lc.n == 1)
    blend_line<IN, OUT, 1, R>(p, lc, b, f, h, w0, tile_out, out);
  else if (!F2 || lc.n == 2)
    blend_line<IN, OUT, 2, R>(p, lc, b, f, h, w0, tile_out, out);
  else
    blend_line<IN, OUT, F2 ? 4 : 2, R>(p, lc, b, f, h, w0, tile_out, out);
}

// Workgroup `bid` of a blend whose first n_cond workgroups take the
// conditioning rows.
template <int IN, int OUT, bool R, bool F2>
__device__ void blend_body(const PlanDev& p, const u32x4* __restrict__ tile_out, const int32_t* __restrict__ cond_row,
                           const int32_t* __restrict__ cond_k, void* __restrict__ out, int bid, int n_cond) {
  // conditioning workgroups first: each is a short dependent chain, so they
  // start early and run under the generated rows
  if (bid < n_cond) {
    if (p.T <= kCondTiles)
      blend_cond_cached<IN, OUT, R>(p, tile_out, cond_row, cond_k, out, bid);
    else
      blend_cond_direct<IN, OUT, R>(p, tile_out, cond_row, cond_k, out, bid);
    return;
  }
  blend_gen<IN, OUT, R, F2>(p, tile_out, out, bid - n_cond);
}
template <int IN, int OUT, bool R, bool F2>
__global__ __launch_bounds__(kBlock) void blend_kernel(const PlanDev p, const u32x4* __restrict__ tile_out,
                                                       const int32_t* __restrict__ cond_row,
                                                       const int32_t* __restrict__ cond_k,
                                                       void* __restrict__ out, int n_gen_blocks) {
  blend_body<IN, OUT, R, F2>(p, tile_out, cond_row, cond_k, out, blockIdx.x, (int)gridDim.x - n_gen_blocks);
}

// Whole plans without conditioning tokens: the blend in one-wave
// workgroups, one unit each.  The per-CU cap holds a workgroup's share of
// the compute unit until its last wave ends; with one wave, a unit that
// finishes frees its share at once instead of waiting for the slowest of
// four (4K-class latent: 18.4 -> 17.8 us).
template <int IN, int OUT, bool F2>
__global__ __launch_bounds__(64) void blend_wave_kernel(const PlanDev p, const u32x4* __restrict__ tile_out,
                                                        void* __restrict__ out) {
  blend_gen<IN, OUT, false, F2, 1>(p, tile_out, out, blockIdx.x);
}

// The latent step of such a plan in one-wave workgroups: generated latent
// rows, then the blend's units.
template <int IN, int OUT, bool F2>
__global__ __launch_bounds__(64) void pipeline_latent_wave_kernel(const PlanDev p, const ExtractArgs a,
                                                                  const u32x4* __restrict__ tile_out,
                                                                  void* __restrict__ out, int n_ext) {
  const int bid = blockIdx.x;
  if (bid < n_ext) {
    extract_latent<false, 1>(p, a, bid);
    return;
  }
  blend_gen<IN, OUT, false, F2, 1>(p, tile_out, out, bid - n_ext);
}

// The first launch of a pipeline step for plans with conditioning tokens:
// the extent parts of one latent's tiles (short chains of loads; every
// tile, since k counts the tiles of all ranks), then the blend of other
// tile outputs (its conditioning rows, then its generated rows; R: a rank's
// partial buffer), so the blend's bulk copy runs under the extent chains.
// The selection launch that follows (select_kernel) holds the selection,
// the positions and the generated latent rows, which stream while the
// selection's chains wait.  The two halves share no buffer.
template <int NP, int IN, int OUT, bool F2, bool R>
__global__ __launch_bounds__(kBlock) void extent_blend_kernel(const PlanDev p, const ExtractArgs a,
                                                              const u32x4* __restrict__ tile_out,
                                                              const int32_t* __restrict__ blend_cond_row,
                                                              const int32_t* __restrict__ blend_cond_k,
                                                              void* __restrict__ out, int n_bcond) {
  const int bid = blockIdx.x;
  if (bid < a.n_ext) {
    extent_body<NP>(p, a, bid);
    return;
  }
  blend_body<IN, OUT, R, F2>(p, tile_out, blend_cond_row, blend_cond_k, out, bid - a.n_ext, n_bcond);
}

// One step of a pipelined loop whose positions do not change (R: a rank's share):
// the latent gather of one latent (tdp_extract_latent: conditioning chunks,
// then generated rows) and the blend of other tile outputs, as one launch.
// Every workgroup is a copy or a short chain; none waits on another.
template <int IN, int OUT, bool F2, bool R>
__global__ __launch_bounds__(kBlock) void pipeline_latent_kernel(const PlanDev p, const ExtractArgs a,
                                                                 const u32x4* __restrict__ tile_out,
                                                                 const int32_t* __restrict__ blend_cond_row,
                                                                 const int32_t* __restrict__ blend_cond_k,
                                                                 void* __restrict__ out, int n_cg, int n_ext,
                                                                 int n_bcond) {
  const int bid = blockIdx.x;
  if (bid < n_cg) {
    gather_cond_tokens<R>(p, a, bid);
    return;
  }
  if (bid < n_ext) {
    extract_latent<R>(p, a, bid - n_cg);
    return;
  }
  blend_body<IN, OUT, R, F2>(p, tile_out, blend_cond_row, blend_cond_k, out, bid - n_ext, n_bcond);
}

// One step of a pipelined loop (plans without conditioning tokens; R: a
// rank's share, its tiles' extract and its partial buffer): the extract of
// one latent and the blend of other tile outputs that share no buffer with
// it, as one launch.  Grid: the extract's workgroups
// (positions, then latent rows) and then the blend's, so the blend's fill
// the compute units as the extract's drain instead of waiting for a kernel
// boundary.  Each workgroup runs exactly the code of its own kernel.
template <int IN, int OUT, bool F2, bool R>
__global__ __launch_bounds__(kBlock) void pipeline_kernel(const PlanDev p, const ExtractArgs a,
                                                          const u32x4* __restrict__ tile_out,
                                                          void* __restrict__ out, int n_ext) {
  __shared__ ExtractShared sm;
  const int bid = blockIdx.x;
  if (bid < n_ext) {
    if (bid < a.n_pos) {
      const PosWork w = pos_work<R>(p, a, bid);
      extract_positions<R>(p, a, sm, w.t, w.slot, w.b, w.d, w.part);
      return;
    }
    extract_latent<R>(p, a, bid - a.n_pos);
    return;
  }
  if constexpr (R) {
    blend_gen<IN, OUT, R, F2>(p, tile_out, out, bid - n_ext);
  } else {
    // the blend's generated rows written out here rather than through
    // blend_gen: the same code, but hipcc then gives this kernel 63 VGPRs
    // instead of 65, and the 4K step is ~0.08 us shorter
    const int unit = __builtin_amdgcn_readfirstlane((bid - n_ext) * kWaves + (int)(threadIdx.x >> 6));
    if (unit >= p.gen_units) return;
    const int rows = p.blend_rows;
    const int line = (int)fastdiv((uint32_t)unit, p.by_blend_chunks);
    const int w0 = (unit - line * p.blend_chunks) * rows;
    const int b = (int)fastdiv((uint32_t)line, p.by_FH);
    const int fh = line - b * (p.F * p.H);
    const int f = (int)fastdiv((uint32_t)fh, p.by_H), h = fh - f * p.H;
    LineCombos lc;
    lc.init(p, f, h);
    if (lc.n == 1)
      blend_line<IN, OUT, 1, false>(p, lc, b, f, h, w0, tile_out, out);
    else if (!F2 || lc.n == 2)
      blend_line<IN, OUT, 2, false>(p, lc, b, f, h, w0, tile_out, out);
    else
      blend_line<IN, OUT, F2 ? 4 : 2, false>(p, lc, b, f, h, w0, tile_out, out);
  }
}

// Occupancy caps.  Both kernels move more bytes per microsecond with fewer
// workgroups sharing a compute unit than the registers allow (7 or 8 per
// CU): fewer requests in flight per CU, and the long position and selection
// workgroups of extract finish sooner.  Measured on the 4K-class latent:
// extract 22.2 us at 7 per CU, 21.0 us at 3, 22.5 us at 2; blend 18.9 us at
// 8, 18.4 us at 4, 19.7 us at 3.  Extracts with fewer latent workgroups are
// set by their position and selection chains and do best at 2 per CU
// (full-res latent 7.7 -> 6.6 us, conditioned 23.2 -> 20.4 us).  A launch
// holds the cap by asking for dynamic LDS that only k workgroups fit in.
struct DeviceShape {
  int lds_per_cu;     // bytes of LDS per compute unit (0: unknown)
  int lds_per_block;  // largest LDS request of one workgroup
  int cus;            // compute units
};
DeviceShape device_shape() {
  static std::atomic<int> cache[64][3];  // value + 1; 0 = not queried yet
  DeviceShape d{0, 0, 0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return d;
  const hipDeviceAttribute_t attr[3] = {hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                        hipDeviceAttributeMaxSharedMemoryPerBlock,
                                        hipDeviceAttributeMultiprocessorCount};
  int v[3];
  for (int i = 0; i < 3; ++i) {
    int c = cache[dev][i].load(std::memory_order_relaxed);
    if (c == 0) {
      int x = 0;
      if (hipDeviceGetAttribute(&x, attr[i], dev) != hipSuccess || x < 0) x = 0;
      c = x + 1;
      cache[dev][i].store(c, std::memory_order_relaxed);
    }
    v[i] = c - 1;
  }
  d.lds_per_cu = v[0];
  d.lds_per_block = v[1];
  d.cus = v[2];
  return d;
}
// Dynamic LDS for a launch that needs `need` bytes and should put at most
// k workgroups on one compute unit (the static LDS of the kernel is small
// and only lowers the count further).
size_t capped_lds(const DeviceShape& d, size_t need, int k) {
  if (d.lds_per_cu <= 0) return need;
  size_t cap = (size_t)d.lds_per_cu / (size_t)(k + 1) + 1;  // k of these fit, k + 1 do not
  if (d.lds_per_block > 0 && cap > (size_t)d.lds_per_block) cap = need;
  return need > cap ? need : cap;
}
constexpr int kExtractWgsPerCu = 3;       // latent-dominated extracts
constexpr int kExtractWgsPerCuChain = 2;  // extracts set by their position / selection chains
constexpr int kBlendWgsPerCu = 4;
constexpr int kWaveWgsPerCu = 16;         // one-wave workgroups (blend and latent step without conditioning tokens)

// Whole plans without conditioning tokens and more than 16 blend units per
// compute unit run the blend (and the latent step) in one-wave workgroups.
// Smaller plans keep four-wave workgroups: there the extra launches of
// single waves cost more than they free (full-res blend 5.2 -> 5.6 us,
// LTX-like 3.4 -> 3.8 us with one wave; 4K-class 18.4 -> 17.8 us).
bool wave_workgroups(const PlanDev& p, const DeviceShape& ds) {
  return p.Nc == 0 && p.world == 1 && p.gen_units > 16 * (ds.cus > 0 ? ds.cus : 256);
}
constexpr int kSelectWgsPerCuLarge = 6;   // selection launches of plans with many chunks per tile
constexpr int kPipelineWgsPerCu = 4;      // pipeline step (extract and blend in one launch)

// The blend's conditioning workgroups, and the LDS of its cached path:
// rowtab, cap, k, n, list (ints), then 8-aligned int64 bases.
// Workgroups of a blend's generated rows: its units, and for a rank plan
// one zero-fill workgroup per line after them.
int blend_gen_blocks(const PlanDev& p) { return (p.gen_units + kWaves - 1) / kWaves + p.zero_lines; }
int blend_cond_blocks(const PlanDev& p) { return p.Nc > 0 ? p.B * ((p.Nc + kCondTokens - 1) / kCondTokens) : 0; }
size_t blend_cond_lds(const PlanDev& p) {
  return p.Nc > 0 && p.T <= kCondTiles
             ? ((size_t)2 * p.T * kCondTokens + p.T + 2 * kCondTokens) * sizeof(int) + 8 + (size_t)p.T * 8
             : 0;
}

template <int IN, int OUT>
hipError_t launch_blend(const PlanDev& p, const void* tile_out, const int32_t* cond_row, const int32_t* cond_k,
                        void* out, hipStream_t s) {
  const u32x4* y = reinterpret_cast<const u32x4*>(tile_out);
  const bool f2 = p.ax[0].n > 1;
  const DeviceShape ds = device_shape();
  if (wave_workgroups(p, ds)) {
    const dim3 wgrid((unsigned)p.gen_units), wblock(64);
    const size_t wlds = capped_lds(ds, 0, kWaveWgsPerCu);
    if (wgrid.x == 0) return hipSuccess;
    if (f2)
      hipLaunchKernelGGL((blend_wave_kernel<IN, OUT, true>), wgrid, wblock, wlds, s, p, y, out);
    else
      hipLaunchKernelGGL((blend_wave_kernel<IN, OUT, false>), wgrid, wblock, wlds, s, p, y, out);
    return hipGetLastError();
  }
  const int n_gen = blend_gen_blocks(p);
  const int n_cond = blend_cond_blocks(p);
  const size_t lds = capped_lds(ds, blend_cond_lds(p), kBlendWgsPerCu);
  const dim3 grid(n_gen + n_cond), block(kBlock);
  if (p.world > 1 && f2)
    hipLaunchKernelGGL((blend_kernel<IN, OUT, true, true>), grid, block, lds, s, p, y, cond_row, cond_k, out, n_gen);
  else if (p.world > 1)
    hipLaunchKernelGGL((blend_kernel<IN, OUT, true, false>), grid, block, lds, s, p, y, cond_row, cond_k, out, n_gen);
  else if (f2)
    hipLaunchKernelGGL((blend_kernel<IN, OUT, false, true>), grid, block, lds, s, p, y, cond_row, cond_k, out, n_gen);
  else
    hipLaunchKernelGGL((blend_kernel<IN, OUT, false, false>), grid, block, lds, s, p, y, cond_row, cond_k, out, n_gen);
  return hipGetLastError();
}

// The latent gather of one latent and the blend of other tile outputs
// (whole and rank plans), one launch: conditioning chunks, generated latent rows,
// then the blend's conditioning and generated workgroups.
template <int IN, int OUT>
hipError_t launch_pipeline_latent(const PlanDev& p, const ExtractArgs& a, const void* tile_out,
                                  const int32_t* blend_cond_row, const int32_t* blend_cond_k, void* out,
                                  const DeviceShape& ds, hipStream_t s) {
  if (wave_workgroups(p, ds)) {
    const dim3 wgrid((unsigned)(p.lat_units + p.gen_units)), wblock(64);
    const size_t wlds = capped_lds(ds, 0, kWaveWgsPerCu);
    if (wgrid.x == 0) return hipSuccess;
    const u32x4* wy = reinterpret_cast<const u32x4*>(tile_out);
    if (p.ax[0].n > 1)
      hipLaunchKernelGGL((pipeline_latent_wave_kernel<IN, OUT, true>), wgrid, wblock, wlds, s, p, a, wy, out,
                         p.lat_units);
    else
      hipLaunchKernelGGL((pipeline_latent_wave_kernel<IN, OUT, false>), wgrid, wblock, wlds, s, p, a, wy, out,
                         p.lat_units);
    return hipGetLastError();
  }
  const int n_cg = gather_cond_blocks(p);
  const int n_ext = n_cg + (p.lat_units + kWaves - 1) / kWaves;
  const int n_bcond = blend_cond_blocks(p);
  const int n_bgen = blend_gen_blocks(p);
  // plans with many conditioning chunks move their rows faster at 6
  // workgroups per CU (16 384 tokens on the conditioned shape: 48.8 -> 47.3
  // us per step), plans with few at 4 (1 024 tokens: 18.6 against 18.8)
  const int cap = p.n_chunks <= kDirectChunks + 1 ? kPipelineWgsPerCu : kSelectWgsPerCuLarge;
  const size_t lds = capped_lds(ds, blend_cond_lds(p), cap);
  const dim3 grid((unsigned)(n_ext + n_bcond + n_bgen)), block(kBlock);
  const u32x4* y = reinterpret_cast<const u32x4*>(tile_out);
  const bool f2 = p.ax[0].n > 1;
  if (p.world > 1 && f2)
    hipLaunchKernelGGL((pipeline_latent_kernel<IN, OUT, true, true>), grid, block, lds, s, p, a, y, blend_cond_row,
                       blend_cond_k, out, n_cg, n_ext, n_bcond);
  else if (p.world > 1)
    hipLaunchKernelGGL((pipeline_latent_kernel<IN, OUT, false, true>), grid, block, lds, s, p, a, y, blend_cond_row,
                       blend_cond_k, out, n_cg, n_ext, n_bcond);
  else if (f2)
    hipLaunchKernelGGL((pipeline_latent_kernel<IN, OUT, true, false>), grid, block, lds, s, p, a, y, blend_cond_row,
                       blend_cond_k, out, n_cg, n_ext, n_bcond);
  else
    hipLaunchKernelGGL((pipeline_latent_kernel<IN, OUT, false, false>), grid, block, lds, s, p, a, y, blend_cond_row,
                       blend_cond_k, out, n_cg, n_ext, n_bcond);
  return hipGetLastError();
}

template <int IN, int OUT>
hipError_t launch_pipeline(const PlanDev& p, const ExtractArgs& a, int n_lat, const void* tile_out, void* out,
                           const DeviceShape& ds, hipStream_t s) {
  const int n_ext = a.n_pos + n_lat;
  const int n_gen = blend_gen_blocks(p);
  const size_t lds = capped_lds(ds, 0, kPipelineWgsPerCu);
  const dim3 grid((unsigned)(n_ext + n_gen)), block(kBlock);
  const u32x4* y = reinterpret_cast<const u32x4*>(tile_out);
  const bool f2 = p.ax[0].n > 1;
  if (p.world > 1 && f2)
    hipLaunchKernelGGL((pipeline_kernel<IN, OUT, true, true>), grid, block, lds, s, p, a, y, out, n_ext);
  else if (p.world > 1)
    hipLaunchKernelGGL((pipeline_kernel<IN, OUT, false, true>), grid, block, lds, s, p, a, y, out, n_ext);
  else if (f2)
    hipLaunchKernelGGL((pipeline_kernel<IN, OUT, true, false>), grid, block, lds, s, p, a, y, out, n_ext);
  else
    hipLaunchKernelGGL((pipeline_kernel<IN, OUT, false, false>), grid, block, lds, s, p, a, y, out, n_ext);
  return hipGetLastError();
}

// Plans whose tiles have few chunks: no waits, every chunk tested in one pass.
bool select_small(const PlanDev& p) { return p.n_chunks <= kDirectChunks + 1; }

// The first launch of the pipeline step of a plan with conditioning tokens:
// the extent parts and the blend (extent_blend_kernel).  Sets the position
// fields of `a` for the selection launch that follows.
template <int IN, int OUT>
hipError_t launch_extent_blend(const PlanDev& p, ExtractArgs& a, const void* tile_out,
                               const int32_t* blend_cond_row, const int32_t* blend_cond_k, void* out,
                               const DeviceShape& ds, hipStream_t s) {
  const int n_bcond = blend_cond_blocks(p);
  const dim3 grid((unsigned)(a.n_ext + n_bcond + blend_gen_blocks(p))), block(kBlock);
  const size_t lds = capped_lds(ds, blend_cond_lds(p), kBlendWgsPerCu);
  const u32x4* y = reinterpret_cast<const u32x4*>(tile_out);
  const int combo = (p.B == 1 ? 0 : 4) + (p.ax[0].n > 1 ? 2 : 0) + (p.world > 1 ? 1 : 0);
#define TDP_EB_LAUNCH(NP, F2, R)                                                                                \
  hipLaunchKernelGGL((extent_blend_kernel<NP, IN, OUT, F2, R>), grid, block, lds, s, p, a, y, blend_cond_row, \
                     blend_cond_k, out, n_bcond)
  switch (combo) {
    case 0: TDP_EB_LAUNCH(3, false, false); break;
    case 1: TDP_EB_LAUNCH(3, false, true); break;
    case 2: TDP_EB_LAUNCH(3, true, false); break;
    case 3: TDP_EB_LAUNCH(3, true, true); break;
    case 4: TDP_EB_LAUNCH(6, false, false); break;
    case 5: TDP_EB_LAUNCH(6, false, true); break;
    case 6: TDP_EB_LAUNCH(6, true, false); break;
    default: TDP_EB_LAUNCH(6, true, true); break;
  }
#undef TDP_EB_LAUNCH
  a.pos_one_pass = 0;
  a.pos_parts = p.pos_parts;
  a.n_pos = p.T_local * p.B * 3 * a.pos_parts;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// streaming blend: one tile at a time into an fp32 accumulator
// ---------------------------------------------------------------------------

constexpr int kStreamRows = 1;  // generated rows per lane in one streaming workgroup (1 measured best: more workgroups per tile launch)

// Generated rows of tile t, batch element b, one lane per 16-byte vector.
// The weight is (wF * wH) * wW, as in blend_kernel.  A voxel's first
// covering tile (smallest index: on every axis, not inside the previous
// tile's overlap) writes fmaf(w, y, +0) without reading the accumulator;
// later tiles add with fmaf.  Run for t = 0, 1, ..., T-1 in order, this is
// blend_kernel's fp32 sum, term by term.  Lanes take their elements as
// blend_kernel does for an fp32 output (LaneIO), so that each accumulator
// load and store instruction covers a contiguous span.
template <int IN>
__device__ void stream_gen_rows(const PlanDev& p, const TileBox& tb, int i, int j, int k, int b, int blk,
                                const u32x4* __restrict__ tile_out, float* __restrict__ acc) {
  constexpr int E = InVec<IN>::E;
  const int V = p.vin;
  const int rpp = p.rpp;
  const int lr = (int)fastdiv(threadIdx.x, p.by_vin), vv = threadIdx.x - lr * V;
  if (lr >= rpp) return;
#pragma unroll
  for (int u = 0; u < kStreamRows; ++u) {
    const int r = (blk * kStreamRows + u) * rpp + lr;
    if (r >= tb.s.gen) return;
    const int line = (int)div_by_size(p.ax[2], (uint32_t)r, tb.sw);
    const int lw = r - line * tb.sw;
    const int lf = (int)div_by_size(p.ax[1], (uint32_t)line, tb.sh);
    const int lh = line - lf * tb.sh;
    const float wa = ramp_weight(p.ax[0], i, lf, tb.sf) * ramp_weight(p.ax[1], j, lh, tb.sh) *
                     ramp_weight(p.ax[2], k, lw, tb.sw);
    const bool first = !(i > 0 && lf < p.ax[0].o) && !(j > 0 && lh < p.ax[1].o) && !(k > 0 && lw < p.ax[2].o);
    using IO = LaneIO<IN, TDP_F32>;
    const u32x4 yv = IO::load(tile_out, ((int64_t)b * tb.s.cap + r) * V + vv, vv, V);
    const int64_t voxel = (int64_t)b * p.rows + ((int64_t)(tb.f0 + lf) * p.H + (tb.h0 + lh)) * p.W + tb.w0 + lw;
    float x[E], old[E];
    InVec<IN>::unpack(yv, x);
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      const f32x4 o = first ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : *IO::quad(acc, voxel, vv, V, q);
      old[4 * q] = o.x;
      old[4 * q + 1] = o.y;
      old[4 * q + 2] = o.z;
      old[4 * q + 3] = o.w;
    }
#pragma unroll
    for (int q = 0; q < E / 4; ++q)
      *IO::quad(acc, voxel, vv, V, q) =
          f32x4{fmaf(wa, x[4 * q], old[4 * q]), fmaf(wa, x[4 * q + 1], old[4 * q + 1]),
                fmaf(wa, x[4 * q + 2], old[4 * q + 2]), fmaf(wa, x[4 * q + 3], old[4 * q + 3])};
  }
}

// Conditioning tokens [c0, c0 + kCondRowsPerBlock) of batch element b for
// tile t: (1/k) * y added in tile order, the first keeping tile
// overwriting.  Tokens no tile keeps (blend_kernel's sum of nothing) are
// set to 0 when t == 0.
template <int IN>
__device__ void stream_cond_rows(const PlanDev& p, int t, int b, int c0, const u32x4* __restrict__ tile_out,
                                 const int32_t* __restrict__ cond_row, const int32_t* __restrict__ cond_k,
                                 float* __restrict__ acc, int cap_t) {
  constexpr int E = InVec<IN>::E;
  const int V = p.vin;
  const int rpp = p.rpp;
  const int lr = (int)fastdiv(threadIdx.x, p.by_vin), vv = threadIdx.x - lr * V;
  if (lr >= rpp) return;
  const int nrows = min(kCondRowsPerBlock, p.Nc - c0);
  for (int jj = lr; jj < nrows; jj += rpp) {
    const int c = c0 + jj;
    const int row = cond_row[(int64_t)t * p.Nc + c];
    const int kc = cond_k[c];
    bool first = true, any = false;  // any: some tile holds a row blend_kernel sums
    for (int u = 0; u < p.T; ++u) {
      const int ru = cond_row[(int64_t)u * p.Nc + c];
      if (ru >= 0) {
        int iu, ju, ku;
        tile_grid(p, u, iu, ju, ku);
        if (ru < tile_slot_whole(p, iu, ju, ku).cap) {
          any = true;
          if (u < t) first = false;
        }
      }
    }
    f32x4* a4 = reinterpret_cast<f32x4*>(acc + (((int64_t)b * p.rows + p.N + c) * V + vv) * E);
    if (row < 0 || row >= cap_t || kc <= 0) {
      if (t == 0 && (!any || kc <= 0))
#pragma unroll
        for (int q = 0; q < E / 4; ++q) a4[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      continue;
    }
    const float inv = 1.0f / (float)kc;
    const u32x4 yv = ld_nt(tile_out + ((int64_t)b * cap_t + row) * V + vv);
    float x[E];
    InVec<IN>::unpack(yv, x);
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      const f32x4 o = first ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : a4[q];
      a4[q] = f32x4{fmaf(inv, x[4 * q], o.x), fmaf(inv, x[4 * q + 1], o.y), fmaf(inv, x[4 * q + 2], o.z),
                    fmaf(inv, x[4 * q + 3], o.w)};
    }
  }
}

// One launch per tile: [0, n_gen) generated-row workgroups (B of them per
// row chunk), then conditioning workgroups per (batch element, chunk).
template <int IN>
__global__ __launch_bounds__(kBlock) void blend_tile_kernel(const PlanDev p, int t, const u32x4* __restrict__ tile_out,
                                                            const int32_t* __restrict__ cond_row,
                                                            const int32_t* __restrict__ cond_k,
                                                            float* __restrict__ acc, int gen_per_b, int n_gen) {
  int i, j, k;
  tile_grid(p, t, i, j, k);
  const TileBox tb = tile_box<false>(p, t);
  const int bid = blockIdx.x;
  if (bid < n_gen) {
    const int b = bid / gen_per_b;
    stream_gen_rows<IN>(p, tb, i, j, k, b, bid - b * gen_per_b, tile_out, acc);
    return;
  }
  const int per_b = (p.Nc + kCondRowsPerBlock - 1) / kCondRowsPerBlock;
  const int cid = bid - n_gen;
  const int b = cid / per_b;
  stream_cond_rows<IN>(p, t, b, (cid - b * per_b) * kCondRowsPerBlock, tile_out, cond_row, cond_k, acc, tb.s.cap);
}

// acc (fp32) -> out (OUT), four values per thread.
template <int OUT>
__global__ __launch_bounds__(kBlock) void blend_finish_kernel(const f32x4* __restrict__ acc, void* __restrict__ out,
                                                              int64_t n4) {
  const int64_t q = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (q >= n4) return;
  const f32x4 v = ld_nt(acc + q);
  const float a[4] = {v.x, v.y, v.z, v.w};
  store_out<OUT, 4>(out, q * 4, a);
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

// Reads of an unpublished look-back flag before a selection wave counts the
// chunk itself (process-wide; tdp_set_lookback_polls).
std::atomic<int> g_lookback_polls{kLookbackPolls};

// Enqueue extract: the gather (with conditioning tokens, the extent parts
// too, into `ws`), then with conditioning tokens the selection launch.
// Arguments are valid.
ExtractArgs extract_args(const PlanDev& p, const void* latent, const float* pos, void* tile_lat, float* tile_pos,
                         int32_t* tile_index, int32_t* tile_count, int32_t* cond_row, int32_t* cond_k, char* ws) {
  ExtractArgs a;
  a.latent = reinterpret_cast<const u32x4*>(latent);
  a.pos = reinterpret_cast<const f32x2*>(pos);
  a.tile_lat = reinterpret_cast<u32x4*>(tile_lat);
  a.tile_pos = reinterpret_cast<f32x2*>(tile_pos);
  a.tile_index = tile_index;
  a.tile_count = tile_count;
  a.cond_row = cond_row;
  a.cond_k = cond_k;
  a.ws = p.Nc > 0 ? ws : nullptr;
  a.n_ext = p.Nc > 0 ? p.T * p.ext_parts : 0;
  a.n_sel = p.Nc > 0 ? p.T * p.n_chunks : 0;
  a.lookback_polls = g_lookback_polls.load(std::memory_order_relaxed);
  a.copy_latent = 1;
  a.pos_one_pass = 0;
  a.pos_parts = p.pos_parts;
  a.n_pos = 0;
  return a;
}

// The extent launch (Nc > 0): the extent parts of every tile.  Sets the
// position fields of `a` for the selection launch, whose workgroups are
// a.n_sel selection, a.n_pos positions (copies: the shift is known) and the
// latent rows.
int launch_extent(const PlanDev& p, ExtractArgs& a, hipStream_t s, const char* who) {
  const dim3 egrid((unsigned)a.n_ext), block(kBlock);
  if (p.B == 1)
    hipLaunchKernelGGL((extent_kernel<3>), egrid, block, 0, s, p, a);
  else
    hipLaunchKernelGGL((extent_kernel<6>), egrid, block, 0, s, p, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TDP_EHIP, "%s: extent launch failed: %s", who, hipGetErrorString(e));
  a.pos_one_pass = 0;
  a.pos_parts = p.pos_parts;
  a.n_pos = p.T_local * p.B * 3 * a.pos_parts;
  return TDP_OK;
}

// The selection launch (Nc > 0, after the extents): a.n_sel selection,
// a.n_pos position and n_lat latent workgroups.  The dynamic LDS holds the
// tile's extent and caps the workgroups per CU: plans with few chunks per
// tile at kExtractWgsPerCu, plans with more (look-back chains, little work
// per workgroup) at kSelectWgsPerCuLarge.
int launch_select(const PlanDev& p, const ExtractArgs& a, int n_lat, const DeviceShape& ds, hipStream_t s,
                  const char* who) {
  const dim3 sgrid((unsigned)(a.n_sel + a.n_pos + n_lat)), block(kBlock);
  const bool small = select_small(p);
  const size_t lds = capped_lds(ds, (size_t)p.B * 3 * sizeof(float2), small ? kExtractWgsPerCu : kSelectWgsPerCuLarge);
  if (p.world > 1 && small)
    hipLaunchKernelGGL((select_kernel<true, true>), sgrid, block, lds, s, p, a);
  else if (p.world > 1)
    hipLaunchKernelGGL((select_kernel<true, false>), sgrid, block, lds, s, p, a);
  else if (small)
    hipLaunchKernelGGL((select_kernel<false, true>), sgrid, block, lds, s, p, a);
  else
    hipLaunchKernelGGL((select_kernel<false, false>), sgrid, block, lds, s, p, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TDP_EHIP, "%s: selection launch failed: %s", who, hipGetErrorString(e));
  return TDP_OK;
}

// Extract without conditioning tokens: more than eight latent workgroups
// per compute unit and the latent copy sets the length (3 per CU, positions
// in one pass); otherwise the position chains do (2 per CU, parts of at most
// 1024 rows), unless one part holds a whole plane: then one pass, with no
// second round of loads (LTX-like latent 4.90 -> 4.72 us per pipeline step,
// the 3x8x8 one 3.90 -> 3.64; full-res, 3 parts a plane, stays at two
// passes: 8.9 against 9.25 us).  Sets the position fields of `a`; returns
// whether the plan is latent-bound.
bool plain_setup(const PlanDev& p, ExtractArgs& a, const DeviceShape& ds, int n_lat) {
  const bool latent_bound = n_lat > 8 * (ds.cus > 0 ? ds.cus : 256);
  const bool one_pass = latent_bound || p.pos_parts_one == 1;
  a.pos_one_pass = one_pass ? 1 : 0;
  a.pos_parts = one_pass ? p.pos_parts_one : p.pos_parts;
  a.n_pos = p.T_local * p.B * 3 * a.pos_parts;
  return latent_bound;
}

int launch_extract(const PlanDev& p, const void* latent, const float* pos, void* tile_lat, float* tile_pos,
                   int32_t* tile_index, int32_t* tile_count, int32_t* cond_row, int32_t* cond_k, char* ws,
                   hipStream_t s, const char* who) {
  ExtractArgs a = extract_args(p, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k, ws);
  const DeviceShape ds = device_shape();
  const int n_lat = (p.lat_units + kWaves - 1) / kWaves;
  const dim3 block(kBlock);
  if (p.Nc > 0) {
    const int st = launch_extent(p, a, s, who);
    return st != TDP_OK ? st : launch_select(p, a, n_lat, ds, s, who);
  }
  const bool latent_bound = plain_setup(p, a, ds, n_lat);
  const dim3 grid(a.n_pos + n_lat);
  if (grid.x == 0) return TDP_OK;  // a rank without tiles: nothing to write
  const size_t lds = capped_lds(ds, 0, latent_bound ? kExtractWgsPerCu : kExtractWgsPerCuChain);
  if (p.world > 1)
    hipLaunchKernelGGL(extract_kernel<true>, grid, block, lds, s, p, a);
  else
    hipLaunchKernelGGL(extract_kernel<false>, grid, block, lds, s, p, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TDP_EHIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
  return TDP_OK;
}

// tdp_extract_positions: what tdp_extract writes except the latent rows.
// Nc > 0: the extent launch, then the selection launch without its latent
// blocks (selection workgroups copy only positions); Nc = 0: the position
// workgroups of the plain extract, in parts of at most 1024 rows.
int launch_positions(const PlanDev& p, const float* pos, float* tile_pos, int32_t* tile_index, int32_t* tile_count,
                     int32_t* cond_row, int32_t* cond_k, char* ws, hipStream_t s, const char* who) {
  ExtractArgs a = extract_args(p, nullptr, pos, nullptr, tile_pos, tile_index, tile_count, cond_row, cond_k, ws);
  a.copy_latent = 0;
  const DeviceShape ds = device_shape();
  const dim3 block(kBlock);
  if (p.Nc > 0) {  // no latent workgroups
    const int st = launch_extent(p, a, s, who);
    return st != TDP_OK ? st : launch_select(p, a, 0, ds, s, who);
  }
  a.n_pos = p.T_local * p.B * 3 * a.pos_parts;
  const dim3 grid((unsigned)a.n_pos);
  if (grid.x == 0) return TDP_OK;  // a rank without tiles: nothing to write
  const size_t lds = capped_lds(ds, 0, kExtractWgsPerCuChain);
  if (p.world > 1)
    hipLaunchKernelGGL(extract_kernel<true>, grid, block, lds, s, p, a);
  else
    hipLaunchKernelGGL(extract_kernel<false>, grid, block, lds, s, p, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TDP_EHIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
  return TDP_OK;
}

// tdp_extract_latent: the latent rows of every held tile.
int launch_gather(const PlanDev& p, const void* latent, const int32_t* cond_row, void* tile_lat, hipStream_t s,
                  const char* who) {
  ExtractArgs a = extract_args(p, latent, nullptr, tile_lat, nullptr, nullptr, nullptr, const_cast<int32_t*>(cond_row),
                               nullptr, nullptr);
  const int n_cg = gather_cond_blocks(p);
  const dim3 grid((unsigned)(n_cg + (p.lat_units + kWaves - 1) / kWaves)), block(kBlock);
  if (grid.x == 0) return TDP_OK;  // a rank without tiles: nothing to write
  const size_t lds = capped_lds(device_shape(), 0, kExtractWgsPerCu);
  if (p.world > 1)
    hipLaunchKernelGGL(gather_kernel<true>, grid, block, lds, s, p, a, n_cg);
  else
    hipLaunchKernelGGL(gather_kernel<false>, grid, block, lds, s, p, a, n_cg);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TDP_EHIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
  return TDP_OK;
}

// A HIP launch counts its work-items in 32 bits.  Every device call of a
// plan refuses, before its first launch, a plan whose workgroups of every
// kind its launches use (extent and selection parts, position parts, latent
// units, gather chunks, blend conditioning and generated units, zero-fill
// lines) would add up to more work-items than that: the sum bounds each
// single launch, so no launch of the call can fail on its size after an
// earlier one has run.
constexpr int64_t kMaxLaunchItems = 0xffffffffLL;
int check_launch_size(const PlanDev& p, const char* who) {
  const int64_t parts = p.pos_parts > p.pos_parts_one ? p.pos_parts : p.pos_parts_one;
  const int64_t sel = p.Nc > 0 ? (int64_t)p.T * (p.ext_parts + p.n_chunks) : 0;
  const int64_t wgs = sel + (int64_t)p.T_local * p.B * 3 * parts + (p.lat_units + kWaves - 1) / kWaves +
                      gather_cond_blocks(p) + blend_cond_blocks(p) + blend_gen_blocks(p);
  if (wgs * kBlock > kMaxLaunchItems)
    return fail(TDP_ESHAPE,
                "%s: the plan's launches need up to %lld work-items, more than the %lld of one HIP launch "
                "(split the batch or the latent over several plans)",
                who, (long long)(wgs * kBlock), (long long)kMaxLaunchItems);
  return TDP_OK;
}

// Work-items of the streaming blend's finish pass: one thread per four
// accumulator floats, in whole workgroups.
int64_t finish_items(const PlanDev& p) {
  const int64_t n4 = (int64_t)p.B * p.rows * p.C / 4;
  return (n4 + kBlock - 1) / kBlock * kBlock;
}

// Checks tdp_extract and tdp_extract_noalloc share (the workspace aside).
int check_extract(const tdp_plan* plan, const void* latent, const float* pos, const void* tile_lat,
                  const float* tile_pos, const int32_t* tile_index, const int32_t* tile_count, const int32_t* cond_row,
                  const int32_t* cond_k, const char* who) {
  if (!plan) return fail(TDP_EINVAL, "%s: null plan", who);
  if (!plan->guarded) return fail(TDP_EGUARD, "%s: plan was built with TDP_UNGUARDED", who);
  const PlanDev& p = plan->dev;
  if (!latent || !pos) return fail(TDP_EINVAL, "%s: null device pointer", who);
  if (p.T_local > 0 && (!tile_lat || !tile_pos || !tile_index || !tile_count))
    return fail(TDP_EINVAL, "%s: null device pointer", who);
  if (p.Nc > 0 && (!cond_row || !cond_k))
    return fail(TDP_EINVAL, "%s: cond_row and cond_k are required when num_cond > 0", who);
  if (!aligned(latent, 16) || !aligned(tile_lat, 16))
    return fail(TDP_EINVAL, "%s: latent and tile_lat must be 16-byte aligned", who);
  if (!aligned(pos, 8) || !aligned(tile_pos, 8) || !aligned(tile_index, 4) || !aligned(tile_count, 4) ||
      !aligned(cond_row, 4) || !aligned(cond_k, 4))
    return fail(TDP_EINVAL, "%s: pos/tile_pos need 8-byte and int buffers 4-byte alignment", who);
  return check_launch_size(p, who);
}

// Checks of tdp_extract_positions' arguments (the workspace aside).
int check_positions(const tdp_plan* plan, const float* pos, const float* tile_pos, const int32_t* tile_index,
                    const int32_t* tile_count, const int32_t* cond_row, const int32_t* cond_k, const char* who) {
  if (!plan) return fail(TDP_EINVAL, "%s: null plan", who);
  if (!plan->guarded) return fail(TDP_EGUARD, "%s: plan was built with TDP_UNGUARDED", who);
  const PlanDev& p = plan->dev;
  if (!pos || (p.T_local > 0 && (!tile_pos || !tile_index || !tile_count)))
    return fail(TDP_EINVAL, "%s: null device pointer", who);
  if (p.Nc > 0 && (!cond_row || !cond_k))
    return fail(TDP_EINVAL, "%s: cond_row and cond_k are required when num_cond > 0", who);
  if (!aligned(pos, 8) || !aligned(tile_pos, 8) || !aligned(tile_index, 4) || !aligned(tile_count, 4) ||
      !aligned(cond_row, 4) || !aligned(cond_k, 4))
    return fail(TDP_EINVAL, "%s: pos/tile_pos need 8-byte and int buffers 4-byte alignment", who);
  return check_launch_size(p, who);
}

// Checks of tdp_extract_latent's arguments (shared with
// tdp_pipeline_latent_step).
int check_gather(const tdp_plan* plan, const void* latent, const int32_t* cond_row, const void* tile_lat,
                 const char* who) {
  if (!plan) return fail(TDP_EINVAL, "%s: null plan", who);
  if (!plan->guarded) return fail(TDP_EGUARD, "%s: plan was built with TDP_UNGUARDED", who);
  const PlanDev& p = plan->dev;
  if (!latent || (p.T_local > 0 && !tile_lat)) return fail(TDP_EINVAL, "%s: null device pointer", who);
  if (p.Nc > 0 && !cond_row) return fail(TDP_EINVAL, "%s: cond_row is required when num_cond > 0", who);
  if (!aligned(latent, 16) || !aligned(tile_lat, 16))
    return fail(TDP_EINVAL, "%s: latent and tile_lat must be 16-byte aligned", who);
  if (!aligned(cond_row, 4)) return fail(TDP_EINVAL, "%s: misaligned cond_row", who);
  return check_launch_size(p, who);
}

// Checks of tdp_blend's arguments (shared with tdp_pipeline_step).
int check_blend(const tdp_plan* plan, const void* tile_out, const int32_t* cond_row, const int32_t* cond_k,
                const void* out, const char* who) {
  if (!plan) return fail(TDP_EINVAL, "%s: null plan", who);
  if (!plan->guarded) return fail(TDP_EGUARD, "%s: plan was built with TDP_UNGUARDED", who);
  const PlanDev& p = plan->dev;
  if (!out || (!tile_out && p.T_local > 0)) return fail(TDP_EINVAL, "%s: null device pointer", who);
  if (p.Nc > 0 && (!cond_row || !cond_k))
    return fail(TDP_EINVAL, "%s: cond_row and cond_k are required when num_cond > 0", who);
  if (!aligned(tile_out, 16) || !aligned(out, 16))
    return fail(TDP_EINVAL, "%s: tile_out and out must be 16-byte aligned", who);
  if (!aligned(cond_row, 4) || !aligned(cond_k, 4)) return fail(TDP_EINVAL, "%s: misaligned cond_row or cond_k", who);
  return check_launch_size(p, who);
}

// The blend of a checked plan, by dtypes.
hipError_t blend_dispatch(const PlanDev& p, const void* tile_out, const int32_t* cond_row, const int32_t* cond_k,
                          void* out, hipStream_t s) {
  if (p.in_dtype == TDP_BF16 && p.out_dtype == TDP_BF16)
    return launch_blend<TDP_BF16, TDP_BF16>(p, tile_out, cond_row, cond_k, out, s);
  if (p.in_dtype == TDP_BF16 && p.out_dtype == TDP_F32)
    return launch_blend<TDP_BF16, TDP_F32>(p, tile_out, cond_row, cond_k, out, s);
  if (p.in_dtype == TDP_F32 && p.out_dtype == TDP_F32)
    return launch_blend<TDP_F32, TDP_F32>(p, tile_out, cond_row, cond_k, out, s);
  return launch_blend<TDP_F32, TDP_BF16>(p, tile_out, cond_row, cond_k, out, s);
}

// Byte ranges [a, a + na) and [b, b + nb) share a byte (null or empty: no).
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

}  // namespace
}  // namespace tdp

using namespace tdp;

// Workspace of tdp_extract_noalloc: one copy on every GPU the library runs
// on, kept until the process ends.  Host code never passes this name to a
// kernel (on the host it only stands for the symbol); it passes the device
// address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) char scratch[TDP_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;
std::atomic<char*> g_scratch[kScratchDevices];  // device address per device; null until looked up

// Address of `scratch` on the current device, looked up on the first call
// with that device current; null (with the error recorded) on failure.
char* scratch_on_current_device(const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(TDP_EHIP, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kScratchDevices) {
    fail(TDP_EHIP, "%s: device %d is beyond the %d the static workspace serves", who, dev, kScratchDevices);
    return nullptr;
  }
  char* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    fail(TDP_EHIP, "%s: no device address for the static workspace: %s", who, hipGetErrorString(e));
    return nullptr;
  }
  g_scratch[dev].store(ptr, std::memory_order_release);  // racing first calls store the same address
  return ptr;
}

}  // namespace

extern "C" {

int tdp_extract(const tdp_plan* plan, const void* latent, const float* pos, void* tile_lat, float* tile_pos,
                int32_t* tile_index, int32_t* tile_count, int32_t* cond_row, int32_t* cond_k, void* workspace,
                void* stream) {
  const int st = check_extract(plan, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k,
                               "tdp_extract");
  if (st != TDP_OK) return st;
  const PlanDev& p = plan->dev;
  if (ws_layout(p).bytes > 0 && !workspace)
    return fail(TDP_EINVAL, "tdp_extract: workspace of %lld bytes is required (tdp_plan_sizes)",
                (long long)ws_layout(p).bytes);
  if (!aligned(workspace, 16)) return fail(TDP_EINVAL, "tdp_extract: workspace must be 16-byte aligned");
  return launch_extract(p, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k,
                        static_cast<char*>(workspace), reinterpret_cast<hipStream_t>(stream), "tdp_extract");
}

int tdp_set_lookback_polls(int32_t polls) {
  if (polls < 0) return fail(TDP_EINVAL, "tdp_set_lookback_polls: polls must be >= 0 (got %d)", polls);
  g_lookback_polls.store(polls, std::memory_order_relaxed);
  return TDP_OK;
}

int tdp_extract_noalloc(const tdp_plan* plan, const void* latent, const float* pos, void* tile_lat,
                        float* tile_pos, int32_t* tile_index, int32_t* tile_count, int32_t* cond_row,
                        int32_t* cond_k, void* stream) {
  const int st = check_extract(plan, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k,
                               "tdp_extract_noalloc");
  if (st != TDP_OK) return st;
  const PlanDev& p = plan->dev;
  const int64_t need = ws_layout(p).bytes;
  if (need > (int64_t)TDP_STATIC_SCRATCH_BYTES)
    return fail(TDP_EINVAL, "tdp_extract_noalloc: the plan needs %lld bytes of workspace, beyond the static %d",
                (long long)need, (int)TDP_STATIC_SCRATCH_BYTES);
  char* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device("tdp_extract_noalloc");
    if (!ws) return TDP_EHIP;
  }
  return launch_extract(p, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k, ws,
                        reinterpret_cast<hipStream_t>(stream), "tdp_extract_noalloc");
}

int tdp_blend_tile(const tdp_plan* plan, int32_t t, const void* tile_out, const int32_t* cond_row,
                   const int32_t* cond_k, float* acc, void* stream) {
  if (!plan) return fail(TDP_EINVAL, "tdp_blend_tile: null plan");
  if (!plan->guarded) return fail(TDP_EGUARD, "tdp_blend_tile: plan was built with TDP_UNGUARDED");
  const PlanDev& p = plan->dev;
  if (p.world > 1) return fail(TDP_EINVAL, "tdp_blend_tile: rank plans take tdp_blend (streaming is for whole plans)");
  if (t < 0 || t >= p.T) return fail(TDP_EINVAL, "tdp_blend_tile: tile index %d out of range [0, %d)", t, p.T);
  if (!tile_out || !acc) return fail(TDP_EINVAL, "tdp_blend_tile: null device pointer");
  if (p.Nc > 0 && (!cond_row || !cond_k))
    return fail(TDP_EINVAL, "tdp_blend_tile: cond_row and cond_k are required when num_cond > 0");
  if (!aligned(tile_out, 16) || !aligned(acc, 16) || !aligned(cond_row, 4) || !aligned(cond_k, 4))
    return fail(TDP_EINVAL, "tdp_blend_tile: tile_out and acc need 16-byte, cond_row and cond_k 4-byte alignment");
  int i, j, k;
  tile_grid(p, t, i, j, k);
  const TileSlot slot = tile_slot_whole(p, i, j, k);
  const int rows_per_block = (kBlock / p.vin) * kStreamRows;
  const int gen_per_b = (slot.gen + rows_per_block - 1) / rows_per_block;
  const int n_gen = p.B * gen_per_b;
  const int n_cond = p.Nc > 0 ? p.B * ((p.Nc + kCondRowsPerBlock - 1) / kCondRowsPerBlock) : 0;
  if (((int64_t)n_gen + n_cond) * kBlock > kMaxLaunchItems || finish_items(p) > kMaxLaunchItems)
    return fail(TDP_ESHAPE, "tdp_blend_tile: the tile's launch or the finish pass needs more work-items than the "
                            "%lld of one HIP launch (split the batch or the latent over several plans)",
                (long long)kMaxLaunchItems);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const u32x4* y = reinterpret_cast<const u32x4*>(tile_out);
  if (p.in_dtype == TDP_BF16)
    hipLaunchKernelGGL(blend_tile_kernel<TDP_BF16>, dim3(n_gen + n_cond), dim3(kBlock), 0, s, p, (int)t, y, cond_row,
                       cond_k, acc, gen_per_b, n_gen);
  else
    hipLaunchKernelGGL(blend_tile_kernel<TDP_F32>, dim3(n_gen + n_cond), dim3(kBlock), 0, s, p, (int)t, y, cond_row,
                       cond_k, acc, gen_per_b, n_gen);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TDP_EHIP, "tdp_blend_tile: kernel launch failed: %s", hipGetErrorString(e));
  return TDP_OK;
}

int tdp_blend_finish(const tdp_plan* plan, const float* acc, void* out, void* stream) {
  if (!plan) return fail(TDP_EINVAL, "tdp_blend_finish: null plan");
  const PlanDev& p = plan->dev;
  if (p.world > 1) return fail(TDP_EINVAL, "tdp_blend_finish: rank plans take tdp_blend (streaming is for whole plans)");
  if (!acc || !out) return fail(TDP_EINVAL, "tdp_blend_finish: null device pointer");
  if (!aligned(acc, 16) || !aligned(out, 16)) return fail(TDP_EINVAL, "tdp_blend_finish: misaligned pointer");
  if (p.out_dtype == TDP_F32 && static_cast<const void*>(acc) == out) return TDP_OK;
  const int64_t n4 = (int64_t)p.B * p.rows * p.C / 4;  // C * 4 bytes is a multiple of 16
  const int64_t blocks = (n4 + kBlock - 1) / kBlock;
  if (finish_items(p) > kMaxLaunchItems)
    return fail(TDP_ESHAPE, "tdp_blend_finish: %lld work-items, more than the %lld of one HIP launch",
                (long long)finish_items(p), (long long)kMaxLaunchItems);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const f32x4* a4 = reinterpret_cast<const f32x4*>(acc);
  if (p.out_dtype == TDP_BF16)
    hipLaunchKernelGGL(blend_finish_kernel<TDP_BF16>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a4, out, n4);
  else
    hipLaunchKernelGGL(blend_finish_kernel<TDP_F32>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a4, out, n4);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TDP_EHIP, "tdp_blend_finish: kernel launch failed: %s", hipGetErrorString(e));
  return TDP_OK;
}

int tdp_blend(const tdp_plan* plan, const void* tile_out, const int32_t* cond_row, const int32_t* cond_k, void* out,
              void* stream) {
  const int st = check_blend(plan, tile_out, cond_row, cond_k, out, "tdp_blend");
  if (st != TDP_OK) return st;
  const hipError_t e = blend_dispatch(plan->dev, tile_out, cond_row, cond_k, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TDP_EHIP, "tdp_blend: kernel launch failed: %s", hipGetErrorString(e));
  return TDP_OK;
}

int tdp_extract_positions(const tdp_plan* plan, const float* pos, float* tile_pos, int32_t* tile_index,
                          int32_t* tile_count, int32_t* cond_row, int32_t* cond_k, void* workspace, void* stream) {
  const char* who = "tdp_extract_positions";
  const int st = check_positions(plan, pos, tile_pos, tile_index, tile_count, cond_row, cond_k, who);
  if (st != TDP_OK) return st;
  const PlanDev& p = plan->dev;
  if (ws_layout(p).bytes > 0 && !workspace)
    return fail(TDP_EINVAL, "%s: workspace of %lld bytes is required (tdp_plan_sizes)", who,
                (long long)ws_layout(p).bytes);
  if (!aligned(workspace, 16)) return fail(TDP_EINVAL, "%s: workspace must be 16-byte aligned", who);
  return launch_positions(p, pos, tile_pos, tile_index, tile_count, cond_row, cond_k, static_cast<char*>(workspace),
                          reinterpret_cast<hipStream_t>(stream), who);
}

int tdp_extract_latent(const tdp_plan* plan, const void* latent, const int32_t* cond_row, void* tile_lat,
                       void* stream) {
  const char* who = "tdp_extract_latent";
  const int st = check_gather(plan, latent, cond_row, tile_lat, who);
  if (st != TDP_OK) return st;
  return launch_gather(plan->dev, latent, cond_row, tile_lat, reinterpret_cast<hipStream_t>(stream), who);
}

int tdp_pipeline_latent_step(const tdp_plan* plan, const void* latent, const int32_t* cond_row, void* tile_lat,
                             const void* tile_out, const int32_t* blend_cond_row, const int32_t* blend_cond_k,
                             void* out, void* stream) {
  const char* who = "tdp_pipeline_latent_step";
  int st = check_gather(plan, latent, cond_row, tile_lat, who);
  if (st != TDP_OK) return st;
  st = check_blend(plan, tile_out, blend_cond_row, blend_cond_k, out, who);
  if (st != TDP_OK) return st;
  const PlanDev& p = plan->dev;
  // the halves may run at the same time: tile_lat is written by the gather
  // and must be none of the blend's buffers, and out none of the gather's
  tdp_sizes z;
  tdp_plan_sizes(plan, &z);
  const int64_t ein = dtype_bytes(p.in_dtype), eout = dtype_bytes(p.out_dtype);
  const int64_t lat_bytes = z.tile_lat_elems * ein, out_bytes = z.out_elems * eout;
  const struct { const void* ptr; int64_t bytes; } bl[] = {
      {tile_out, lat_bytes}, {blend_cond_row, z.cond_row_ints * 4}, {blend_cond_k, z.cond_k_ints * 4}, {out, out_bytes}},
    gr[] = {{latent, (int64_t)p.B * p.rows * p.C * ein}, {cond_row, z.cond_row_ints * 4}};
  for (const auto& b : bl)
    if (overlap(tile_lat, lat_bytes, b.ptr, b.bytes))
      return fail(TDP_EINVAL, "%s: the blend reads or writes tile_lat, which the gather writes", who);
  for (const auto& g : gr)
    if (overlap(g.ptr, g.bytes, out, out_bytes))
      return fail(TDP_EINVAL, "%s: the blend writes a buffer the gather reads", who);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const ExtractArgs a = extract_args(p, latent, nullptr, tile_lat, nullptr, nullptr, nullptr,
                                     const_cast<int32_t*>(cond_row), nullptr, nullptr);
  const DeviceShape ds = device_shape();
  hipError_t e;
  if (p.in_dtype == TDP_BF16 && p.out_dtype == TDP_BF16)
    e = launch_pipeline_latent<TDP_BF16, TDP_BF16>(p, a, tile_out, blend_cond_row, blend_cond_k, out, ds, s);
  else if (p.in_dtype == TDP_BF16 && p.out_dtype == TDP_F32)
    e = launch_pipeline_latent<TDP_BF16, TDP_F32>(p, a, tile_out, blend_cond_row, blend_cond_k, out, ds, s);
  else if (p.in_dtype == TDP_F32 && p.out_dtype == TDP_F32)
    e = launch_pipeline_latent<TDP_F32, TDP_F32>(p, a, tile_out, blend_cond_row, blend_cond_k, out, ds, s);
  else
    e = launch_pipeline_latent<TDP_F32, TDP_BF16>(p, a, tile_out, blend_cond_row, blend_cond_k, out, ds, s);
  if (e != hipSuccess) return fail(TDP_EHIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
  return TDP_OK;
}

int tdp_pipeline_step(const tdp_plan* plan, const void* latent, const float* pos, void* tile_lat, float* tile_pos,
                      int32_t* tile_index, int32_t* tile_count, int32_t* cond_row, int32_t* cond_k, void* workspace,
                      const void* tile_out, const int32_t* blend_cond_row, const int32_t* blend_cond_k, void* out,
                      void* stream) {
  const char* who = "tdp_pipeline_step";
  int st = check_extract(plan, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k, who);
  if (st != TDP_OK) return st;
  st = check_blend(plan, tile_out, blend_cond_row, blend_cond_k, out, who);
  if (st != TDP_OK) return st;
  const PlanDev& p = plan->dev;
  const int64_t ws_bytes = ws_layout(p).bytes;
  if (ws_bytes > 0 && !workspace)
    return fail(TDP_EINVAL, "%s: workspace of %lld bytes is required (tdp_plan_sizes)", who, (long long)ws_bytes);
  if (!aligned(workspace, 16)) return fail(TDP_EINVAL, "%s: workspace must be 16-byte aligned", who);
  // the blend's buffers must be none of the extract's: the two halves may
  // run at the same time
  tdp_sizes z;
  tdp_plan_sizes(plan, &z);
  const int64_t ein = dtype_bytes(p.in_dtype), eout = dtype_bytes(p.out_dtype);
  const int64_t rows = (int64_t)p.B * p.rows;
  const struct { const void* ptr; int64_t bytes; } ext_w[] = {
      {tile_lat, z.tile_lat_elems * ein}, {tile_pos, z.tile_pos_floats * 4}, {tile_index, z.tile_index_ints * 4},
      {tile_count, z.num_slots * 4},      {cond_row, z.cond_row_ints * 4},   {cond_k, z.cond_k_ints * 4},
      {workspace, ws_bytes}},
    ext_r[] = {{latent, rows * p.C * ein}, {pos, rows * 3 * 8}},
    bl_r[] = {{tile_out, z.tile_lat_elems * ein}, {blend_cond_row, z.cond_row_ints * 4}, {blend_cond_k, z.cond_k_ints * 4}};
  const int64_t out_bytes = z.out_elems * eout;
  for (const auto& w : ext_w) {
    for (const auto& r : bl_r)
      if (overlap(w.ptr, w.bytes, r.ptr, r.bytes))
        return fail(TDP_EINVAL, "%s: the blend reads a buffer the extract writes", who);
    if (overlap(w.ptr, w.bytes, out, out_bytes))
      return fail(TDP_EINVAL, "%s: the blend writes a buffer the extract writes", who);
  }
  for (const auto& r : ext_r)
    if (overlap(r.ptr, r.bytes, out, out_bytes))
      return fail(TDP_EINVAL, "%s: the blend writes a buffer the extract reads", who);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const DeviceShape ds = device_shape();
  if (p.Nc > 0) {  // extents and the blend, then the selection launch with the latent rows
    ExtractArgs ca = extract_args(p, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k,
                                  static_cast<char*>(workspace));
    hipError_t e;
    if (p.in_dtype == TDP_BF16 && p.out_dtype == TDP_BF16)
      e = launch_extent_blend<TDP_BF16, TDP_BF16>(p, ca, tile_out, blend_cond_row, blend_cond_k, out, ds, s);
    else if (p.in_dtype == TDP_BF16 && p.out_dtype == TDP_F32)
      e = launch_extent_blend<TDP_BF16, TDP_F32>(p, ca, tile_out, blend_cond_row, blend_cond_k, out, ds, s);
    else if (p.in_dtype == TDP_F32 && p.out_dtype == TDP_F32)
      e = launch_extent_blend<TDP_F32, TDP_F32>(p, ca, tile_out, blend_cond_row, blend_cond_k, out, ds, s);
    else
      e = launch_extent_blend<TDP_F32, TDP_BF16>(p, ca, tile_out, blend_cond_row, blend_cond_k, out, ds, s);
    if (e != hipSuccess) return fail(TDP_EHIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
    return launch_select(p, ca, (p.lat_units + kWaves - 1) / kWaves, ds, s, who);
  }
  ExtractArgs a = extract_args(p, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k, nullptr);
  const int n_lat = (p.lat_units + kWaves - 1) / kWaves;
  plain_setup(p, a, ds, n_lat);
  hipError_t e;
  if (p.in_dtype == TDP_BF16 && p.out_dtype == TDP_BF16)
    e = launch_pipeline<TDP_BF16, TDP_BF16>(p, a, n_lat, tile_out, out, ds, s);
  else if (p.in_dtype == TDP_BF16 && p.out_dtype == TDP_F32)
    e = launch_pipeline<TDP_BF16, TDP_F32>(p, a, n_lat, tile_out, out, ds, s);
  else if (p.in_dtype == TDP_F32 && p.out_dtype == TDP_F32)
    e = launch_pipeline<TDP_F32, TDP_F32>(p, a, n_lat, tile_out, out, ds, s);
  else
    e = launch_pipeline<TDP_F32, TDP_BF16>(p, a, n_lat, tile_out, out, ds, s);
  if (e != hipSuccess) return fail(TDP_EHIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
  return TDP_OK;
}

}  // extern "C"
