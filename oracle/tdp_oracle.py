"""Plain CPU oracle for tiled-data-parallel (TDP) latent tiling.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library under
``overlap_tiling_trapezoidal_amd`` never imports it, and this module imports
nothing from the library: the two share no code, tables or helpers.

Everything here is the slow, obvious definition of what the tiled hot path
computes, written from these pages:

* LTX-2 docs, "Tiled Data Parallelism (TDP)": sections "What it is",
  "Position normalization", "Shared negative (reference) positions", "API".
* mold issue #673 (porting TDP tiling to one GPU): sections "Why", "Scope",
  "A bug found while porting" (the window-sum table) and "Verification".

Floating point is fp64 unless a value must match a fixed-precision result bit
for bit (fp32 position shifts, bf16 rounding).  The pages leave several steps
open; each function names the reading it takes.  Every function is pinned
by ``tests/test_oracle_pins.py`` against values the pages print, closed forms
or invariants.  Two readings stay parity unpinned: which strides of
``split_by_count`` take the remainder when ``dim - overlap`` is not a multiple
of the tile count (the pages' table is met by more than one choice), and the
order of the tiles (the pages say round-robin but give no order; the blend
is pinned not to depend on it beyond summation rounding).
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

AXES = ("frames", "height", "width")


# --------------------------------------------------------------------------
# Interval split and guard
# --------------------------------------------------------------------------

def split_by_count(dim: int, num_tiles: int, overlap: int) -> list[tuple[int, int]]:
    """Split one latent axis of ``dim`` cells into ``num_tiles`` half-open intervals.

    Source: TDP docs, section "API" (tiling is given as tile *counts* per axis
    with an overlap in latent grid units) and mold #673, "A bug found while
    porting" (the window sums of the split for dim 21, overlap 8, 2/3/4 tiles;
    the guard derived from ``tile_size >= 2*overlap``).

    Reading (the pages never print the formula): the free length
    ``dim - overlap`` is cut into ``num_tiles`` strides with starts
    ``a_i = floor(i * (dim - overlap) / num_tiles)`` for i = 0..num_tiles, and
    tile i is ``[a_i, a_{i+1} + overlap)``; the last end is therefore ``dim``.
    Every adjacent pair shares exactly ``overlap`` cells.  This is the rule
    under which the printed window sums (1, up to 1.074, up to 1.161) come
    out; which strides receive the remainder of the division is not fixed by
    the pages (a floor spread is taken).
    """
    if num_tiles < 1:
        raise ValueError("num_tiles must be >= 1")
    if overlap < 0:
        raise ValueError("overlap must be >= 0")
    free = dim - overlap
    if free < num_tiles:
        raise ValueError("stride below one cell: dim - overlap must be >= num_tiles")
    starts = [(i * free) // num_tiles for i in range(num_tiles + 1)]
    return [(starts[i], starts[i + 1] + overlap) for i in range(num_tiles)]


def guard_holds(dim: int, num_tiles: int, overlap: int) -> bool:
    """The port's overlap guard ``overlap <= dim / (num_tiles + 1)``.

    Source: mold #673, "A bug found while porting": requiring a tile to be at
    least twice the overlap gives this bound.  Written in integers as
    ``overlap * (num_tiles + 1) <= dim``.  A single tile must have no overlap
    (an untiled axis asks for zero overlap).
    """
    if num_tiles == 1:
        return overlap == 0
    return overlap * (num_tiles + 1) <= dim


# --------------------------------------------------------------------------
# Trapezoidal windows
# --------------------------------------------------------------------------

def window_exact(intervals: list[tuple[int, int]], i: int, overlap: int) -> list[Fraction]:
    """1-D trapezoidal blend window of tile ``i`` as exact rationals.

    Source: TDP docs, "What it is" (overlaps are blended with trapezoidal
    masks that sum to 1 globally) and mold #673, "Why" (a separable
    trapezoidal window recombines the tiles) and the window-sum table of
    "A bug found while porting".

    Reading: over the first ``overlap`` cells of a tile that has a left
    neighbour the weight rises as (j+1)/(overlap+1), j = 0..overlap-1; over
    its last ``overlap`` cells, when it has a right neighbour, it falls
    mirror-wise; elsewhere it is 1.  Border tiles stay flat up to the latent
    edge.  A cell inside both ramps (possible only when the guard is off)
    takes the product of the two.
    """
    n = len(intervals)
    a, b = intervals[i]
    size = b - a
    out = []
    for j in range(size):
        w = Fraction(1)
        if i > 0 and j < overlap:
            w *= Fraction(j + 1, overlap + 1)
        if i < n - 1 and j >= size - overlap:
            w *= Fraction(size - j, overlap + 1)
        out.append(w)
    return out


def window_f64(intervals: list[tuple[int, int]], i: int, overlap: int) -> np.ndarray:
    """The same window in fp64."""
    return np.array([float(w) for w in window_exact(intervals, i, overlap)], dtype=np.float64)


def window_sums_exact(dim: int, num_tiles: int, overlap: int) -> list[Fraction]:
    """Sum over tiles of the 1-D windows at every cell of one axis, exactly.

    Source: mold #673, "A bug found while porting", the window-sum table.
    """
    ivs = split_by_count(dim, num_tiles, overlap)
    sums = [Fraction(0)] * dim
    for i, (a, _) in enumerate(ivs):
        for j, w in enumerate(window_exact(ivs, i, overlap)):
            sums[a + j] += w
    return sums


# --------------------------------------------------------------------------
# Tile enumeration
# --------------------------------------------------------------------------

def enumerate_tiles(shape, tiling):
    """All tiles of a (frames, height, width) latent, in row-major order.

    Source: mold #673, "Scope" (interval splitting, blend window, tile
    enumeration) and TDP docs, "What it is" (round-robin assignment).
    Reading: the tile list is the Cartesian product of the per-axis
    intervals with the width index fastest, so tile
    ``t = (i_f * n_h + i_h) * n_w + i_w``; on P ranks tile t runs on rank
    ``t mod P``.

    ``shape`` = (F, H, W); ``tiling`` = ((n_f, o_f), (n_h, o_h), (n_w, o_w)).
    """
    ivs = [split_by_count(d, n, o) for d, (n, o) in zip(shape, tiling)]
    tiles = []
    for t, grid in enumerate(itertools.product(*[range(len(v)) for v in ivs])):
        origin = tuple(ivs[d][grid[d]][0] for d in range(3))
        size = tuple(ivs[d][grid[d]][1] - ivs[d][grid[d]][0] for d in range(3))
        tiles.append({"index": t, "grid": grid, "origin": origin, "size": size})
    return tiles


def round_robin_rank(t: int, world: int) -> int:
    """Rank that runs tile t (TDP docs, "What it is": tiles go round-robin)."""
    return t % world


def tile_generated_tokens(tile, shape) -> np.ndarray:
    """Patchified indices of the tile's generated tokens, tile-local row-major.

    Source: TDP docs, "What it is" (the patchified (frames, height, width)
    latent is split into tiles).  Reading: tokens are numbered
    ``(f * H + h) * W + w`` and a tile lists its box in the same order.
    """
    _, H, W = shape
    (f0, h0, w0), (sf, sh, sw) = tile["origin"], tile["size"]
    idx = [(f * H + h) * W + w
           for f in range(f0, f0 + sf)
           for h in range(h0, h0 + sh)
           for w in range(w0, w0 + sw)]
    return np.array(idx, dtype=np.int64)


# --------------------------------------------------------------------------
# Extract: per-tile latent, normalized positions, kept conditioning tokens
# --------------------------------------------------------------------------

def extract(latent: np.ndarray, pos: np.ndarray, shape, tiling, num_cond: int,
            normalize: bool = True):
    """Gather every tile's tokens and positions.

    ``latent``: (B, N + num_cond, C), any dtype (copied bit for bit).
    ``pos``: (B, 3, N + num_cond, 2) float32 ``[start, end)`` per axis.

    Source: TDP docs, "What it is" (each tile runs on its own part of the
    latent), "Position normalization" (offset = minimum start of the tile's
    generated tokens per batch element and axis, subtracted from generated and
    conditioning tokens; widths unchanged) and "Shared negative (reference)
    positions" (conditioning tokens follow the generated ones; a tile keeps
    one whose interval overlaps the tile on all three axes or whose time
    coordinate is negative).

    Readings taken where the pages are open:
      * the tile's extent on an axis is ``[min start, max end)`` over its
        generated tokens, in position units; "overlaps" is the half-open test
        ``start < extent_end and end > extent_start`` (touching or
        zero-width intervals are not kept);
      * "negative time coordinate" is a negative start on the time axis;
        both tests use the positions before normalization;
      * with batch > 1 a token is kept when any batch element keeps it, so a
        tile holds one token set for the whole batch;
      * kept tokens follow the generated rows in ascending original order.

    Returns a dict with per-tile lists ``rows`` (source token index per tile
    row), ``latent`` (B, N_t, C), ``pos`` (B, 3, N_t, 2) float32, ``offset``
    (B, 3) float32, ``n_gen``, ``kept`` (conditioning indices) and the
    per-token keep count ``k`` (num_cond,).
    """
    F, H, W = shape
    N = F * H * W
    B = latent.shape[0]
    assert latent.shape[1] == N + num_cond and pos.shape == (B, 3, N + num_cond, 2)
    assert pos.dtype == np.float32
    tiles = enumerate_tiles(shape, tiling)
    cond = pos[:, :, N:, :]
    per_tile = []
    keep_matrix = np.zeros((len(tiles), num_cond), dtype=bool)
    for tile in tiles:
        gen = tile_generated_tokens(tile, shape)
        gen_pos = pos[:, :, gen, :]
        lo = gen_pos[..., 0].min(axis=2)          # (B, 3) min start
        hi = gen_pos[..., 1].max(axis=2)          # (B, 3) max end
        overlaps = (cond[..., 0] < hi[:, :, None]) & (cond[..., 1] > lo[:, :, None])
        keep_b = overlaps.all(axis=1) | (cond[:, 0, :, 0] < 0)
        keep = keep_b.any(axis=0)
        keep_matrix[tile["index"]] = keep
        kept = np.nonzero(keep)[0]
        rows = np.concatenate([gen, N + kept])
        offset = lo.astype(np.float32) if normalize else np.zeros((B, 3), np.float32)
        tile_pos = pos[:, :, rows, :] - offset[:, :, None, None]
        per_tile.append({
            "tile": tile,
            "rows": rows,
            "n_gen": len(gen),
            "kept": kept,
            "offset": offset,
            "extent": np.stack([lo, hi], axis=-1),
            "latent": latent[:, rows, :],
            "pos": tile_pos.astype(np.float32),
        })
    k = keep_matrix.sum(axis=0).astype(np.int64)
    return {"tiles": per_tile, "k": k, "keep": keep_matrix, "N": N}


# --------------------------------------------------------------------------
# Blend
# --------------------------------------------------------------------------

def tile_weights(tile, shape, tiling) -> np.ndarray:
    """Separable 3-D weight of each generated row of a tile (fp64, row-major).

    Source: TDP docs, "What it is" (trapezoidal masks) and mold #673, "Why"
    (a separable trapezoidal window): the weight of a cell is the product of
    the three 1-D windows.
    """
    ws = []
    for d, (n, o) in enumerate(tiling):
        ivs = split_by_count(shape[d], n, o)
        ws.append(window_f64(ivs, tile["grid"][d], o))
    w3 = ws[0][:, None, None] * ws[1][None, :, None] * ws[2][None, None, :]
    return w3.reshape(-1)


def blend(tile_outputs, extracted, shape, tiling, num_cond: int, tiles=None):
    """Recombine tile outputs into the full latent (fp64).

    ``tile_outputs[t]``: (B, N_t, C) floats, rows in the order ``extract``
    produced.  Source: TDP docs, "What it is" (overlaps blended with
    trapezoidal masks, then summed; the masks sum to one) and "Shared
    negative (reference) positions" (a token kept by k tiles is weighted
    1/k); mold #673, "A bug found while porting" (the blend has no
    normalization pass).

    ``tiles``: the tile indices whose terms are added (default: every tile).
    A subset gives the full-size partial buffer of the ranks that ran those
    tiles; k still counts every tile that keeps the token.

    Readings: the sum runs over tiles in ascending tile index and starts
    from a zero buffer (so an all-zero sum is +0.0); a conditioning token
    kept by no tile comes out as zero (a sum of nothing).

    Returns ``(out, magnitude)`` where ``magnitude`` is the sum of
    ``|weight * y|`` over the same terms (used to scale tolerances).
    """
    N = extracted["N"]
    k = extracted["k"]
    T = len(extracted["tiles"])
    chosen = sorted(set(range(T) if tiles is None else tiles))
    B = extracted["tiles"][0]["latent"].shape[0]
    C = extracted["tiles"][0]["latent"].shape[2]
    out = np.zeros((B, N + num_cond, C), dtype=np.float64)
    mag = np.zeros_like(out)
    for t in chosen:
        et = extracted["tiles"][t]
        y = np.asarray(tile_outputs[t], dtype=np.float64)
        n_gen = et["n_gen"]
        gen_rows = et["rows"][:n_gen]
        w = tile_weights(et["tile"], shape, tiling)
        term = w[None, :, None] * y[:, :n_gen, :]
        out[:, gen_rows, :] += term
        mag[:, gen_rows, :] += np.abs(term)
        for j, c in enumerate(et["kept"]):
            term = y[:, n_gen + j, :] / float(k[c])
            out[:, N + c, :] += term
            mag[:, N + c, :] += np.abs(term)
    return out, mag


def rank_partial(tile_outputs, extracted, shape, tiling, num_cond: int, world: int, rank: int):
    """The buffer one rank contributes to the all_reduce (fp64).

    Source: TDP docs, "What it is": tiles go to ranks round-robin, each rank
    adds its tiles' masked outputs into a buffer of the full latent's shape,
    and one all_reduce (a sum) over the ranks gives the blended latent.  So
    rank r's buffer is the blend restricted to tiles t with t mod world == r;
    rows no such tile covers stay zero, and the buffers of all ranks add up
    to ``blend``.  Returns ``(partial, magnitude)`` like ``blend``.
    """
    T = len(extracted["tiles"])
    mine = [t for t in range(T) if round_robin_rank(t, world) == rank]
    return blend(tile_outputs, extracted, shape, tiling, num_cond, tiles=mine)


# --------------------------------------------------------------------------
# Spatial blend of decoded pixel tiles
# --------------------------------------------------------------------------

def pixel_intervals(dim: int, num_tiles: int, overlap: int, scale: int) -> list[tuple[int, int]]:
    """Pixel rows (or columns) that the decode of each latent tile covers.

    Source: mold #673, "Scope" (the VAE decode is tiled spatially so that a
    large frame need not be decoded whole) and DistVAE docs, "Choosing a tile
    window" (tiles and overlaps are set per spatial axis).  Reading: a latent
    cell decodes to ``scale`` pixels on the axis, so latent tile [a, b)
    decodes to pixels [scale*a, scale*b) and neighbours overlap by
    scale*overlap pixels.
    """
    return [(scale * a, scale * b) for a, b in split_by_count(dim, num_tiles, overlap)]


def pixel_blend(tiles, latent_hw, tiling_hw, scale_hw):
    """Recombine decoded pixel tiles (fp64).

    ``tiles[t]``: (B, C, frames, h_t, w_t) arrays, tile t = i_h * n_w + i_w;
    ``latent_hw`` = (H, W) latent cells, ``tiling_hw`` = ((n_h, o_h),
    (n_w, o_w)), ``scale_hw`` = pixels per cell.  Source: TDP docs, "What it
    is" (overlaps are blended with trapezoidal masks that sum to one) and
    mold #673, "Scope" (spatial VAE decode tiling).  Reading: the windows are
    those of the latent blend taken in pixel units, ramps over the
    scale*overlap overlapping pixels; frames are not tiled; the sum runs over
    tiles in ascending index from zero.  Returns ``(out, magnitude)``.
    """
    ivs = [pixel_intervals(d, n, o, s) for d, (n, o), s in zip(latent_hw, tiling_hw, scale_hw)]
    ovl = [o * s for (_, o), s in zip(tiling_hw, scale_hw)]
    B, C, Fo = tiles[0].shape[:3]
    out = np.zeros((B, C, Fo, latent_hw[0] * scale_hw[0], latent_hw[1] * scale_hw[1]), dtype=np.float64)
    mag = np.zeros_like(out)
    for t, (i, j) in enumerate(itertools.product(range(len(ivs[0])), range(len(ivs[1])))):
        (y0, y1), (x0, x1) = ivs[0][i], ivs[1][j]
        w = np.outer(window_f64(ivs[0], i, ovl[0]), window_f64(ivs[1], j, ovl[1]))
        term = w * np.asarray(tiles[t], dtype=np.float64)
        out[:, :, :, y0:y1, x0:x1] += term
        mag[:, :, :, y0:y1, x0:x1] += np.abs(term)
    return out, mag


# --------------------------------------------------------------------------
# bf16 storage
# --------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32: bf16 is the top half of fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns, round-to-nearest-even; NaN stays NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


# --------------------------------------------------------------------------
# Geometry helpers used by checks
# --------------------------------------------------------------------------

def tiling_quality(dims, intervals, world: int) -> dict:
    """Plan-quality figures of a tiling, exact (integers and Fractions).

    Source: DistVAE docs, "Choosing a tile window": section "The two axes
    cost differently" (a tiling decodes more than the latent's area because
    tiles repeat their overlaps; tiles hold a share of the activations; each
    pair of neighbouring tiles leaves a seam), "Clipping unbalances a grid,
    not the tile count" (ranks that get the same number of tiles can get
    different amounts of work; imbalance is the heaviest rank against an
    even split) and "The tile count caps the GPU count".

    ``dims`` are the axis lengths; ``intervals[d]`` the half-open intervals
    of axis d.  Tiles are the Cartesian product in row-major order, and on
    ``world`` ranks tile t goes to rank t mod world (TDP docs, "What it
    is").  Readings: a tile's work is its cell count; a seam is a pair of
    tiles whose grid indices differ by one on exactly one axis; the even
    split divides the total work by ``world`` (idle ranks included).
    """
    grid_cells = 1
    for d in dims:
        grid_cells *= int(d)
    counts = [len(v) for v in intervals]
    cells = []
    for grid in itertools.product(*[range(c) for c in counts]):
        c = 1
        for d, i in enumerate(grid):
            a, b = intervals[d][i]
            c *= int(b) - int(a)
        cells.append(c)
    seams = 0
    grids = list(itertools.product(*[range(c) for c in counts]))
    for x in range(len(grids)):
        for y in range(x + 1, len(grids)):
            diff = [abs(p - q) for p, q in zip(grids[x], grids[y])]
            if sorted(diff)[-1] == 1 and sum(diff) == 1:
                seams += 1
    rank_cells = [0] * world
    for t, c in enumerate(cells):
        rank_cells[round_robin_rank(t, world)] += c
    total = sum(cells)
    return {
        "total_cells": total,
        "grid_cells": grid_cells,
        "largest_cells": max(cells),
        "seams": seams,
        "rank_cells": rank_cells,
        "max_rank_cells": max(rank_cells),
        "area_ratio": Fraction(total, grid_cells),
        "largest_fraction": Fraction(max(cells), grid_cells),
        "imbalance": Fraction(max(rank_cells) * world, total) - 1,
    }


def decoded_area_ratio(shape, tiling) -> float:
    """Total generated tokens over all tiles divided by N (tiles re-process overlaps)."""
    tiles = enumerate_tiles(shape, tiling)
    total = sum(int(np.prod(t["size"])) for t in tiles)
    return total / float(np.prod(shape))
