"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/), closed forms, invariants the pages state, and
hand-built cases with answers worked out by hand.  ``test_mutants_fail_pins``
plants plausible mistakes in copies of oracle functions and checks that a pin
catches each one.
"""
import collections
import itertools
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle as O
from oracle import tdp_oracle as OT
from synth import WORKLOADS, Workload, denoiser_params, grid_positions, make_inputs

GOLDEN = Path(__file__).parent / "golden"


def load_window_table():
    rows = []
    for line in (GOLDEN / "window_sums.txt").read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        dim, n, o, printed = line.split()
        rows.append((int(dim), int(n), int(o), float(printed)))
    return rows


def table_pin_holds(window_sums) -> bool:
    """The printed window-sum table, as a predicate over a window-sum function."""
    for dim, n, o, printed in load_window_table():
        sums = window_sums(dim, n, o)
        if printed == 1.0:
            if any(s != 1 for s in sums):
                return False
        elif abs(float(max(sums)) - printed) > 1e-3:
            return False
        if min(sums) < 1 - 1e-12:   # stacking only ever adds weight
            return False
    return True


# --- p1: the pages' window-sum table -------------------------------------

def test_window_sum_table_matches_pages():
    assert table_pin_holds(O.window_sums_exact)


def test_window_sum_prose_value():
    # "as much as 1.16" for the 4-tile split
    assert round(float(max(O.window_sums_exact(21, 4, 8))), 2) == 1.16


def test_window_sums_hand_derived():
    # (21, 3, 8): tiles [0,12), [4,16), [8,21); cell 9 lies in all three:
    # 3/9 (falling ramp of tile 0) + (6/9)(7/9) (both ramps of tile 1) + 2/9.
    sums = O.window_sums_exact(21, 3, 8)
    assert sums[9] == Fraction(3, 9) + Fraction(6, 9) * Fraction(7, 9) + Fraction(2, 9)
    assert max(sums) == Fraction(29, 27)
    assert O.split_by_count(21, 3, 8) == [(0, 12), (4, 16), (8, 21)]


# --- p2: partition of unity on every guarded split -------------------------

def test_guarded_splits_are_partitions_of_unity():
    checked = 0
    for dim in range(1, 41):
        for n in range(1, 7):
            for o in range(0, 11):
                if dim - o < n or not O.guard_holds(dim, n, o):
                    continue
                assert all(s == 1 for s in O.window_sums_exact(dim, n, o)), (dim, n, o)
                checked += 1
    assert checked > 300


def test_guard_matches_tile_size_bound():
    # The guard is "tile size >= 2*overlap" under the average tile size
    # (dim + (n-1)*o)/n: o*(n+1) <= dim  <=>  (dim + (n-1)o)/n >= 2o.
    for dim in range(1, 60):
        for n in range(2, 8):
            for o in range(0, 20):
                lhs = O.guard_holds(dim, n, o)
                rhs = Fraction(dim + (n - 1) * o, n) >= 2 * o
                assert lhs == rhs
    assert not O.guard_holds(21, 2, 8)        # 8 * 3 > 21
    assert O.guard_holds(21, 4, 4)
    assert not O.guard_holds(10, 1, 1)        # an untiled axis takes no overlap


def test_guarded_split_never_triple_overlaps():
    for dim in range(2, 60):
        for n in range(2, 8):
            for o in range(1, 15):
                if dim - o < n or not O.guard_holds(dim, n, o):
                    continue
                ivs = O.split_by_count(dim, n, o)
                cover = [sum(a <= x < b for a, b in ivs) for x in range(dim)]
                assert max(cover) <= 2


def test_3d_weights_partition_of_unity():
    for shape, tiling in [((9, 20, 31), ((2, 2), (3, 4), (4, 5))),
                          ((16, 68, 120), ((1, 0), (4, 8), (4, 16))),
                          ((16, 32, 48), ((2, 2), (3, 6), (3, 8)))]:
        total = np.zeros(shape)
        for tile in O.enumerate_tiles(shape, tiling):
            (f0, h0, w0), (sf, sh, sw) = tile["origin"], tile["size"]
            total[f0:f0 + sf, h0:h0 + sh, w0:w0 + sw] += \
                O.tile_weights(tile, shape, tiling).reshape(sf, sh, sw)
        np.testing.assert_allclose(total, 1.0, rtol=0, atol=1e-12)


# --- p3: interval invariants ----------------------------------------------

def test_interval_invariants():
    for dim in range(1, 80):
        for n in range(1, 9):
            for o in range(0, 12):
                if dim - o < n:
                    with pytest.raises(ValueError):
                        O.split_by_count(dim, n, o)
                    continue
                ivs = O.split_by_count(dim, n, o)
                assert len(ivs) == n
                assert ivs[0][0] == 0 and ivs[-1][1] == dim
                for (a0, b0), (a1, b1) in zip(ivs, ivs[1:]):
                    assert b0 - a1 == o           # neighbours share exactly o cells
                    assert a1 > a0
                sizes = [b - a for a, b in ivs]
                assert sum(sizes) == dim + (n - 1) * o
                assert max(sizes) - min(sizes) <= 1
                assert all(0 <= a < b <= dim for a, b in ivs)


def test_split_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.split_by_count(10, 0, 0)
    with pytest.raises(ValueError):
        O.split_by_count(10, 2, -1)
    with pytest.raises(ValueError):
        O.split_by_count(4, 3, 2)


# --- p8: geometry ---------------------------------------------------------

@pytest.mark.parametrize("name", list(WORKLOADS))
def test_decoded_area_closed_form(name):
    wl = WORKLOADS[name]
    expect = 1.0
    for dim, (n, o) in zip(wl.shape, wl.tiling):
        expect *= (dim + (n - 1) * o) / dim
    assert O.decoded_area_ratio(wl.shape, wl.tiling) == pytest.approx(expect, rel=1e-15)
    for dim, (n, o) in zip(wl.shape, wl.tiling):
        assert O.guard_holds(dim, n, o)


def test_tile_order_is_a_free_reading():
    """The pages fix round-robin (TDP docs, "What it is": 16 tiles on 4
    GPUs) but no tile order, so the row-major order (reading g6) is a free
    choice, parity unpinned.  What holds for any order is pinned here:
    the enumeration lists every cell of the tile grid once, 16 tiles on 4
    ranks give each rank 4, and the blend does not depend on the order
    beyond summation rounding (the same tiles in a shuffled order agree to
    fp64 rounding)."""
    shape, tiling = (4, 10, 12), ((2, 1), (2, 2), (3, 3))
    tiles = O.enumerate_tiles(shape, tiling)
    grids = [tuple(t["grid"]) for t in tiles]
    assert len(set(grids)) == len(grids) == 2 * 2 * 3
    assert set(grids) == set(itertools.product(range(2), range(2), range(3)))
    sixteen = O.enumerate_tiles((1, 16, 16), ((1, 0), (4, 2), (4, 2)))
    per_rank = collections.Counter(O.round_robin_rank(t["index"], 4) for t in sixteen)
    assert sorted(per_rank.values()) == [4, 4, 4, 4]
    wl = Workload("order", 2, 8, shape, tiling, num_cond=40, num_ref=10, dtype="f32", seed=3)
    inp = make_inputs(wl)
    ex = O.extract(inp["latent"], inp["pos"], shape, tiling, wl.num_cond)
    rng = np.random.default_rng(17)
    ys = [rng.standard_normal((2, len(et["rows"]), 8)) for et in ex["tiles"]]
    ref, _ = O.blend(ys, ex, shape, tiling, wl.num_cond)
    perm = rng.permutation(len(ys))
    shuffled = dict(ex, tiles=[ex["tiles"][i] for i in perm])
    out, _ = O.blend([ys[i] for i in perm], shuffled, shape, tiling, wl.num_cond)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# --- p4: extract moves the right rows -------------------------------------

def _coordinate_latent(B, shape, C, num_cond=0):
    """int64 latent whose entries spell out (b, f, h, w, c) in decimal fields."""
    F, H, W = shape
    lat = np.empty((B, F * H * W + num_cond, C), dtype=np.int64)
    for b in range(B):
        for f in range(F):
            for h in range(H):
                for w in range(W):
                    n = (f * H + h) * W + w
                    for c in range(C):
                        lat[b, n, c] = (((b * 100 + f) * 1000 + h) * 1000 + w) * 100 + c
        for j in range(num_cond):
            lat[b, F * H * W + j, :] = -(b * 10000 + j)
    return lat


def test_extract_rows_brute_force():
    shape, tiling, B, C = (5, 9, 11), ((2, 1), (3, 2), (2, 3)), 2, 3
    lat = _coordinate_latent(B, shape, C)
    pos = grid_positions(B, shape, (1, 1, 1))
    ex = O.extract(lat, pos, shape, tiling, 0)
    assert len(ex["tiles"]) == 12
    for et in ex["tiles"]:
        (f0, h0, w0), (sf, sh, sw) = et["tile"]["origin"], et["tile"]["size"]
        row = 0
        for lf in range(sf):
            for lh in range(sh):
                for lw in range(sw):
                    for b in range(B):
                        for c in range(C):
                            v = int(et["latent"][b, row, c])
                            assert v % 100 == c
                            v //= 100
                            assert v % 1000 == w0 + lw
                            v //= 1000
                            assert v % 1000 == h0 + lh
                            v //= 1000
                            assert v % 100 == f0 + lf
                            assert v // 100 == b
                    row += 1
        assert row == et["n_gen"] == len(et["rows"])


@pytest.mark.parametrize("name", ["tiny", "ltx", "fullres", "conditioned"])
def test_identity_denoiser_reproduces_input(name):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
    if wl.num_cond:
        assert ex["k"].min() >= 1
    if wl.dtype == "bf16":
        ys = [O.bf16_bits_to_f32(et["latent"]) for et in ex["tiles"]]
    else:
        ys = [et["latent"] for et in ex["tiles"]]
    out, _ = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    if wl.dtype == "bf16":
        # Compared as values: a -0.0 input sums to +0.0 (the sum starts from zero).
        got = O.bf16_bits_to_f32(O.f32_to_bf16_bits(out.astype(np.float32)))
        assert np.array_equal(got, O.bf16_bits_to_f32(inp["latent"]))
    else:
        np.testing.assert_allclose(out, inp["latent"], rtol=0, atol=2e-6 * np.abs(inp["latent"]).max())


# --- p5: positions --------------------------------------------------------

def test_normalized_grid_positions_equal_tile_grid():
    # Per-tile normalization is what building positions at the tile's own
    # shape gives (mold #673, "Scope").
    for name in ["ltx", "4k", "conditioned"]:
        wl = WORKLOADS[name]
        B, N = wl.batch, wl.tokens
        pos = grid_positions(B, wl.shape, wl.pos_scale)
        ex = O.extract(np.zeros((B, N, 1), np.float32), pos, wl.shape, wl.tiling, 0)
        for et in ex["tiles"]:
            want = grid_positions(B, et["tile"]["size"], wl.pos_scale)
            assert np.array_equal(et["pos"], want)


def test_normalized_positions_start_at_zero_and_keep_widths():
    rng = np.random.default_rng(7)
    shape, tiling, B = (4, 10, 12), ((2, 1), (2, 3), (3, 2)), 2
    N = 4 * 10 * 12
    start = rng.uniform(-50, 50, size=(B, 3, N)).astype(np.float32)
    width = rng.uniform(0.5, 3, size=(B, 3, N)).astype(np.float32)
    pos = np.stack([start, start + width], axis=-1).astype(np.float32)
    ex = O.extract(np.zeros((B, N, 1), np.float32), pos, shape, tiling, 0)
    for et in ex["tiles"]:
        p = et["pos"]
        assert np.all(p[..., 0].min(axis=2) == 0.0)
        src = pos[:, :, et["rows"], :]
        assert np.array_equal(p, src - et["offset"][:, :, None, None])
        np.testing.assert_allclose(p[..., 1] - p[..., 0], src[..., 1] - src[..., 0], atol=1e-4)
    ex_raw = O.extract(np.zeros((B, N, 1), np.float32), pos, shape, tiling, 0, normalize=False)
    for et in ex_raw["tiles"]:
        assert np.array_equal(et["pos"], pos[:, :, et["rows"], :])


# --- p6: conditioning selection ------------------------------------------

def test_selection_hand_built():
    # Time axis split (4, 2 tiles, overlap 1) -> tiles [0,2) and [1,4) in
    # position units (scale 1); height and width untiled, extent [0,4).
    shape, tiling, B = (4, 4, 4), ((2, 1), (1, 0), (1, 0)), 2
    N = 64
    full = (0.0, 4.0)
    cond = [  # (time, height, width) intervals, batch 0 then batch 1 if different
        ((2, 3), full, full),          # c0: only tile 1 (tile 0 ends at 2)
        ((1, 2), full, full),          # c1: both tiles
        ((-3, -2), (9, 10), (9, 10)),  # c2: negative time -> every tile
        ((0, 0), full, full),          # c3: zero width -> none
        ((0, 1), (4, 5), full),        # c4: touches height end -> none
        ((0, 1), (3, 4), (3, 4)),      # c5: tile 0 only (tile 1 starts at 1)
        ((10, 11), full, full),        # c6: batch 0 outside; batch 1 below -> tile 0
    ]
    pos = np.zeros((B, 3, N + len(cond), 2), np.float32)
    pos[:, :, :N, :] = grid_positions(B, shape, (1, 1, 1))
    for c, ivs in enumerate(cond):
        for d in range(3):
            pos[:, d, N + c, :] = ivs[d]
    pos[1, 0, N + 6, :] = (0, 1)
    lat = np.zeros((B, N + len(cond), 1), np.float32)
    ex = O.extract(lat, pos, shape, tiling, len(cond))
    want = np.array([[0, 1, 1, 0, 0, 1, 1],
                     [1, 1, 1, 0, 0, 0, 0]], dtype=bool)
    assert np.array_equal(ex["keep"], want)
    assert ex["k"].tolist() == [1, 2, 2, 0, 0, 1, 1]
    assert ex["tiles"][0]["kept"].tolist() == [1, 2, 5, 6]
    # kept rows follow the generated rows in ascending order
    assert ex["tiles"][0]["rows"][ex["tiles"][0]["n_gen"]:].tolist() == [N + 1, N + 2, N + 5, N + 6]
    # a token kept by no tile blends to zero
    ys = [np.ones((B, len(et["rows"]), 1)) for et in ex["tiles"]]
    out, _ = O.blend(ys, ex, shape, tiling, len(cond))
    assert np.all(out[:, N + 3] == 0) and np.all(out[:, N + 4] == 0)
    assert np.allclose(out[:, N + 1], 1.0)


@pytest.mark.parametrize("name", ["tiny", "conditioned"])
def test_tables_depend_on_positions_only(name):
    """Reading g17: the shift (TDP docs, "Position normalization") and the
    keep rule (TDP docs, "Shared negative (reference) positions") read the
    positions only.  Two latents on the same positions give the same index
    maps, counts, kept lists, shifted positions and k, and the second
    latent's tile rows are its rows taken through the first's index map."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    other = make_inputs(wl, seed=wl.seed + 7)["latent"]
    assert not np.array_equal(other, inp["latent"])
    a = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
    b = O.extract(other, inp["pos"], wl.shape, wl.tiling, wl.num_cond)
    assert np.array_equal(a["k"], b["k"]) and np.array_equal(a["keep"], b["keep"])
    for ta, tb in zip(a["tiles"], b["tiles"]):
        for key in ("rows", "kept", "offset", "extent", "pos"):
            assert np.array_equal(np.asarray(ta[key]), np.asarray(tb[key])), key
        assert ta["n_gen"] == tb["n_gen"]
        assert np.array_equal(tb["latent"], other[:, ta["rows"], :])


def test_reference_tokens_kept_by_every_tile():
    wl = WORKLOADS["conditioned"]
    inp = make_inputs(wl)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
    T = len(ex["tiles"])
    assert T == 18
    assert np.all(ex["k"][:wl.num_ref] == T)
    assert np.all(ex["keep"][:, :wl.num_ref])
    assert np.all(ex["k"] >= 1) and np.all(ex["k"] <= T)


# --- p7: blend closed forms ----------------------------------------------

def test_blend_equal_affine_is_affine():
    wl = WORKLOADS["conditioned"]
    inp = make_inputs(wl)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
    a, b = 1.375, -0.625
    ys = [a * O.bf16_bits_to_f32(et["latent"]).astype(np.float64) + b for et in ex["tiles"]]
    out, _ = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    x = O.bf16_bits_to_f32(inp["latent"]).astype(np.float64)
    np.testing.assert_allclose(out, a * x + b, rtol=1e-12, atol=1e-12)


def test_blend_per_tile_affine_voxelwise():
    # Voxel-driven restatement: out(v) = x(v) * sum_t W_t(v) a_t + sum_t W_t(v) b_t,
    # with the covering tiles found by interval membership.
    wl = WORKLOADS["ltx"]
    inp = make_inputs(wl)
    x = O.bf16_bits_to_f32(inp["latent"]).astype(np.float64)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, 0)
    T = len(ex["tiles"])
    a, b = denoiser_params(wl.seed, T, "affine")
    ys = [a[t] * O.bf16_bits_to_f32(et["latent"]).astype(np.float64) + b[t]
          for t, et in enumerate(ex["tiles"])]
    out, _ = O.blend(ys, ex, wl.shape, wl.tiling, 0)
    F, H, W = wl.shape
    ivs = [O.split_by_count(d, n, o) for d, (n, o) in zip(wl.shape, wl.tiling)]
    wins = [[O.window_exact(ivs[d], i, wl.tiling[d][1]) for i in range(len(ivs[d]))] for d in range(3)]
    rng = np.random.default_rng(0)
    for n in rng.choice(F * H * W, size=300, replace=False):
        f, h, w = n // (H * W), (n // W) % H, n % W
        sa = sb = Fraction(0)
        for t, (i, j, k) in enumerate(itertools.product(*[range(len(v)) for v in ivs])):
            cells = (f, h, w)
            idx = (i, j, k)
            if all(ivs[d][idx[d]][0] <= cells[d] < ivs[d][idx[d]][1] for d in range(3)):
                wt = Fraction(1)
                for d in range(3):
                    wt *= wins[d][idx[d]][cells[d] - ivs[d][idx[d]][0]]
                sa += wt * Fraction(float(a[t]))
                sb += wt * Fraction(float(b[t]))
        np.testing.assert_allclose(out[0, n], x[0, n] * float(sa) + float(sb), rtol=1e-12, atol=1e-12)


# --- rank partials (round-robin share of the all_reduce) ------------------

def _affine_outputs(wl, ex):
    a, b = denoiser_params(wl.seed, len(ex["tiles"]), "affine")
    return [a[t] * O.bf16_bits_to_f32(et["latent"]).astype(np.float64) + b[t]
            for t, et in enumerate(ex["tiles"])], a, b


def test_rank_partials_add_up_to_blend():
    # The all_reduce sums the ranks' buffers: for any world size the
    # partials add up to the whole blend, and one rank is the whole blend.
    wl = WORKLOADS["conditioned"]
    inp = make_inputs(wl)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
    ys, _, _ = _affine_outputs(wl, ex)
    full, mag = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    one, _ = O.rank_partial(ys, ex, wl.shape, wl.tiling, wl.num_cond, 1, 0)
    assert np.array_equal(one, full)
    for world in (2, 4, 5, 18, 25):
        total = sum(O.rank_partial(ys, ex, wl.shape, wl.tiling, wl.num_cond, world, r)[0] for r in range(world))
        assert np.all(np.abs(total - full) <= 1e-12 * mag + 1e-300), world


def test_rank_partial_voxelwise():
    # Rank 1 of 3 on the LTX-like grid, restated per voxel with exact
    # windows: the sum over the rank's tiles (t mod 3 == 1) that contain
    # the voxel, zero where none does.
    wl = WORKLOADS["ltx"]
    inp = make_inputs(wl)
    x = O.bf16_bits_to_f32(inp["latent"]).astype(np.float64)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, 0)
    ys, a, b = _affine_outputs(wl, ex)
    world, rank = 3, 1
    part, _ = O.rank_partial(ys, ex, wl.shape, wl.tiling, 0, world, rank)
    F, H, W = wl.shape
    ivs = [O.split_by_count(d, n, o) for d, (n, o) in zip(wl.shape, wl.tiling)]
    wins = [[O.window_exact(ivs[d], i, wl.tiling[d][1]) for i in range(len(ivs[d]))] for d in range(3)]
    rng = np.random.default_rng(5)
    zeros = 0
    for n in rng.choice(F * H * W, size=400, replace=False):
        cells = (n // (H * W), (n // W) % H, n % W)
        sa = sb = Fraction(0)
        covered = False
        for t, idx in enumerate(itertools.product(*[range(len(v)) for v in ivs])):
            if t % world != rank:
                continue
            if all(ivs[d][idx[d]][0] <= cells[d] < ivs[d][idx[d]][1] for d in range(3)):
                covered = True
                wt = Fraction(1)
                for d in range(3):
                    wt *= wins[d][idx[d]][cells[d] - ivs[d][idx[d]][0]]
                sa += wt * Fraction(float(a[t]))
                sb += wt * Fraction(float(b[t]))
        if not covered:
            zeros += 1
            assert np.all(part[0, n] == 0.0)
        np.testing.assert_allclose(part[0, n], x[0, n] * float(sa) + float(sb), rtol=1e-12, atol=1e-12)
    assert zeros > 0   # the sample meets voxels outside the rank's tiles


def test_rank_partial_conditioning_uses_global_k():
    # All-ones tile outputs: a conditioning row of rank r's buffer is
    # (tiles of rank r that keep c) / (tiles that keep c), so the ranks'
    # rows add up to one for every kept token.
    wl = WORKLOADS["conditioned"]
    inp = make_inputs(wl)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
    ones = [np.ones(et["latent"].shape) for et in ex["tiles"]]
    keep = ex["keep"]
    T = keep.shape[0]
    world = 4
    total = np.zeros(wl.num_cond)
    for r in range(world):
        part, _ = O.rank_partial(ones, ex, wl.shape, wl.tiling, wl.num_cond, world, r)
        mine = keep[[t for t in range(T) if t % world == r]].sum(axis=0)
        want = mine / keep.sum(axis=0)
        np.testing.assert_allclose(part[:, wl.tokens:, :], np.broadcast_to(want[None, :, None], part[:, wl.tokens:, :].shape),
                                   rtol=1e-15, atol=0)
        total += part[0, wl.tokens:, 0]
    np.testing.assert_allclose(total, 1.0, rtol=1e-15)


def test_mutant_rank_local_k_fails_pin():
    # Planted mistake: each rank divides by the number of its own tiles that
    # keep the token.  The ranks' conditioning rows then no longer add to one.
    wl = WORKLOADS["conditioned"]
    inp = make_inputs(wl)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
    ones = [np.ones(et["latent"].shape) for et in ex["tiles"]]
    keep = ex["keep"]
    T, world = keep.shape[0], 4
    total = np.zeros(wl.num_cond)
    for r in range(world):
        mine = [t for t in range(T) if t % world == r]
        wrong = dict(ex, k=keep[mine].sum(axis=0))
        part, _ = O.blend(ones, wrong, wl.shape, wl.tiling, wl.num_cond, tiles=mine)
        total += part[0, wl.tokens:, 0]
    assert not np.allclose(total, 1.0, rtol=1e-15)


# --- bf16 storage --------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.integers(0, 2**32, 100000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 1.0 + 2**-8, 1.0 + 3 * 2**-8], np.float32),
    ])
    x = x[~np.isnan(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(x), want)
    assert np.array_equal(O.bf16_bits_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())
    assert np.isnan(O.bf16_bits_to_f32(O.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


# --- the pins catch planted mistakes -------------------------------------

def _mutant_sums(window_fn=None, split_fn=None):
    def sums(dim, n, o):
        ivs = (split_fn or O.split_by_count)(dim, n, o)
        s = [Fraction(0)] * dim
        for i, (a0, _) in enumerate(ivs):
            for j, w in enumerate((window_fn or O.window_exact)(ivs, i, o)):
                if 0 <= a0 + j < dim:
                    s[a0 + j] += w
        return s
    return sums


def test_mutants_fail_pins():
    def ramp_j_over_o(ivs, i, o):          # ramp j/o instead of (j+1)/(o+1)
        n, (a, b) = len(ivs), ivs[i]
        size, out = b - a, []
        for j in range(size):
            w = Fraction(1)
            if i > 0 and j < o:
                w *= Fraction(j, o)
            if i < n - 1 and j >= size - o:
                w *= Fraction(size - 1 - j, o)
            out.append(w)
        return out

    def ramp_min_combine(ivs, i, o):       # both ramps -> min instead of product
        n, (a, b) = len(ivs), ivs[i]
        size, out = b - a, []
        for j in range(size):
            ws = [Fraction(1)]
            if i > 0 and j < o:
                ws.append(Fraction(j + 1, o + 1))
            if i < n - 1 and j >= size - o:
                ws.append(Fraction(size - j, o + 1))
            out.append(min(ws))
        return out

    def split_ceil_clip(dim, n, o):        # ceil tile size, last tile clipped
        size = -(-(dim + (n - 1) * o) // n)
        return [(i * (size - o), min(dim, i * (size - o) + size)) for i in range(n)]

    def split_overlap_minus_one(dim, n, o):
        return O.split_by_count(dim, n, max(o - 1, 0))

    for mutant in [_mutant_sums(window_fn=ramp_j_over_o),
                   _mutant_sums(window_fn=ramp_min_combine),
                   _mutant_sums(split_fn=split_ceil_clip),
                   _mutant_sums(split_fn=split_overlap_minus_one)]:
        assert not table_pin_holds(mutant)
    assert table_pin_holds(_mutant_sums())


def test_mutant_blend_dropped_term_fails_identity():
    wl = WORKLOADS["ltx"]
    inp = make_inputs(wl)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, 0)
    ys = [O.bf16_bits_to_f32(et["latent"]) for et in ex["tiles"]]
    ys[3] = np.zeros_like(ys[3])          # a tile's contribution dropped
    out, _ = O.blend(ys, ex, wl.shape, wl.tiling, 0)
    got = O.bf16_bits_to_f32(O.f32_to_bf16_bits(out.astype(np.float32)))
    assert not np.array_equal(got, O.bf16_bits_to_f32(inp["latent"]))


# --------------------------------------------------------------------------
# Plan-quality figures (DistVAE docs, "Choosing a tile window")
# --------------------------------------------------------------------------

def _read_fixture(name):
    vals = {}
    for line in open(GOLDEN / name):
        line = line.split("#", 1)[0].split()
        if line:
            vals[line[0]] = [float(x) if "." in x else int(x) for x in line[1:]]
    return vals


def _strips_from_fixture(fx):
    h, w = fx["latent"]
    rows = fx["strip_rows"]
    full, last = rows[0], rows[-1]
    stride = (h - last) // (len(rows) - 1)
    starts = [i * stride for i in range(len(rows))]
    ivs = [(a, min(a + full, h)) for a in starts]
    assert [b - a for a, b in ivs] == rows          # the printed row counts
    assert full - last == full - stride             # last strip shorter by exactly the overlap
    return (h, w), [ivs, [(0, w)]]


def test_quality_distvae_strips():
    fx = _read_fixture("distvae_strips.txt")
    dims, ivs = _strips_from_fixture(fx)
    q = O.tiling_quality(dims, ivs, fx["ranks"][0])
    assert q["area_ratio"] == Fraction(161, 128)
    assert round(float(q["area_ratio"]), 2) == fx["area_ratio"][0]
    assert round(float(q["largest_fraction"]), 2) == fx["activations_fraction"][0]
    assert q["seams"] == fx["strip_seams"][0]
    assert q["rank_cells"] == [r * dims[1] for r in fx["strip_rows"]]
    assert q["imbalance"] == Fraction(11, 161)
    assert round(100 * float(q["imbalance"]), 1) == fx["imbalance_percent"][0]


def test_quality_grid_seams_and_closed_form():
    fx = _read_fixture("distvae_strips.txt")
    nh, nw = fx["grid"]
    q = O.tiling_quality((128, 128), [O.split_by_count(128, nh, 8), O.split_by_count(128, nw, 8)], 4)
    assert q["seams"] == fx["grid_seams"][0]
    # seams = sum over axes of (n_d - 1) * prod of the other counts
    rng = np.random.default_rng(11)
    for _ in range(40):
        counts = [int(x) for x in rng.integers(1, 5, 3)]
        ivs = [O.split_by_count(64, n, 0) for n in counts]
        expect = sum((counts[d] - 1) * int(np.prod([counts[e] for e in range(3) if e != d])) for d in range(3))
        assert O.tiling_quality((64, 64, 64), ivs, 3)["seams"] == expect


def test_quality_ratio_matches_geometry_and_balance():
    # area ratio = prod (dim + (n-1) o) / dim for count-based splits
    for shape, tiling in [((16, 68, 120), ((1, 0), (4, 8), (4, 16))), ((16, 32, 48), ((2, 2), (3, 6), (3, 8)))]:
        ivs = [O.split_by_count(d, n, o) for d, (n, o) in zip(shape, tiling)]
        q = O.tiling_quality(shape, ivs, 4)
        assert q["area_ratio"] == Fraction(int(np.prod([d + (n - 1) * o for d, (n, o) in zip(shape, tiling)])),
                                           int(np.prod(shape)))
        assert sum(q["rank_cells"]) == q["total_cells"]
    # the 4K grid on 4 ranks: rank r gets the column i_w = r, all equal
    q = O.tiling_quality((16, 68, 120), [O.split_by_count(16, 1, 0), O.split_by_count(68, 4, 8),
                                         O.split_by_count(120, 4, 16)], 4)
    assert q["imbalance"] == 0
    # more ranks than tiles: idle ranks count in the even split
    fx = _read_fixture("distvae_strips.txt")
    dims, ivs = _strips_from_fixture(fx)
    q = O.tiling_quality(dims, ivs, 8)
    assert q["rank_cells"][4:] == [0, 0, 0, 0]
    assert q["imbalance"] == Fraction(43 * 8, 161) - 1


# --------------------------------------------------------------------------
# Spatial blend of decoded pixel tiles (mold #673, "Scope")
# --------------------------------------------------------------------------

def test_pixel_windows_partition_of_unity_exact():
    rng = np.random.default_rng(41)
    for _ in range(40):
        dim = int(rng.integers(2, 30))
        n = int(rng.integers(1, 5))
        o = 0 if n == 1 else int(rng.integers(0, dim // (n + 1) + 1))
        if dim - o < n:
            continue
        s = int(rng.integers(1, 9))
        ivs = O.pixel_intervals(dim, n, o, s)
        assert ivs[0][0] == 0 and ivs[-1][1] == dim * s
        sums = [Fraction(0)] * (dim * s)
        for i, (a, _) in enumerate(ivs):
            for jj, w in enumerate(OT.window_exact(ivs, i, o * s)):
                sums[a + jj] += w
        assert all(x == 1 for x in sums), (dim, n, o, s)


def test_pixel_blend_reassembles_an_image():
    """Tiles cut from one image blend back to it: the windows sum to one."""
    rng = np.random.default_rng(42)
    for hw, tiling, scale in [((6, 10), ((2, 2), (3, 2)), (4, 8)), ((5, 7), ((1, 0), (2, 1)), (3, 2)),
                              ((9, 9), ((3, 2), (3, 2)), (2, 2))]:
        B, C, Fo = 2, 3, 2
        img = rng.standard_normal((B, C, Fo, hw[0] * scale[0], hw[1] * scale[1]))
        ivs = [O.pixel_intervals(d, n, o, s) for d, (n, o), s in zip(hw, tiling, scale)]
        tiles = [img[:, :, :, y0:y1, x0:x1] for (y0, y1) in ivs[0] for (x0, x1) in ivs[1]]
        out, mag = O.pixel_blend(tiles, hw, tiling, scale)
        assert np.allclose(out, img, rtol=0, atol=1e-14 * np.abs(img).max() * 4)
        assert np.all(mag >= np.abs(out) - 1e-12)


def test_pixel_blend_scale_one_is_the_latent_blend():
    """At one pixel per cell the pixel blend is the latent blend of a one-frame grid."""
    rng = np.random.default_rng(43)
    hw, tiling = (8, 12), ((2, 2), (3, 2))
    shape, tiling3 = (1,) + hw, ((1, 0),) + tiling
    N = int(np.prod(shape))
    ex = O.extract(np.zeros((1, N, 4), np.float32), OT_grid(shape), shape, tiling3, 0)
    ys, tiles = [], []
    for et in ex["tiles"]:
        y = rng.standard_normal((1, len(et["rows"]), 4))
        ys.append(y)
        _, sh, sw = et["tile"]["size"]
        tiles.append(y.reshape(1, sh, sw, 4).transpose(0, 3, 1, 2)[:, :, None])   # (B, C, 1, h, w)
    ref, _ = O.blend(ys, ex, shape, tiling3, 0)
    out, _ = O.pixel_blend(tiles, hw, tiling, (1, 1))
    assert np.array_equal(out[:, :, 0].transpose(0, 2, 3, 1).reshape(1, N, 4), ref)


def OT_grid(shape):
    return grid_positions(1, shape, (1, 1, 1))
