"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Extract results (tile rows, positions, index maps, counts, selection, k)
must match bit for bit; blends must sit within the stated tolerances:
fp32 output |gpu - ref| <= 2e-6 * sum|w*y|, bf16 output adds 4e-3 * |ref|
for the final rounding (ref = the oracle's unrounded fp64 value).
Every input is seeded; every comparison covers every element.
"""
import numpy as np
import pytest
import torch

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp
from harness import (check_blend, check_extract, cond_tables, gpu_blend, gpu_extract, latent_bits, note,
                     oracle_tile_floats, plan_for, slot_buffer_from_tiles)
from synth import WORKLOADS, Workload, denoiser_params, grid_positions, make_inputs, random_tile_outputs

pytestmark = pytest.mark.gpu

ALL = list(WORKLOADS)


def oracle_extract(wl, inp, normalize=True):
    return O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond, normalize=normalize)


@pytest.mark.parametrize("name", ALL)
def test_extract_bit_exact(name, cuda):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    plan = plan_for(wl)
    _, _, bufs = gpu_extract(plan, inp, cuda, name)
    check_extract(plan, bufs, oracle_extract(wl, inp), wl.num_cond)


@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_blend_random_tiles(name, out_dtype, cuda):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    plan = plan_for(wl, out_dtype=out_dtype)
    ex = oracle_extract(wl, inp)
    rng = np.random.default_rng(100 + wl.seed)
    tiles = [random_tile_outputs(rng, wl.batch, len(et["rows"]), wl.channels, wl.dtype) for et in ex["tiles"]]
    buf = slot_buffer_from_tiles(plan, tiles, plan.cfg.in_dtype, rng)
    ys = [O.bf16_bits_to_f32(y) if y.dtype == np.uint16 else y for y in tiles]
    ref, mag = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    cond_row, cond_k = cond_tables(plan, ex, wl.num_cond, cuda)
    out = gpu_blend(plan, buf, cond_row, cond_k, cuda, f"{name} {out_dtype}")
    check_blend(out, ref, mag, plan.cfg.out_dtype)


@pytest.mark.parametrize("name", ALL)
def test_end_to_end_stand_in_denoiser(name, cuda):
    """extract -> y_t = a_t * x + b_t (torch, per tile) -> blend, on both sides."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    plan = plan_for(wl)
    _, _, bufs = gpu_extract(plan, inp, cuda, name)
    counts = bufs["tile_count"].cpu().numpy()
    views = tdp.tile_views(plan, bufs, counts)
    T = len(views)
    a, b = denoiser_params(wl.seed, T, wl.denoiser)
    tile_out = torch.empty_like(bufs["tile_lat"])
    out_views = tdp.tile_views(plan, {"tile_lat": tile_out, "tile_pos": bufs["tile_pos"],
                                      "tile_index": bufs["tile_index"]}, counts)
    for t in range(T):
        x = views[t]["lat"].float()
        out_views[t]["lat"].copy_(torch.add(torch.mul(x, float(a[t])), float(b[t])).to(tile_out.dtype))
    out = tdp.allocate_output(plan, cuda)
    note(f"blend e2e {name}")
    tdp.tdp_blend(plan, tile_out, bufs["cond_row"], bufs["cond_k"], out)
    torch.cuda.synchronize()

    ex = oracle_extract(wl, inp)
    ys = []
    for t, et in enumerate(ex["tiles"]):
        x = torch.from_numpy(oracle_tile_floats(et).astype(np.float32))
        y = torch.add(torch.mul(x, float(a[t])), float(b[t]))
        ys.append(y.to(torch.bfloat16).float().numpy() if wl.dtype == "bf16" else y.numpy())
    ref, mag = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    check_blend(out, ref, mag, plan.cfg.out_dtype)


@pytest.mark.parametrize("name", ["tiny", "ltx", "fullres", "4k", "conditioned"])
def test_identity_round_trip(name, cuda):
    """Extract then blend with y = x returns the input (bf16: exactly)."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    plan = plan_for(wl)
    lat, _, bufs = gpu_extract(plan, inp, cuda, name)
    out = tdp.allocate_output(plan, cuda)
    note(f"blend identity {name}")
    tdp.tdp_blend(plan, bufs["tile_lat"], bufs["cond_row"], bufs["cond_k"], out)
    torch.cuda.synchronize()
    if wl.dtype == "bf16":
        assert torch.equal(out.float(), lat.float())   # -0.0 may come back as +0.0
    else:
        torch.testing.assert_close(out, lat, rtol=0, atol=2e-6 * float(lat.abs().max()))


def test_deterministic_repeat(cuda):
    wl = WORKLOADS["conditioned"]
    inp = make_inputs(wl)
    plan = plan_for(wl)
    results = []
    for rep in range(2):
        _, _, bufs = gpu_extract(plan, inp, cuda, f"conditioned rep {rep}")
        out = tdp.allocate_output(plan, cuda)
        note(f"blend conditioned rep {rep}")
        tdp.tdp_blend(plan, bufs["tile_lat"], bufs["cond_row"], bufs["cond_k"], out)
        torch.cuda.synchronize()
        counts = bufs["tile_count"].cpu().numpy()
        views = tdp.tile_views(plan, bufs, counts)
        results.append((latent_bits(out), [latent_bits(v["lat"]) for v in views],
                        [v["pos"].cpu().numpy().tobytes() for v in views]))
    assert np.array_equal(results[0][0], results[1][0])
    for x, y in zip(results[0][1], results[1][1]):
        assert np.array_equal(x, y)
    assert results[0][2] == results[1][2]


@pytest.mark.parametrize("name", ["conditioned", "4k"])
def test_positions_not_normalized(name, cuda):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    plan = plan_for(wl, normalize=False)
    _, _, bufs = gpu_extract(plan, inp, cuda, f"{name} raw positions")
    check_extract(plan, bufs, oracle_extract(wl, inp, normalize=False), wl.num_cond)


# --- edge cases ---------------------------------------------------------------

def _custom_case(shape, tiling, batch=1, channels=128, dtype="bf16", num_cond=0, seed=0, random_pos=False):
    wl = Workload("custom", batch, channels, shape, tiling, num_cond=num_cond, num_ref=num_cond // 4,
                  dtype=dtype, seed=seed)
    inp = make_inputs(wl)
    if random_pos:
        rng = np.random.default_rng(seed + 1)
        N = wl.tokens
        start = rng.uniform(-40, 40, size=(batch, 3, N)).astype(np.float32)
        width = rng.uniform(0.25, 4, size=(batch, 3, N)).astype(np.float32)
        inp["pos"][:, :, :N, 0] = start
        inp["pos"][:, :, :N, 1] = start + width
    return wl, inp


EDGE = {
    "single_tile": dict(shape=(2, 5, 7), tiling=((1, 0), (1, 0), (1, 0))),
    "ragged_width": dict(shape=(3, 7, 37), tiling=((1, 0), (2, 2), (3, 9))),
    "max_tiles_axis": dict(shape=(2, 6, 70), tiling=((1, 0), (1, 0), (32, 1))),
    "w_one": dict(shape=(4, 9, 1), tiling=((2, 1), (3, 2), (1, 0))),
    "frame_tiles": dict(shape=(12, 6, 10), tiling=((3, 3), (2, 2), (2, 1))),
    "wide_channels": dict(shape=(2, 6, 20), tiling=((1, 0), (2, 2), (2, 3)), channels=512),
    "narrow_channels": dict(shape=(2, 6, 20), tiling=((1, 0), (2, 2), (2, 3)), channels=8),
    "odd_vectors": dict(shape=(2, 6, 20), tiling=((1, 0), (2, 2), (2, 3)), channels=48),
    "f32_channels": dict(shape=(3, 9, 13), tiling=((1, 0), (2, 3), (3, 3)), channels=36, dtype="f32"),
    "batch3_random_pos": dict(shape=(3, 8, 12), tiling=((2, 1), (2, 2), (2, 3)), batch=3, random_pos=True),
    "cond_random_pos": dict(shape=(4, 10, 12), tiling=((2, 1), (2, 3), (3, 3)), batch=2, num_cond=300,
                            random_pos=True),
    "wide_4096": dict(shape=(1, 2, 4096), tiling=((1, 0), (2, 0), (3, 512)), channels=16),
    # more than 256 tiles with conditioning: the blend's per-tile conditioning path
    "tiles272_cond": dict(shape=(1, 16, 17), tiling=((1, 0), (16, 0), (17, 0)), channels=16, num_cond=20, seed=6),
    # twelve selection chunks: kept tokens counted across chunks
    "many_cond": dict(shape=(2, 8, 12), tiling=((1, 0), (2, 2), (2, 3)), num_cond=3000, seed=7),
    # five selection workgroups per tile (4096 tokens each) and a ragged last
    # chunk: the kept tokens before a chunk come from earlier superchunks' totals
    "cond_16k": dict(shape=(2, 12, 20), tiling=((1, 0), (2, 2), (3, 3)), batch=2, num_cond=16484, seed=11),
    # a superchunk boundary with a one-token last chunk, odd batch
    "cond_4097_batch3": dict(shape=(3, 10, 14), tiling=((2, 1), (2, 2), (2, 3)), batch=3, num_cond=4097,
                             seed=12, random_pos=True),
    # rows too wide to load a whole chunk at once (512 channels): kept rows
    # are copied after the test; and with fp32 rows, batch 2
    "cond_wide_rows": dict(shape=(2, 6, 20), tiling=((1, 0), (2, 2), (2, 3)), channels=512, num_cond=300, seed=13),
    "cond_f32_batch2": dict(shape=(2, 8, 12), tiling=((1, 0), (2, 2), (2, 3)), batch=2, channels=36, dtype="f32",
                            num_cond=150, seed=14, random_pos=True),
    "batch64": dict(shape=(2, 4, 6), tiling=((1, 0), (2, 1), (2, 2)), batch=64, channels=16, seed=8),
    # more than eight latent workgroups per compute unit: one-pass position
    # workgroups (parts held in registers), width not a multiple of the
    # wave's rows, random positions; the second also tiles frames and batch
    "latent_bound_random_pos": dict(shape=(8, 64, 130), tiling=((1, 0), (3, 6), (4, 10)), random_pos=True, seed=9),
    "latent_bound_batch2_frames": dict(shape=(8, 40, 130), tiling=((2, 2), (2, 4), (3, 8)), batch=2,
                                       random_pos=True, seed=10),
}


@pytest.mark.parametrize("case", list(EDGE))
def test_edge_cases(case, cuda):
    kw = dict(EDGE[case])
    wl, inp = _custom_case(**kw)
    plan = plan_for(wl, out_dtype="f32")
    _, _, bufs = gpu_extract(plan, inp, cuda, case)
    ex = oracle_extract(wl, inp)
    check_extract(plan, bufs, ex, wl.num_cond)
    rng = np.random.default_rng(5)
    tiles = [random_tile_outputs(rng, wl.batch, len(et["rows"]), wl.channels, wl.dtype) for et in ex["tiles"]]
    buf = slot_buffer_from_tiles(plan, tiles, plan.cfg.in_dtype, rng)
    ys = [O.bf16_bits_to_f32(y) if y.dtype == np.uint16 else y for y in tiles]
    ref, mag = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    out = gpu_blend(plan, buf, bufs["cond_row"], bufs["cond_k"], cuda, case)
    check_blend(out, ref, mag, tdp.TDP_F32)


@pytest.mark.parametrize("polls", [0, 1])
@pytest.mark.parametrize("case", ["cond_16k", "many_cond", "cond_4097_batch3", "cond_random_pos"])
def test_lookback_counts_unpublished_chunks_itself(case, polls, cuda):
    """With a tiny poll limit a selection wave counts an earlier chunk from
    its tokens whenever that chunk's flag is not yet published: the same
    rows, counts and k as the oracle, bit for bit."""
    kw = dict(EDGE[case])
    wl, inp = _custom_case(**kw)
    plan = plan_for(wl)
    tdp.tdp_set_lookback_polls(polls)
    try:
        _, _, bufs = gpu_extract(plan, inp, cuda, f"{case} lookback polls={polls}")
    finally:
        tdp.tdp_set_lookback_polls(256)
    check_extract(plan, bufs, oracle_extract(wl, inp), wl.num_cond)


def test_cond_tokens_kept_by_no_tile(cuda):
    """Tokens outside every tile with non-negative time: k = 0, output 0."""
    shape, tiling = (4, 8, 8), ((1, 0), (2, 2), (2, 2))
    wl = Workload("k0", 1, 16, shape, tiling, num_cond=70, num_ref=0, dtype="bf16", seed=9)
    inp = make_inputs(wl)
    N = wl.tokens
    inp["pos"][:, :, N:, :] = grid_positions(1, (1, 1, 70), (1, 1, 1))[:, :, :, :]
    inp["pos"][:, 0, N:, :] += 1000.0      # far beyond the last frame
    inp["pos"][:, 1, N + 5, :] = (3.0, 3.0)  # and an empty interval
    plan = plan_for(wl, out_dtype="f32")
    _, _, bufs = gpu_extract(plan, inp, cuda, "k0")
    ex = oracle_extract(wl, inp)
    assert ex["k"].max() == 0
    check_extract(plan, bufs, ex, wl.num_cond)
    out = tdp.allocate_output(plan, cuda)
    note("blend k0")
    tdp.tdp_blend(plan, bufs["tile_lat"], bufs["cond_row"], bufs["cond_k"], out)
    torch.cuda.synchronize()
    assert torch.all(out[:, N:] == 0)


def test_mixed_dtypes(cuda):
    for in_dtype, out_dtype in [("f32", "bf16"), ("bf16", "f32")]:
        wl, inp = _custom_case(shape=(3, 10, 17), tiling=((1, 0), (2, 3), (3, 4)), dtype=in_dtype, channels=64)
        plan = plan_for(wl, out_dtype=out_dtype)
        ex = oracle_extract(wl, inp)
        rng = np.random.default_rng(8)
        tiles = [random_tile_outputs(rng, wl.batch, len(et["rows"]), wl.channels, wl.dtype) for et in ex["tiles"]]
        buf = slot_buffer_from_tiles(plan, tiles, plan.cfg.in_dtype, rng)
        ys = [O.bf16_bits_to_f32(y) if y.dtype == np.uint16 else y for y in tiles]
        ref, mag = O.blend(ys, ex, wl.shape, wl.tiling, 0)
        cond_row, cond_k = cond_tables(plan, ex, 0, cuda)
        out = gpu_blend(plan, buf, cond_row, cond_k, cuda, f"{in_dtype}->{out_dtype}")
        check_blend(out, ref, mag, plan.cfg.out_dtype)


def test_window_weights_bit_exact(cuda):
    """One-hot tile outputs expose each fp32 weight product (wF*wH)*wW."""
    wl = Workload("onehot", 1, 16, (6, 14, 21), ((2, 2), (3, 3), (3, 5)), dtype="f32", seed=3)
    inp = make_inputs(wl)
    plan = plan_for(wl, out_dtype="f32")
    ex = oracle_extract(wl, inp)
    tiles = [np.ones((1, len(et["rows"]), 16), np.float32) for et in ex["tiles"]]
    out = gpu_blend(plan, slot_buffer_from_tiles(plan, tiles, tdp.TDP_F32), *cond_tables(plan, ex, 0, cuda),
                    cuda, "onehot")
    got = out.cpu().numpy()[0, :, 0]
    # expected: fp32 sum over covering tiles of fl(fl(wF*wH)*wW) with plan windows
    want = np.zeros(wl.tokens, np.float32)
    wins = [[tdp.tdp_plan_window(plan, d, i) for i in range(wl.tiling[d][0])] for d in range(3)]
    F, H, W = wl.shape
    for et in ex["tiles"]:
        (i, j, k), (f0, h0, w0) = et["tile"]["grid"], et["tile"]["origin"]
        for r, n in enumerate(et["rows"]):
            f, h, w = n // (H * W), (n // W) % H, n % W
            wt = np.float32(np.float32(wins[0][i][f - f0] * wins[1][j][h - h0]) * wins[2][k][w - w0])
            want[n] = np.float32(want[n] + wt)
    assert np.array_equal(got, want)


def test_bf16_output_rounding_bit_exact(cuda):
    """One tile, no overlap: out = RNE_bf16(y) exactly, compared with the oracle's rounding."""
    rng = np.random.default_rng(21)
    C, W = 64, 64
    y = rng.standard_normal((1, W, C)).astype(np.float32)
    u = y.view(np.uint32)
    u[0, :8, :] = (u[0, :8, :] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exact ties
    u[0, 8, :] = np.arange(C, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)  # ties, both parities
    y[0, 9, :4] = [0.0, -0.0, 3.3895314e38, -3.3895314e38]                    # zeros, near overflow
    y[0, 10, :] = rng.standard_normal(C).astype(np.float32) * np.float32(1e-30)  # tiny normals
    wl = Workload("round", 1, C, (1, 1, W), ((1, 0), (1, 0), (1, 0)), dtype="f32", seed=0)
    plan = plan_for(wl, out_dtype="bf16")
    ex = O.extract(y, grid_positions(1, (1, 1, W), (1, 1, 1)), wl.shape, wl.tiling, 0)
    out = gpu_blend(plan, slot_buffer_from_tiles(plan, [y], tdp.TDP_F32), *cond_tables(plan, ex, 0, cuda),
                    cuda, "rounding")
    ref, _ = O.blend([y], ex, wl.shape, wl.tiling, 0)   # one term: exact in fp32 (-0.0 sums to +0.0)
    want = O.f32_to_bf16_bits(ref.astype(np.float32))
    got = latent_bits(out)
    bad = np.argwhere(got != want)
    assert len(bad) == 0, [(tuple(i), hex(int(y[tuple(i)].view(np.uint32))), hex(int(got[tuple(i)])),
                            hex(int(want[tuple(i)]))) for i in bad[:5]]


def _random_axis(rng, dim_max):
    while True:
        dim = int(rng.integers(1, dim_max + 1))
        n = int(rng.integers(1, min(dim, 5) + 1))
        o = 0 if n == 1 else int(rng.integers(0, dim // (n + 1) + 1))
        if dim - o >= n:
            return dim, (n, o)


@pytest.mark.parametrize("seed", range(24))
def test_random_configs(seed, cuda):
    """Seeded random guarded plans: random tilings on all three axes, batch,
    channel count, dtype, conditioning tokens and positions."""
    rng = np.random.default_rng(1000 + seed)
    axes = [_random_axis(rng, m) for m in (6, 14, 40)]
    shape = tuple(d for d, _ in axes)
    tiling = tuple(t for _, t in axes)
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    channels = int(rng.choice([4, 8, 12, 36]) if dtype == "f32" else rng.choice([8, 16, 24, 48, 128]))
    batch = int(rng.integers(1, 4))
    num_cond = int(rng.choice([0, 0, 5, 40, 300]))
    wl, inp = _custom_case(shape, tiling, batch=batch, channels=channels, dtype=dtype, num_cond=num_cond,
                           seed=seed, random_pos=bool(rng.random() < 0.5))
    normalize = bool(rng.random() < 0.7)
    label = f"seed {seed}: {shape} {tiling} B{batch} C{channels} {dtype} Nc{num_cond} normalize={normalize}"
    out_dtype = "bf16" if rng.random() < 0.5 else "f32"
    plan = plan_for(wl, out_dtype=out_dtype, normalize=normalize)
    _, _, bufs = gpu_extract(plan, inp, cuda, label)
    ex = oracle_extract(wl, inp, normalize=normalize)
    check_extract(plan, bufs, ex, wl.num_cond)
    tiles = [random_tile_outputs(rng, wl.batch, len(et["rows"]), wl.channels, wl.dtype) for et in ex["tiles"]]
    buf = slot_buffer_from_tiles(plan, tiles, plan.cfg.in_dtype, rng)
    ys = [O.bf16_bits_to_f32(y) if y.dtype == np.uint16 else y for y in tiles]
    ref, mag = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    out = gpu_blend(plan, buf, bufs["cond_row"], bufs["cond_k"], cuda, label)
    check_blend(out, ref, mag, plan.cfg.out_dtype)
