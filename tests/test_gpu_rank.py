"""GPU parity of rank plans: one rank's round-robin share of the tiles.

A rank plan's extract must reproduce the oracle's rows, positions, index
maps and counts bit for bit for the tiles the rank holds, and the selection
(cond_row, hence k) for every tile.  Its blend is the rank's full-size
partial buffer, compared with ``oracle.rank_partial`` at the blend
tolerances (fp32 output |gpu - ref| <= 2e-6 * sum|w*y|; bf16 adds
4e-3 * |ref|).  The fp32 partials of all ranks, added in rank order as an
all_reduce would, must match the oracle's whole blend at the fp32 bound.
"""
import numpy as np
import pytest
import torch

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp
from harness import POISON, check_blend, check_extract, gpu_extract, note, slot_buffer_from_tiles
from synth import WORKLOADS, Workload, make_inputs, random_tile_outputs
from test_gpu_parity import EDGE, _custom_case, _random_axis

pytestmark = pytest.mark.gpu


def rank_plan(wl, world, rank, out_dtype="f32", normalize=True):
    cfg = tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond, in_dtype=wl.dtype,
                          out_dtype=out_dtype, normalize=normalize)
    return tdp.tdp_plan_create_rank(cfg, world, rank)


def gpu_partial(plan, buf_np, cond_row, cond_k, device, label):
    if buf_np.dtype == np.uint16:
        y = torch.from_numpy(buf_np.view(np.int16)).view(torch.bfloat16).to(device)
    else:
        y = torch.from_numpy(buf_np).to(device)
    out = tdp.allocate_output(plan, device)
    out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32).fill_(POISON)
    note(f"rank blend {label}")
    tdp.tdp_blend(plan, y, cond_row, cond_k, out)
    torch.cuda.synchronize()
    return out


def run_all_ranks(wl, inp, world, device, seed, out_dtype="f32", normalize=True):
    """Every rank: extract checked bit for bit, partial checked against the
    oracle; returns the fp32 sum of the partials and the oracle's blend."""
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond, normalize=normalize)
    rng = np.random.default_rng(seed)
    tiles = [random_tile_outputs(rng, wl.batch, len(et["rows"]), wl.channels, wl.dtype) for et in ex["tiles"]]
    ys = [O.bf16_bits_to_f32(y) if y.dtype == np.uint16 else y for y in tiles]
    total = None
    for rank in range(world):
        label = f"{wl.name} world {world} rank {rank}"
        plan = rank_plan(wl, world, rank, out_dtype, normalize)
        _, _, bufs = gpu_extract(plan, inp, device, label)
        check_extract(plan, bufs, ex, wl.num_cond)
        buf = slot_buffer_from_tiles(plan, tiles, plan.cfg.in_dtype, rng)
        out = gpu_partial(plan, buf, bufs["cond_row"], bufs["cond_k"], device, label)
        ref, mag = O.rank_partial(ys, ex, wl.shape, wl.tiling, wl.num_cond, world, rank)
        check_blend(out, ref, mag, plan.cfg.out_dtype)
        if out.dtype == torch.float32:
            total = out.clone() if total is None else total.add_(out)
    full, mag = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    return total, full, mag


@pytest.mark.parametrize("name,world", [("tiny", 2), ("tiny", 3), ("ltx", 3), ("fullres", 4),
                                        ("conditioned", 2), ("conditioned", 4), ("conditioned", 7),
                                        ("4k", 4), ("4k", 5)])
def test_rank_shares_match_oracle(name, world, cuda):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    total, full, mag = run_all_ranks(wl, inp, world, cuda, seed=300 + world)
    check_blend(total, full, mag, tdp.TDP_F32)   # the all_reduce of the partials


@pytest.mark.parametrize("case,world", [("single_tile", 3), ("ragged_width", 4), ("max_tiles_axis", 7),
                                        ("w_one", 5), ("frame_tiles", 3), ("f32_channels", 2),
                                        ("batch3_random_pos", 3), ("cond_random_pos", 5),
                                        ("cond_random_pos", 16), ("tiles272_cond", 5), ("many_cond", 3),
                                        ("cond_4097_batch3", 4), ("cond_wide_rows", 3),
                                        ("wide_4096", 2), ("odd_vectors", 3)])
def test_rank_edge_cases(case, world, cuda):
    """Includes ranks that hold no tile (world above the tile count), plans
    above 256 tiles with conditioning, and ragged widths."""
    wl, inp = _custom_case(**EDGE[case])
    total, full, mag = run_all_ranks(wl, inp, world, cuda, seed=17)
    check_blend(total, full, mag, tdp.TDP_F32)


def test_rank_bf16_partials(cuda):
    wl = WORKLOADS["conditioned"]
    inp = make_inputs(wl)
    run_all_ranks(wl, inp, 3, cuda, seed=5, out_dtype="bf16")


def test_rank_positions_not_normalized(cuda):
    wl = WORKLOADS["conditioned"]
    inp = make_inputs(wl)
    run_all_ranks(wl, inp, 4, cuda, seed=6, normalize=False)


def test_rank_identity_all_reduce_returns_latent(cuda):
    """4K-class latent on 4 ranks with the identity in place of the denoiser:
    each rank blends its own extracted tiles; the sum of the fp32 partials
    is the input to within the fp32 bound."""
    wl = WORKLOADS["4k"]
    inp = make_inputs(wl)
    total = None
    for rank in range(4):
        plan = rank_plan(wl, 4, rank)
        lat, _, bufs = gpu_extract(plan, inp, cuda, f"4k identity rank {rank}")
        out = tdp.allocate_output(plan, cuda)
        note(f"rank blend identity 4k rank {rank}")
        tdp.tdp_blend(plan, bufs["tile_lat"], bufs["cond_row"], bufs["cond_k"], out)
        torch.cuda.synchronize()
        total = out.clone() if total is None else total.add_(out)
    x = lat.float()
    assert torch.all((total - x).abs() <= 2e-6 * x.abs() + 1e-30)


@pytest.mark.parametrize("seed", range(12))
def test_rank_random_configs(seed, cuda):
    rng = np.random.default_rng(2000 + seed)
    axes = [_random_axis(rng, m) for m in (6, 14, 40)]
    shape = tuple(d for d, _ in axes)
    tiling = tuple(t for _, t in axes)
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    channels = int(rng.choice([4, 8, 12, 36]) if dtype == "f32" else rng.choice([8, 16, 24, 48, 128]))
    batch = int(rng.integers(1, 4))
    num_cond = int(rng.choice([0, 0, 5, 40, 300]))
    wl, inp = _custom_case(shape, tiling, batch=batch, channels=channels, dtype=dtype, num_cond=num_cond,
                           seed=seed, random_pos=bool(rng.random() < 0.5))
    T = int(np.prod([n for n, _ in tiling]))
    world = int(rng.integers(2, max(3, T + 2)))
    print(f"seed {seed}: {shape} {tiling} B{batch} C{channels} {dtype} Nc{num_cond} world {world}", flush=True)
    total, full, mag = run_all_ranks(wl, inp, world, cuda, seed=seed)
    check_blend(total, full, mag, tdp.TDP_F32)
