"""GPU parity of the streaming blend (tdp_blend_tile + tdp_blend_finish).

Tiles added one at a time, in index order, into an fp32 accumulator that
starts as NaN must give tdp_blend's output bit for bit (fp32 and bf16), and
so the oracle's blend within its tolerance.  Every comparison covers every
element; every input is seeded.
"""
import numpy as np
import pytest
import torch

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp
from harness import check_blend, cond_tables, gpu_blend, gpu_extract, note, plan_for, slot_buffer_from_tiles
from synth import WORKLOADS, Workload, make_inputs, random_tile_outputs

pytestmark = pytest.mark.gpu

EDGE = {
    "single_tile": Workload("single_tile", 1, 16, (2, 5, 7), ((1, 0), (1, 0), (1, 0)), dtype="bf16", seed=31),
    "frame_tiles": Workload("frame_tiles", 2, 24, (12, 6, 10), ((3, 3), (2, 2), (2, 1)), dtype="bf16", seed=32),
    "f32_ragged": Workload("f32_ragged", 1, 36, (3, 9, 13), ((1, 0), (2, 3), (3, 3)), dtype="f32", seed=33),
    "cond_frames": Workload("cond_frames", 2, 16, (6, 9, 10), ((2, 2), (2, 3), (2, 3)), num_cond=130, num_ref=20,
                            dtype="bf16", seed=34),
    "tiles272_cond": Workload("tiles272_cond", 1, 16, (1, 16, 17), ((1, 0), (16, 0), (17, 0)), num_cond=20,
                              num_ref=5, dtype="bf16", seed=35),
}
CASES = {**WORKLOADS, **EDGE}


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


def stream_blend(plan, y, cond_row, cond_k, device, separate=False, label=""):
    """Blend tile by tile; `separate` hands each tile over in its own buffer."""
    c = plan.cfg
    acc = tdp.allocate_accumulator(plan, device)
    acc.fill_(float("nan"))
    note(f"stream {label}")
    for t in range(tdp.tdp_plan_num_tiles(plan)):
        info = tdp.tdp_plan_tile(plan, t)
        view = y[info.lat_offset: info.lat_offset + c.batch * info.capacity * c.channels]
        tdp.tdp_blend_tile(plan, t, view.clone() if separate else view, cond_row, cond_k, acc)
    out = tdp.allocate_output(plan, device)
    out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32).fill_(-7)
    tdp.tdp_blend_finish(plan, acc, out)
    torch.cuda.synchronize()
    return acc, out


def _setup(wl, out_dtype, device):
    inp = make_inputs(wl)
    plan = plan_for(wl, out_dtype=out_dtype)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
    rng = np.random.default_rng(300 + wl.seed)
    tiles = [random_tile_outputs(rng, wl.batch, len(et["rows"]), wl.channels, wl.dtype) for et in ex["tiles"]]
    buf = slot_buffer_from_tiles(plan, tiles, plan.cfg.in_dtype, rng)
    ys = [O.bf16_bits_to_f32(y) if y.dtype == np.uint16 else y for y in tiles]
    ref, mag = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    cond_row, cond_k = cond_tables(plan, ex, wl.num_cond, device)
    if buf.dtype == np.uint16:
        y = torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).to(device)
    else:
        y = torch.from_numpy(buf).to(device)
    return plan, buf, y, cond_row, cond_k, ref, mag


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_stream_equals_blend_bit_exact(name, out_dtype, cuda):
    wl = CASES[name]
    plan, buf, y, cond_row, cond_k, ref, mag = _setup(wl, out_dtype, cuda)
    whole = gpu_blend(plan, buf, cond_row, cond_k, cuda, f"{name} {out_dtype}")
    acc, out = stream_blend(plan, y, cond_row, cond_k, cuda, label=f"{name} {out_dtype}")
    assert torch.equal(_bits(out), _bits(whole))
    check_blend(out, ref, mag, plan.cfg.out_dtype)
    if out_dtype == "f32":
        assert torch.equal(_bits(acc), _bits(whole))


@pytest.mark.parametrize("name", ["conditioned", "cond_frames", "tiny"])
def test_stream_separate_tile_buffers(name, cuda):
    wl = CASES[name]
    plan, buf, y, cond_row, cond_k, ref, mag = _setup(wl, "f32", cuda)
    _, joined = stream_blend(plan, y, cond_row, cond_k, cuda, label=f"{name} joined")
    _, apart = stream_blend(plan, y, cond_row, cond_k, cuda, separate=True, label=f"{name} separate")
    assert torch.equal(_bits(apart), _bits(joined))
    check_blend(apart, ref, mag, plan.cfg.out_dtype)


def test_stream_tokens_kept_by_no_tile(cuda):
    """Conditioning tokens that no tile keeps come out 0 from a NaN accumulator."""
    from synth import grid_positions
    wl = Workload("k0s", 1, 16, (4, 8, 8), ((1, 0), (2, 2), (2, 2)), num_cond=70, num_ref=0, dtype="bf16", seed=9)
    inp = make_inputs(wl)
    N = wl.tokens
    inp["pos"][:, :, N:, :] = grid_positions(1, (1, 1, 70), (1, 1, 1))[:, :, :, :]
    inp["pos"][:, 0, N:10 + N, :] += 1000.0   # first ten beyond the last frame: kept by none
    plan = plan_for(wl, out_dtype="f32")
    _, _, bufs = gpu_extract(plan, inp, cuda, "k0s")
    whole = tdp.allocate_output(plan, cuda)
    tdp.tdp_blend(plan, bufs["tile_lat"], bufs["cond_row"], bufs["cond_k"], whole)
    acc, out = stream_blend(plan, bufs["tile_lat"], bufs["cond_row"], bufs["cond_k"], cuda, label="k0s")
    assert torch.all(out[:, N:N + 10] == 0)
    assert torch.equal(_bits(out), _bits(whole))


@pytest.mark.parametrize("seed", range(10))
def test_stream_random_configs(seed, cuda):
    """Seeded random plans: streaming equals the fused blend bit for bit."""
    from test_gpu_parity import _random_axis
    rng = np.random.default_rng(2000 + seed)
    axes = [_random_axis(rng, m) for m in (5, 12, 30)]
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    wl = Workload(f"rand{seed}", int(rng.integers(1, 3)), int(rng.choice([8, 16, 24]) if dtype == "bf16" else 8),
                  tuple(d for d, _ in axes), tuple(t for _, t in axes), num_cond=int(rng.choice([0, 7, 64])),
                  num_ref=2, dtype=dtype, seed=3000 + seed)
    out_dtype = "bf16" if rng.random() < 0.5 else "f32"
    plan, buf, y, cond_row, cond_k, ref, mag = _setup(wl, out_dtype, cuda)
    whole = gpu_blend(plan, buf, cond_row, cond_k, cuda, f"rand {seed}")
    _, out = stream_blend(plan, y, cond_row, cond_k, cuda, label=f"rand {seed}")
    assert torch.equal(_bits(out), _bits(whole))
    check_blend(out, ref, mag, plan.cfg.out_dtype)
