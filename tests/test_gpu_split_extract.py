"""The extract in two halves, through the C ABI: tdp_extract_positions (once
per positions set) and tdp_extract_latent (per latent), and the pipelined
step tdp_pipeline_latent_step (latent gather + blend).

Every output must equal, bit for bit, what tdp_extract (and tdp_blend) give
on the same inputs, including for a second latent gathered with the tables
of the first positions call; small cases are also held to the oracle.
Covers whole plans with and without conditioning tokens (few chunks per
tile, look-back chunks, fp32 rows, more than 256 tiles, wide rows, 16 384
tokens), a tiled frame axis, ragged and narrow rows, rank plans, mixed
dtypes, the refusal of shared buffers and a replayed graph of steps; then
every edge case and the 24 seeded random plans of the extract parity tests.
"""
import numpy as np
import pytest
import torch

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp
from harness import check_blend, check_extract, note, oracle_tile_floats, poisoned_buffers, to_device_latent
from synth import WORKLOADS, Workload, make_inputs
from test_gpu_parity import EDGE as PARITY_EDGE
from test_gpu_parity import _custom_case as custom_case
from test_gpu_parity import _random_axis as random_axis

pytestmark = pytest.mark.gpu

OUT_KEYS = ("tile_lat", "tile_pos", "tile_index", "tile_count", "cond_row", "cond_k")

CASES = {
    "frame_tiles": Workload("frame_tiles", 1, 128, (12, 6, 10), ((3, 3), (2, 2), (2, 1)), seed=41),
    "f32_rows": Workload("f32_rows", 2, 36, (3, 9, 13), ((1, 0), (2, 3), (3, 3)), dtype="f32", seed=42),
    "odd_vectors": Workload("odd_vectors", 1, 48, (2, 6, 20), ((1, 0), (2, 2), (2, 3)), seed=43),
    "narrow_rows": Workload("narrow_rows", 1, 8, (2, 6, 20), ((1, 0), (2, 2), (2, 3)), seed=44),
    "many_cond": Workload("many_cond", 1, 128, (2, 8, 12), ((1, 0), (2, 2), (2, 3)), num_cond=3000, num_ref=750,
                          seed=45),
    "cond_f32": Workload("cond_f32", 2, 36, (2, 8, 12), ((1, 0), (2, 2), (2, 3)), num_cond=150, num_ref=37,
                         dtype="f32", seed=46),
    "tiles272_cond": Workload("tiles272_cond", 1, 16, (1, 16, 17), ((1, 0), (16, 0), (17, 0)), num_cond=20,
                              num_ref=5, seed=47),
    "cond_wide_rows": Workload("cond_wide_rows", 1, 512, (2, 6, 20), ((1, 0), (2, 2), (2, 3)), num_cond=300,
                               num_ref=75, seed=48),
    "cond_16384": Workload("cond_16384", 2, 128, (16, 32, 48), ((2, 2), (3, 6), (3, 8)), num_cond=16384,
                           num_ref=4096, seed=49),
}


def _case(name):
    return WORKLOADS[name] if name in WORKLOADS else CASES[name]


def _bits(t):
    t = t.detach().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def _plan(wl, out_dtype=None, world=1, rank=0):
    cfg = tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond, in_dtype=wl.dtype,
                          out_dtype=out_dtype or wl.dtype)
    return tdp.tdp_plan_create(cfg) if world == 1 else tdp.tdp_plan_create_rank(cfg, world, rank)


def _dev(inp, cuda):
    return to_device_latent(inp["latent"], cuda), torch.from_numpy(inp["pos"]).to(cuda)


def _halves(plan, lat, pos, bufs):
    tdp.tdp_extract_positions(plan, pos, bufs["tile_pos"], bufs["tile_index"], bufs["tile_count"], bufs["cond_row"],
                              bufs["cond_k"], bufs["workspace"])
    tdp.tdp_extract_latent(plan, lat, bufs["cond_row"], bufs["tile_lat"])


def _halves_vs_extract(wl, cuda, world=1, rank=0):
    plan = _plan(wl, world=world, rank=rank)
    inp = make_inputs(wl)
    lat, pos = _dev(inp, cuda)
    ref = poisoned_buffers(plan, cuda)
    note(f"split {wl.name} world {world} rank {rank}: tdp_extract")
    tdp.tdp_extract(plan, lat, pos, **ref)
    got = poisoned_buffers(plan, cuda)
    note(f"split {wl.name}: tdp_extract_positions + tdp_extract_latent")
    _halves(plan, lat, pos, got)
    torch.cuda.synchronize()
    for k in OUT_KEYS:
        assert np.array_equal(_bits(got[k]), _bits(ref[k])), f"{wl.name}: {k} differs from tdp_extract"
    # a second latent on the same positions: only the latent half runs again
    inp2 = make_inputs(wl, seed=wl.seed + 100)
    lat2 = to_device_latent(inp2["latent"], cuda)
    ref2 = poisoned_buffers(plan, cuda)
    note(f"split {wl.name}: second latent, tdp_extract and tdp_extract_latent")
    tdp.tdp_extract(plan, lat2, pos, **ref2)
    tdp.tdp_extract_latent(plan, lat2, got["cond_row"], got["tile_lat"])
    torch.cuda.synchronize()
    assert np.array_equal(_bits(got["tile_lat"]), _bits(ref2["tile_lat"])), f"{wl.name}: second latent differs"
    return plan, inp2["latent"], inp["pos"], got


@pytest.mark.parametrize("name", ["tiny", "ltx", "fullres", "4k", "conditioned", "frame_tiles", "f32_rows",
                                  "odd_vectors", "narrow_rows", "many_cond", "cond_f32", "tiles272_cond",
                                  "cond_wide_rows", "cond_16384"])
def test_positions_then_latent_equal_extract(name, cuda):
    wl = _case(name)
    plan, latent2, pos, got = _halves_vs_extract(wl, cuda)
    if wl.tokens * wl.batch <= 200_000 and wl.num_cond <= 4096:
        # the second latent's tiles with the first call's tables, against the oracle
        check_extract(plan, got, O.extract(latent2, pos, wl.shape, wl.tiling, wl.num_cond), wl.num_cond)


@pytest.mark.parametrize("world,rank", [(4, 1), (3, 0), (4, 3)])
@pytest.mark.parametrize("name", ["fullres", "conditioned", "many_cond"])
def test_rank_plans(name, world, rank, cuda):
    _halves_vs_extract(_case(name), cuda, world=world, rank=rank)


@pytest.mark.parametrize("name,world,rank", [("many_cond", 6, 5), ("fullres", 5, 4)])
def test_rank_without_tiles(name, world, rank, cuda):
    """A rank past the last tile holds none: the positions call still writes
    the selection tables (k counts every rank's tiles), and the gather and the
    latent step have nothing to copy."""
    wl = _case(name)
    plan = _plan(wl, world=world, rank=rank)
    assert tdp.held_tiles(plan) == []
    _halves_vs_extract(wl, cuda, world=world, rank=rank)
    _step_vs_two_calls(wl, cuda, out_dtype="f32", world=world, rank=rank)


def _step_vs_two_calls(wl, cuda, out_dtype=None, world=1, rank=0):
    plan = _plan(wl, out_dtype, world, rank)
    inp_a, inp_b = make_inputs(wl), make_inputs(wl, seed=wl.seed + 1)
    lat_a, pos = _dev(inp_a, cuda)
    lat_b = to_device_latent(inp_b["latent"], cuda)
    tables = poisoned_buffers(plan, cuda)
    note(f"latent step {wl.name}: positions")
    tdp.tdp_extract_positions(plan, pos, tables["tile_pos"], tables["tile_index"], tables["tile_count"],
                              tables["cond_row"], tables["cond_k"], tables["workspace"])
    tile_b = poisoned_buffers(plan, cuda)["tile_lat"]
    tdp.tdp_extract_latent(plan, lat_b, tables["cond_row"], tile_b)
    # reference: the two calls
    ref_lat = poisoned_buffers(plan, cuda)["tile_lat"]
    ref_out = tdp.allocate_output(plan, cuda)
    note(f"latent step {wl.name}: gather + blend as two calls")
    tdp.tdp_extract_latent(plan, lat_a, tables["cond_row"], ref_lat)
    tdp.tdp_blend(plan, tile_b, tables["cond_row"], tables["cond_k"], ref_out)
    got_lat = poisoned_buffers(plan, cuda)["tile_lat"]
    got_out = tdp.allocate_output(plan, cuda)
    got_out.view(torch.int16 if got_out.dtype == torch.bfloat16 else torch.int32).fill_(-7)
    note(f"latent step {wl.name}: tdp_pipeline_latent_step")
    tdp.tdp_pipeline_latent_step(plan, lat_a, tables["cond_row"], got_lat, tile_out=tile_b,
                                 blend_cond_row=tables["cond_row"], blend_cond_k=tables["cond_k"], out=got_out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(got_lat), _bits(ref_lat)), f"{wl.name}: gather half differs"
    assert np.array_equal(_bits(got_out), _bits(ref_out)), f"{wl.name}: blend half differs"
    return plan, {"latent": inp_b["latent"], "pos": inp_a["pos"]}, got_out


@pytest.mark.parametrize("name", ["tiny", "ltx", "fullres", "4k", "conditioned", "frame_tiles", "f32_rows",
                                  "odd_vectors", "narrow_rows", "many_cond", "cond_f32", "tiles272_cond",
                                  "cond_wide_rows"])
def test_latent_step_equals_two_calls(name, cuda):
    _step_vs_two_calls(_case(name), cuda)


@pytest.mark.parametrize("name", ["ltx", "conditioned"])
def test_latent_step_fp32_output_against_oracle(name, cuda):
    wl = WORKLOADS[name]
    plan, inp_b, out = _step_vs_two_calls(wl, cuda, out_dtype="f32")
    ex = O.extract(inp_b["latent"], inp_b["pos"], wl.shape, wl.tiling, wl.num_cond)
    ys = [oracle_tile_floats(et) for et in ex["tiles"]]
    ref, mag = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    check_blend(out, ref, mag, tdp.TDP_F32)


@pytest.mark.parametrize("world,rank", [(4, 1), (3, 0)])
def test_latent_step_rank_plans(world, rank, cuda):
    _step_vs_two_calls(WORKLOADS["fullres"], cuda, out_dtype="f32", world=world, rank=rank)
    _step_vs_two_calls(WORKLOADS["conditioned"], cuda, out_dtype="f32", world=world, rank=rank)


def test_latent_step_refuses_shared_buffers(cuda):
    wl = WORKLOADS["conditioned"]
    plan = _plan(wl)
    lat, pos = _dev(make_inputs(wl), cuda)
    bufs = poisoned_buffers(plan, cuda)
    out = tdp.allocate_output(plan, cuda)
    with pytest.raises(tdp.TdpError) as ei:   # blending the tiles this very step gathers
        tdp.tdp_pipeline_latent_step(plan, lat, bufs["cond_row"], bufs["tile_lat"], tile_out=bufs["tile_lat"],
                                     blend_cond_row=bufs["cond_row"], blend_cond_k=bufs["cond_k"], out=out)
    assert ei.value.status == tdp.TDP_EINVAL and "tile_lat, which the gather writes" in str(ei.value)
    with pytest.raises(tdp.TdpError) as ei:   # writing into the latent the gather reads
        tdp.tdp_pipeline_latent_step(plan, lat, bufs["cond_row"], bufs["tile_lat"],
                                     tile_out=torch.empty_like(bufs["tile_lat"]), blend_cond_row=bufs["cond_row"],
                                     blend_cond_k=bufs["cond_k"], out=lat.view(out.shape))
    assert ei.value.status == tdp.TDP_EINVAL and "writes a buffer the gather reads" in str(ei.value)


def test_latent_step_graph_replays(cuda):
    """Four pipelined steps over four latents sharing one positions set,
    captured once; every replay (with eager work in between) gives the
    eager result."""
    wl = WORKLOADS["conditioned"]
    plan = _plan(wl)
    R, D = 4, 2
    inp = make_inputs(wl)
    _, pos = _dev(inp, cuda)
    tables = poisoned_buffers(plan, cuda)
    tdp.tdp_extract_positions(plan, pos, tables["tile_pos"], tables["tile_index"], tables["tile_count"],
                              tables["cond_row"], tables["cond_k"], tables["workspace"])
    lats = [to_device_latent(make_inputs(wl, seed=wl.seed + 10 + r)["latent"], cuda) for r in range(R)]
    tiles = [poisoned_buffers(plan, cuda)["tile_lat"] for _ in range(R)]
    outs = [tdp.allocate_output(plan, cuda) for _ in range(R)]
    st = torch.cuda.Stream(cuda)
    for r in range(R):
        tdp.tdp_extract_latent(plan, lats[r], tables["cond_row"], tiles[r], stream=st)

    def step(i):
        q = (i - D) % R
        tdp.tdp_pipeline_latent_step(plan, lats[i % R], tables["cond_row"], tiles[i % R], tile_out=tiles[q],
                                     blend_cond_row=tables["cond_row"], blend_cond_k=tables["cond_k"], out=outs[q],
                                     stream=st)

    note("latent step graph: eager reference")
    with torch.cuda.stream(st):
        for i in range(R):
            step(i)
    torch.cuda.synchronize()
    ref_tiles, ref_outs = [_bits(t) for t in tiles], [_bits(o) for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for i in range(R):
            step(i)
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        note(f"latent step graph: replay {rep}")
        with torch.cuda.stream(st):
            g.replay()
        torch.cuda.synchronize()
        for r in range(R):
            assert np.array_equal(_bits(tiles[r]), ref_tiles[r]), f"replay {rep}: tile set {r}"
            assert np.array_equal(_bits(outs[r]), ref_outs[r]), f"replay {rep}: output {r}"


def _halves_equal_extract(plan, inp, cuda, label):
    """tdp_extract_positions + tdp_extract_latent against tdp_extract on the
    same inputs, every output bit for bit; returns the split buffers."""
    lat, pos = _dev(inp, cuda)
    ref = poisoned_buffers(plan, cuda)
    note(f"split {label}: tdp_extract")
    tdp.tdp_extract(plan, lat, pos, **ref)
    got = poisoned_buffers(plan, cuda)
    note(f"split {label}: tdp_extract_positions + tdp_extract_latent")
    _halves(plan, lat, pos, got)
    torch.cuda.synchronize()
    for k in OUT_KEYS:
        assert np.array_equal(_bits(got[k]), _bits(ref[k])), f"{label}: {k} differs from tdp_extract"
    return lat, got


@pytest.mark.parametrize("case", list(PARITY_EDGE))
def test_split_on_edge_cases(case, cuda):
    wl, inp = custom_case(**PARITY_EDGE[case])
    _halves_equal_extract(_plan(wl, out_dtype="f32"), inp, cuda, case)


@pytest.mark.parametrize("seed", range(24))
def test_split_random_configs(seed, cuda):
    """The seeded random plans of the extract parity tests (tilings, batch,
    channels, dtypes, conditioning tokens, positions, normalization): the
    two halves equal tdp_extract, and the latent step equals the gather and
    the blend as two calls."""
    rng = np.random.default_rng(1000 + seed)
    axes = [random_axis(rng, m) for m in (6, 14, 40)]
    shape = tuple(d for d, _ in axes)
    tiling = tuple(t for _, t in axes)
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    channels = int(rng.choice([4, 8, 12, 36]) if dtype == "f32" else rng.choice([8, 16, 24, 48, 128]))
    batch = int(rng.integers(1, 4))
    num_cond = int(rng.choice([0, 0, 5, 40, 300]))
    wl, inp = custom_case(shape, tiling, batch=batch, channels=channels, dtype=dtype, num_cond=num_cond,
                          seed=seed, random_pos=bool(rng.random() < 0.5))
    normalize = bool(rng.random() < 0.7)
    out_dtype = "bf16" if rng.random() < 0.5 else "f32"
    label = f"seed {seed}: {shape} {tiling} B{batch} C{channels} {dtype} Nc{num_cond} normalize={normalize}"
    cfg = tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond, in_dtype=wl.dtype,
                          out_dtype=out_dtype, normalize=normalize)
    plan = tdp.tdp_plan_create(cfg)
    lat, tables = _halves_equal_extract(plan, inp, cuda, label)
    # latent step: gather this latent, blend the first gather's tiles
    ref_lat = poisoned_buffers(plan, cuda)["tile_lat"]
    ref_out = tdp.allocate_output(plan, cuda)
    tdp.tdp_extract_latent(plan, lat, tables["cond_row"], ref_lat)
    tdp.tdp_blend(plan, tables["tile_lat"], tables["cond_row"], tables["cond_k"], ref_out)
    got_lat = poisoned_buffers(plan, cuda)["tile_lat"]
    got_out = tdp.allocate_output(plan, cuda)
    note(f"split {label}: tdp_pipeline_latent_step")
    tdp.tdp_pipeline_latent_step(plan, lat, tables["cond_row"], got_lat, tile_out=tables["tile_lat"],
                                 blend_cond_row=tables["cond_row"], blend_cond_k=tables["cond_k"], out=got_out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(got_lat), _bits(ref_lat)), f"{label}: gather half differs"
    assert np.array_equal(_bits(got_out), _bits(ref_out)), f"{label}: blend half differs"
