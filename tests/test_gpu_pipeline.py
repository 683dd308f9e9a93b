"""tdp_pipeline_step: the extract of one latent and the blend of another's
tile outputs as one step (one launch for whole plans without conditioning
tokens), through the C ABI.

Every output must equal, bit for bit, what tdp_extract and tdp_blend give
as two calls on the same inputs; the extract half is also held to the
oracle, and the blend half to the oracle's tolerance.  Covers fused plans
(bf16 and fp32 rows, bf16 and fp32 output, a tiled frame axis, ragged and
narrow rows), plans with conditioning tokens (two launches, every dtype
pairing), rank plans (one launch without conditioning tokens, two with
them), seeded random plans of both kinds, and a replayed graph of steps.
"""
import numpy as np
import pytest
import torch

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp
from harness import (check_blend, check_extract, note, oracle_tile_floats, plan_for, poisoned_buffers,
                     slot_buffer_from_tiles, to_device_latent)
from synth import WORKLOADS, Workload, make_inputs, random_tile_outputs

pytestmark = pytest.mark.gpu

OUT_KEYS = ("tile_lat", "tile_pos", "tile_index", "tile_count", "cond_row", "cond_k")


def _bits(t):
    t = t.detach().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def _case(name):
    if name in WORKLOADS:
        return WORKLOADS[name]
    custom = {
        "frame_tiles": Workload("frame_tiles", 1, 128, (12, 6, 10), ((3, 3), (2, 2), (2, 1)), seed=21),
        "f32_rows": Workload("f32_rows", 2, 36, (3, 9, 13), ((1, 0), (2, 3), (3, 3)), dtype="f32", seed=22),
        "odd_vectors": Workload("odd_vectors", 1, 48, (2, 6, 20), ((1, 0), (2, 2), (2, 3)), seed=23),
        "narrow_rows": Workload("narrow_rows", 1, 8, (2, 6, 20), ((1, 0), (2, 2), (2, 3)), seed=24),
        "wide_4096": Workload("wide_4096", 1, 16, (1, 2, 4096), ((1, 0), (2, 0), (3, 512)), seed=25),
        # conditioning tokens: few chunks per tile, many (look-back), fp32
        # rows, more than 256 tiles, rows too wide for one round of loads
        "many_cond": Workload("many_cond", 1, 128, (2, 8, 12), ((1, 0), (2, 2), (2, 3)), num_cond=3000, num_ref=750,
                              seed=26),
        "cond_f32": Workload("cond_f32", 2, 36, (2, 8, 12), ((1, 0), (2, 2), (2, 3)), num_cond=150, num_ref=37,
                             dtype="f32", seed=27),
        "tiles272_cond": Workload("tiles272_cond", 1, 16, (1, 16, 17), ((1, 0), (16, 0), (17, 0)), num_cond=20,
                                  num_ref=5, seed=28),
        "cond_wide_rows": Workload("cond_wide_rows", 1, 512, (2, 6, 20), ((1, 0), (2, 2), (2, 3)), num_cond=300,
                                   num_ref=75, seed=29),
    }
    return custom[name]


def _step_vs_two_calls(wl, cuda, out_dtype=None, world=1, rank=0):
    cfg = tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond, in_dtype=wl.dtype,
                          out_dtype=out_dtype or wl.dtype)
    plan = tdp.tdp_plan_create(cfg) if world == 1 else tdp.tdp_plan_create_rank(cfg, world, rank)
    inp_a = make_inputs(wl)                    # extracted by the step
    inp_b = make_inputs(wl, seed=wl.seed + 1)  # its tiles blended by the step
    lat_a, pos_a = to_device_latent(inp_a["latent"], cuda), torch.from_numpy(inp_a["pos"]).to(cuda)
    lat_b, pos_b = to_device_latent(inp_b["latent"], cuda), torch.from_numpy(inp_b["pos"]).to(cuda)
    # B: its extract (two calls' way) gives the tile outputs the step blends
    buf_b = poisoned_buffers(plan, cuda)
    note(f"pipeline {wl.name}: extract of the blended latent")
    tdp.tdp_extract(plan, lat_b, pos_b, **buf_b)
    # reference: the two calls
    ref_a = poisoned_buffers(plan, cuda)
    note(f"pipeline {wl.name}: extract + blend as two calls")
    tdp.tdp_extract(plan, lat_a, pos_a, **ref_a)
    ref_out = tdp.allocate_output(plan, cuda)
    tdp.tdp_blend(plan, buf_b["tile_lat"], buf_b["cond_row"], buf_b["cond_k"], ref_out)
    # the step
    got_a = poisoned_buffers(plan, cuda)
    got_out = tdp.allocate_output(plan, cuda)
    got_out.view(torch.int16 if got_out.dtype == torch.bfloat16 else torch.int32).fill_(-7)
    note(f"pipeline {wl.name}: tdp_pipeline_step")
    tdp.tdp_pipeline_step(plan, lat_a, pos_a, **got_a, tile_out=buf_b["tile_lat"], blend_cond_row=buf_b["cond_row"],
                          blend_cond_k=buf_b["cond_k"], out=got_out)
    torch.cuda.synchronize()
    for k in OUT_KEYS:
        assert np.array_equal(_bits(got_a[k]), _bits(ref_a[k])), f"{wl.name}: extract output {k} differs"
    assert np.array_equal(_bits(got_out), _bits(ref_out)), f"{wl.name}: blend output differs"
    return plan, inp_a, inp_b, got_a, got_out, buf_b


@pytest.mark.parametrize("name", ["tiny", "ltx", "fullres", "4k", "conditioned", "frame_tiles", "f32_rows",
                                  "odd_vectors", "narrow_rows", "wide_4096", "many_cond", "cond_f32",
                                  "tiles272_cond", "cond_wide_rows"])
def test_step_equals_extract_then_blend(name, cuda):
    wl = _case(name)
    plan, inp_a, _, got_a, _, _ = _step_vs_two_calls(wl, cuda)
    if wl.tokens * wl.batch <= 200_000:
        check_extract(plan, got_a, O.extract(inp_a["latent"], inp_a["pos"], wl.shape, wl.tiling, wl.num_cond),
                      wl.num_cond)


def test_step_fp32_output_and_oracle_blend(cuda):
    wl = WORKLOADS["ltx"]
    plan, _, inp_b, _, out, _ = _step_vs_two_calls(wl, cuda, out_dtype="f32")
    ex = O.extract(inp_b["latent"], inp_b["pos"], wl.shape, wl.tiling, wl.num_cond)
    ys = [oracle_tile_floats(et) for et in ex["tiles"]]
    ref, mag = O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
    check_blend(out, ref, mag, tdp.TDP_F32)


@pytest.mark.parametrize("world,rank", [(4, 1), (3, 0)])
def test_step_rank_plans(world, rank, cuda):
    _step_vs_two_calls(WORKLOADS["fullres"], cuda, out_dtype="f32", world=world, rank=rank)
    _step_vs_two_calls(WORKLOADS["conditioned"], cuda, out_dtype="f32", world=world, rank=rank)


@pytest.mark.parametrize("name,out_dtype", [("conditioned", "f32"), ("cond_f32", "bf16"), ("many_cond", "f32")])
def test_step_conditioned_mixed_dtypes(name, out_dtype, cuda):
    """Tiles and output of different dtypes with conditioning tokens (the
    fused conditioned step for each pairing)."""
    _step_vs_two_calls(_case(name), cuda, out_dtype=out_dtype)


def test_step_refuses_shared_buffers(cuda):
    wl = WORKLOADS["tiny"]
    plan = plan_for(wl)
    inp = make_inputs(wl)
    lat, pos = to_device_latent(inp["latent"], cuda), torch.from_numpy(inp["pos"]).to(cuda)
    bufs = poisoned_buffers(plan, cuda)
    out = tdp.allocate_output(plan, cuda)
    with pytest.raises(tdp.TdpError) as ei:   # blending the tiles this very step extracts
        tdp.tdp_pipeline_step(plan, lat, pos, **bufs, tile_out=bufs["tile_lat"], out=out)
    assert ei.value.status == tdp.TDP_EINVAL and "reads a buffer the extract writes" in str(ei.value)
    with pytest.raises(tdp.TdpError) as ei:   # writing into the latent the extract reads
        tdp.tdp_pipeline_step(plan, lat, pos, **bufs, tile_out=torch.empty_like(bufs["tile_lat"]),
                              out=lat.view(out.shape))
    assert ei.value.status == tdp.TDP_EINVAL and "writes a buffer the extract reads" in str(ei.value)


def test_step_graph_replays(cuda):
    """Four pipelined steps over four buffer sets captured once; every replay
    (with eager work in between) gives the eager result."""
    wl = WORKLOADS["fullres"]
    plan = plan_for(wl)
    R, D = 4, 2
    sets = []
    for r in range(R):
        inp = make_inputs(wl, seed=wl.seed + 10 + r)
        sets.append({"lat": to_device_latent(inp["latent"], cuda), "pos": torch.from_numpy(inp["pos"]).to(cuda),
                     "bufs": poisoned_buffers(plan, cuda), "out": tdp.allocate_output(plan, cuda)})
    stream = torch.cuda.Stream(cuda)

    def steps():
        for i in range(R, 2 * R):
            s, q = sets[i % R], sets[(i - D) % R]
            tdp.tdp_pipeline_step(plan, s["lat"], s["pos"], **s["bufs"], tile_out=q["bufs"]["tile_lat"],
                                  blend_cond_row=q["bufs"]["cond_row"], blend_cond_k=q["bufs"]["cond_k"],
                                  out=q["out"], stream=stream)
    with torch.cuda.stream(stream):
        for s in sets:
            tdp.tdp_extract(plan, s["lat"], s["pos"], stream=stream, **s["bufs"])
        note("pipeline graph: eager steps")
        steps()
    torch.cuda.synchronize()
    want = [(_bits(s["out"]), _bits(s["bufs"]["tile_lat"])) for s in sets]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        steps()
    for rep in range(3):
        for s in sets:
            s["out"].view(torch.int16).fill_(-7)
        torch.cuda.synchronize()
        note(f"pipeline graph: replay {rep}")
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        for (w_out, w_lat), s in zip(want, sets):
            assert np.array_equal(_bits(s["out"]), w_out), f"replay {rep}: blend output differs"
            assert np.array_equal(_bits(s["bufs"]["tile_lat"]), w_lat), f"replay {rep}: tile rows differ"


@pytest.mark.parametrize("seed", range(24))
def test_step_random_configs(seed, cuda):
    """Seeded random plans, whole and rank (up to 3 ranks): random tilings on
    all three axes, batch, channels, row and output dtypes, conditioning
    tokens, grid or random positions, normalization on or off.  The step
    extracts latent A and blends random tile outputs laid out on latent B's
    selection; it must equal the two calls bit for bit, its extract the
    oracle's, and its blend (a rank's partial for rank plans) the oracle's
    within tolerance."""
    from test_gpu_parity import _custom_case, _random_axis
    rng = np.random.default_rng(5000 + seed)
    axes = [_random_axis(rng, m) for m in (6, 14, 40)]
    shape = tuple(d for d, _ in axes)
    tiling = tuple(t for _, t in axes)
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    channels = int(rng.choice([4, 8, 12, 36]) if dtype == "f32" else rng.choice([8, 16, 24, 48, 128]))
    batch = int(rng.integers(1, 4))
    num_cond = int(rng.choice([0, 0, 5, 40, 300]))
    random_pos = bool(rng.random() < 0.5)
    normalize = bool(rng.random() < 0.7)
    out_dtype = "bf16" if rng.random() < 0.5 else "f32"
    world = int(rng.choice([1, 1, 2, 3]))
    rank = int(rng.integers(0, world))
    wl, inp_a = _custom_case(shape, tiling, batch=batch, channels=channels, dtype=dtype, num_cond=num_cond,
                             seed=seed, random_pos=random_pos)
    _, inp_b = _custom_case(shape, tiling, batch=batch, channels=channels, dtype=dtype, num_cond=num_cond,
                            seed=seed + 500, random_pos=random_pos)
    cfg = tdp.make_config(batch, channels, shape, tiling, num_cond, in_dtype=dtype, out_dtype=out_dtype,
                          normalize=normalize)
    plan = tdp.tdp_plan_create(cfg) if world == 1 else tdp.tdp_plan_create_rank(cfg, world, rank)
    label = (f"seed {seed}: {shape} {tiling} B{batch} C{channels} {dtype}->{out_dtype} Nc{num_cond} "
             f"world {world} rank {rank} normalize={normalize}")
    # B: its selection from the library's extract of its positions; its tile
    # outputs random, in the slot layout, unused slot rows garbage
    lat_b, pos_b = to_device_latent(inp_b["latent"], cuda), torch.from_numpy(inp_b["pos"]).to(cuda)
    buf_b = poisoned_buffers(plan, cuda)
    note(f"pipeline random {label}: extract of B")
    tdp.tdp_extract(plan, lat_b, pos_b, **buf_b)
    ex_b = O.extract(inp_b["latent"], inp_b["pos"], shape, tiling, num_cond, normalize=normalize)
    tiles = [random_tile_outputs(rng, batch, len(et["rows"]), channels, dtype) for et in ex_b["tiles"]]
    y_np = slot_buffer_from_tiles(plan, tiles, plan.cfg.in_dtype, rng)
    tile_out = to_device_latent(y_np, cuda) if y_np.dtype == np.uint16 else torch.from_numpy(y_np).to(cuda)
    lat_a, pos_a = to_device_latent(inp_a["latent"], cuda), torch.from_numpy(inp_a["pos"]).to(cuda)

    def poisoned_out():
        o = tdp.allocate_output(plan, cuda)
        o.view(torch.int16 if o.dtype == torch.bfloat16 else torch.int32).fill_(-7)
        return o
    ref_a, ref_out = poisoned_buffers(plan, cuda), poisoned_out()
    note(f"pipeline random {label}: two calls")
    tdp.tdp_extract(plan, lat_a, pos_a, **ref_a)
    tdp.tdp_blend(plan, tile_out, buf_b["cond_row"], buf_b["cond_k"], ref_out)
    got_a, got_out = poisoned_buffers(plan, cuda), poisoned_out()
    note(f"pipeline random {label}: tdp_pipeline_step")
    tdp.tdp_pipeline_step(plan, lat_a, pos_a, **got_a, tile_out=tile_out, blend_cond_row=buf_b["cond_row"],
                          blend_cond_k=buf_b["cond_k"], out=got_out)
    torch.cuda.synchronize()
    for k in OUT_KEYS:
        assert np.array_equal(_bits(got_a[k]), _bits(ref_a[k])), f"{label}: extract output {k} differs"
    assert np.array_equal(_bits(got_out), _bits(ref_out)), f"{label}: blend output differs"
    check_extract(plan, got_a, O.extract(inp_a["latent"], inp_a["pos"], shape, tiling, num_cond,
                                         normalize=normalize), num_cond)
    ys = [O.bf16_bits_to_f32(y) if y.dtype == np.uint16 else y for y in tiles]
    if world == 1:
        ref, mag = O.blend(ys, ex_b, shape, tiling, num_cond)
    else:
        ref, mag = O.rank_partial(ys, ex_b, shape, tiling, num_cond, world, rank)
    check_blend(got_out, ref, mag, plan.cfg.out_dtype)
