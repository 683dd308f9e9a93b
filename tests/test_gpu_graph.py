"""The device entry points under HIP graph capture.

They allocate nothing and issue no memset, so a captured extract + blend
(and a captured streaming blend) must replay to exactly the eager results.
The graph is replayed several times, with eager work and synchronizations
between the replays, and every replay is checked.
"""
import numpy as np
import pytest
import torch

import overlap_tiling_trapezoidal_amd as tdp
from harness import note, plan_for, to_device_latent
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).clone()


@pytest.mark.parametrize("name", ["conditioned", "fullres"])
def test_graph_replays_match_eager(name, cuda):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    plan = plan_for(wl)
    lat = to_device_latent(inp["latent"], cuda)
    pos = torch.from_numpy(inp["pos"]).to(cuda)
    bufs = tdp.allocate_extract_outputs(plan, cuda)
    out = tdp.allocate_output(plan, cuda)
    acc = tdp.allocate_accumulator(plan, cuda)
    out_s = tdp.allocate_output(plan, cuda)
    T = tdp.tdp_plan_num_tiles(plan)
    c = plan.cfg
    infos = [tdp.tdp_plan_tile(plan, t) for t in range(T)]
    s = torch.cuda.Stream(cuda)

    def step():
        tdp.tdp_extract(plan, lat, pos, bufs["tile_lat"], bufs["tile_pos"], bufs["tile_index"],
                        bufs["tile_count"], bufs["cond_row"], bufs["cond_k"], bufs["workspace"], s)
        tdp.tdp_blend(plan, bufs["tile_lat"], bufs["cond_row"], bufs["cond_k"], out, s)
        for t, inf in enumerate(infos):
            view = bufs["tile_lat"][inf.lat_offset: inf.lat_offset + c.batch * inf.capacity * c.channels]
            tdp.tdp_blend_tile(plan, t, view, bufs["cond_row"], bufs["cond_k"], acc, s)
        tdp.tdp_blend_finish(plan, acc, out_s, s)

    outputs = (out, out_s, acc, bufs["tile_lat"], bufs["tile_pos"], bufs["cond_row"], bufs["cond_k"],
               bufs["workspace"])

    def scramble():
        # slot rows past tile_count are never written: give them the same
        # bytes before the eager run and before every replay
        for t in outputs:
            t.view(torch.uint8).fill_(0x5A)

    note(f"graph eager {name}")
    scramble()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    ref = {k: _bits(v) for k, v in (("out", out), ("out_s", out_s), ("tile_lat", bufs["tile_lat"]),
                                    ("tile_pos", bufs["tile_pos"]), ("cond_row", bufs["cond_row"]),
                                    ("cond_k", bufs["cond_k"]))}
    assert torch.equal(ref["out"], ref["out_s"])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(3):
        # eager work between replays: scramble every output, then replay
        scramble()
        torch.cuda.synchronize()
        note(f"graph replay {name} #{rep}")
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for k, v in (("out", out), ("out_s", out_s), ("tile_lat", bufs["tile_lat"]),
                     ("tile_pos", bufs["tile_pos"]), ("cond_row", bufs["cond_row"]), ("cond_k", bufs["cond_k"])):
            assert torch.equal(_bits(v), ref[k]), (rep, k)


@pytest.mark.parametrize("world,rank", [(4, 1), (3, 2)])
def test_rank_plan_graph_replays_match_eager(world, rank, cuda):
    """A rank plan's extract and partial blend under capture, replayed
    three times with eager work in between, equal the eager run."""
    wl = WORKLOADS["conditioned"]
    inp = make_inputs(wl)
    cfg = tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond, in_dtype=wl.dtype,
                          out_dtype="f32")
    plan = tdp.tdp_plan_create_rank(cfg, world, rank)
    lat = to_device_latent(inp["latent"], cuda)
    pos = torch.from_numpy(inp["pos"]).to(cuda)
    bufs = tdp.allocate_extract_outputs(plan, cuda)
    out = tdp.allocate_output(plan, cuda)
    s = torch.cuda.Stream(cuda)

    def step():
        tdp.tdp_extract(plan, lat, pos, bufs["tile_lat"], bufs["tile_pos"], bufs["tile_index"],
                        bufs["tile_count"], bufs["cond_row"], bufs["cond_k"], bufs["workspace"], s)
        tdp.tdp_blend(plan, bufs["tile_lat"], bufs["cond_row"], bufs["cond_k"], out, s)

    outputs = (out, bufs["tile_lat"], bufs["tile_pos"], bufs["tile_index"], bufs["cond_row"], bufs["cond_k"])

    def scramble():
        for t in outputs:
            t.view(torch.uint8).fill_(0x5A)

    note(f"rank graph eager {world}/{rank}")
    scramble()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    ref = [_bits(v) for v in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(3):
        scramble()
        torch.cuda.synchronize()
        note(f"rank graph replay {world}/{rank} #{rep}")
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for i, v in enumerate(outputs):
            assert torch.equal(_bits(v), ref[i]), (rep, i)
