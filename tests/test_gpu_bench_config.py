"""The pipelined step at full size, in the launch configuration bench.py times.

bench.py runs tdp_pipeline_step (``--step latent``: tdp_pipeline_latent_step
with the tables of one tdp_extract_positions call) over 8 rotating buffer
sets, the blend 4 steps behind the extract, with the K timed steps captured
in one HIP graph on a side stream and replayed.  Here 20 such steps run the
same way, from poisoned buffers and with no priming extract, so each set's
last blend reads tiles that an earlier step of the same graph wrote.  Every
set has a latent of its own (seeded), so a blend that read another set's
tiles, or ran before the extract it depends on, is seen.  After each of two
replays:
- every set's extract outputs match the oracle's extract of its latent bit
  for bit;
- every set's blended output matches the oracle's blend of those tiles
  within the blend tolerance, and, since the tile outputs are the extracted
  tiles themselves, equals its latent exactly (bf16).
"""
import numpy as np
import pytest
import torch

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp
from harness import check_blend, check_extract, note, plan_for, poisoned_buffers, to_device_latent
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

SETS, BEHIND, STEPS = 8, 4, 20


def _poisoned_output(plan, device):
    out = tdp.allocate_output(plan, device)
    out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32).fill_(-7)
    return out


@pytest.mark.parametrize("mode", ["full", "latent"])
@pytest.mark.parametrize("name", ["4k", "conditioned"])
def test_graph_of_pipelined_steps_matches_oracle(name, mode, cuda):
    wl = WORKLOADS[name]
    plan = plan_for(wl)
    pos_np = make_inputs(wl)["pos"]  # one positions set, as in bench.py
    pos = torch.from_numpy(pos_np).to(cuda)
    latents = [make_inputs(wl, seed=wl.seed + 100 + r)["latent"] for r in range(SETS)]
    sets = [{"latent": to_device_latent(latents[r], cuda), "bufs": poisoned_buffers(plan, cuda),
             "out": _poisoned_output(plan, cuda)} for r in range(SETS)]
    tables = None
    if mode == "latent":
        tables = poisoned_buffers(plan, cuda)
        note(f"bench configuration {name}: tdp_extract_positions")
        tdp.tdp_extract_positions(plan, pos, tables["tile_pos"], tables["tile_index"], tables["tile_count"],
                                  tables["cond_row"], tables["cond_k"], tables["workspace"])
        torch.cuda.synchronize()
    side = torch.cuda.Stream(cuda)

    def step(i):
        s, q = sets[i % SETS], sets[(i - BEHIND) % SETS]
        b = s["bufs"]
        if mode == "latent":
            tdp.tdp_pipeline_latent_step(plan, s["latent"], tables["cond_row"], b["tile_lat"],
                                         tile_out=q["bufs"]["tile_lat"], blend_cond_row=tables["cond_row"],
                                         blend_cond_k=tables["cond_k"], out=q["out"], stream=side)
        else:
            tdp.tdp_pipeline_step(plan, s["latent"], pos, b["tile_lat"], b["tile_pos"], b["tile_index"],
                                  b["tile_count"], b["cond_row"], b["cond_k"], b["workspace"],
                                  tile_out=q["bufs"]["tile_lat"], blend_cond_row=q["bufs"]["cond_row"],
                                  blend_cond_k=q["bufs"]["cond_k"], out=q["out"], stream=side)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    note(f"bench configuration {name} {mode}: capture {STEPS} steps")
    with torch.cuda.graph(graph, stream=side):
        for i in range(STEPS):
            step(i)
    refs = []
    for r in range(SETS):
        ex = O.extract(latents[r], pos_np, wl.shape, wl.tiling, wl.num_cond)
        ys = [O.bf16_bits_to_f32(et["latent"]) for et in ex["tiles"]]
        refs.append((ex, *O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)))
    for rep in range(2):
        note(f"bench configuration {name} {mode}: replay {rep}")
        with torch.cuda.stream(side):
            graph.replay()
        torch.cuda.synchronize()
        for r, s in enumerate(sets):
            ex, ref, mag = refs[r]
            got = dict(tables, tile_lat=s["bufs"]["tile_lat"]) if mode == "latent" else s["bufs"]
            check_extract(plan, got, ex, wl.num_cond)
            check_blend(s["out"], ref, mag, plan.cfg.out_dtype)
            assert torch.equal(s["out"].float(), s["latent"].float()), f"set {r}: blend is not the identity"
    del graph
