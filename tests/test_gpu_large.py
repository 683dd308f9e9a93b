"""Extract and blend with buffers past 2^31 16-byte vectors.

Every element offset the kernels form is 64-bit and every row index stays
within int32 by the planner's limits; this case checks that at a size where
an offset computed in 32 bits would wrap.  The latent is 17 x 512 x 4096
tokens of 512 bf16 channels (1 KiB rows, the widest row a plan takes): 34
GiB, 2.28e9 vectors; tiled (1, 2, 2) with overlaps (0, 16, 64), the tile
buffer holds 2.39e9 vectors.  About 110 GiB of device memory in all.

The latent is seeded N(0, 1) drawn on the device (the checks compare the
library's tile rows with the latent's own rows, so the oracle needs no copy
of it).  Checked against the oracle's tile geometry
(oracle.enumerate_tiles), every row:
- tile_count and tile_index bit for bit (each tile row's source token);
- tile_lat: each tile row equals the latent row it names;
- tile_pos: on grid positions the normalized positions are the source
  row's interval minus the tile origin times the cell size, exactly (the
  tile's minimum start; TDP docs, "Position normalization");
- the blend of the extracted tiles returns the latent exactly (identity
  round trip: the weights of a voxel sum to one in fp32 far inside half a
  bf16 ulp).
"""
import numpy as np
import pytest
import torch

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp
from harness import note
from synth import grid_positions

pytestmark = pytest.mark.gpu

SHAPE = (17, 512, 4096)
TILING = ((1, 0), (2, 16), (2, 64))
CHANNELS = 512
SCALE = (8, 32, 32)


def test_extract_blend_past_2_31_vectors(cuda):
    free, _ = torch.cuda.mem_get_info(cuda)
    if free < 130 << 30:
        pytest.skip(f"needs ~130 GiB of free device memory, {free >> 30} GiB free")
    plan = tdp.tdp_plan_create(tdp.make_config(1, CHANNELS, SHAPE, TILING))
    F, H, W = SHAPE
    N = F * H * W
    s = tdp.tdp_plan_sizes(plan)
    assert s.tile_lat_elems * 2 // 16 > 2 ** 31 and N * CHANNELS * 2 // 16 > 2 ** 31
    gen = torch.Generator(device=cuda)
    gen.manual_seed(77)
    lat = torch.randn((1, N, CHANNELS), generator=gen, device=cuda, dtype=torch.bfloat16)
    pos_np = grid_positions(1, SHAPE, SCALE)
    pos = torch.from_numpy(pos_np).to(cuda)
    bufs = tdp.allocate_extract_outputs(plan, cuda)
    note("large: tdp_extract, 34 GiB latent")
    tdp.tdp_extract(plan, lat, pos, **bufs)
    torch.cuda.synchronize()
    counts = bufs["tile_count"].cpu().numpy()
    tiles = O.enumerate_tiles(SHAPE, TILING)
    assert counts.tolist() == [int(np.prod(t["size"])) for t in tiles]
    views = tdp.tile_views(plan, bufs, counts)
    for t, v in zip(tiles, views):
        (f0, h0, w0), (sf, sh, sw) = t["origin"], t["size"]
        f = np.arange(f0, f0 + sf)[:, None, None]
        h = np.arange(h0, h0 + sh)[None, :, None]
        w = np.arange(w0, w0 + sw)[None, None, :]
        src = ((f * H + h) * W + w).reshape(-1)
        assert np.array_equal(v["index"].cpu().numpy(), src.astype(np.int32)), t["index"]
        idx = torch.from_numpy(src).to(cuda)
        assert torch.equal(v["lat"][0].view(torch.int16), lat[0].index_select(0, idx).view(torch.int16)), t["index"]
        shift = torch.tensor([t["origin"][d] * SCALE[d] for d in range(3)], dtype=torch.float32, device=cuda)
        want = pos[0].index_select(1, idx) - shift[:, None, None]
        assert torch.equal(v["pos"][0], want), t["index"]
        del idx, want
    out = tdp.allocate_output(plan, cuda)
    note("large: tdp_blend")
    tdp.tdp_blend(plan, bufs["tile_lat"], None, None, out)
    torch.cuda.synchronize()
    chunk = 1 << 22
    for r in range(0, N, chunk):   # -0.0 may come back as +0.0: compare values
        assert torch.equal(out[0, r:r + chunk].float(), lat[0, r:r + chunk].float()), r
    del lat, pos, bufs, out, views
    torch.cuda.empty_cache()
