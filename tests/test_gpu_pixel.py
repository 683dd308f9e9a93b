"""GPU parity of the pixel-tile blend through the C ABI against the oracle.

Random tiles: fp32 output within 2e-6 * sum|w*y|, bf16 output within
4e-3 * |ref| more.  Tiles cut from one image must give it back bit for bit
in bf16.  Every element is compared; inputs are seeded.
"""
import numpy as np
import pytest
import torch

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp
from harness import note
from test_pixel_cabi import CONFIGS, make

pytestmark = pytest.mark.gpu


def _pack(plan, tiles, dt):
    tile_elems, _, _ = tdp.tdp_pixel_plan_sizes(plan)
    buf = np.empty(tile_elems, dtype=np.float32)
    for t, arr in enumerate(tiles):
        info = tdp.tdp_pixel_plan_tile(plan, t)
        buf[info.offset: info.offset + info.elems] = arr.reshape(-1)
    x = torch.from_numpy(buf)
    return x.to(torch.bfloat16) if dt == "bf16" else x


def _tiles_random(cfg, rng):
    B, C, Fo, hw, s, tiling, dt = cfg
    ivs = [O.pixel_intervals(d, n, o, sc) for d, (n, o), sc in zip(hw, tiling, s)]
    tiles = []
    for (y0, y1) in ivs[0]:
        for (x0, x1) in ivs[1]:
            a = rng.standard_normal((B, C, Fo, y1 - y0, x1 - x0)).astype(np.float32)
            if dt == "bf16":   # values the input dtype holds exactly
                a = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
            tiles.append(a)
    return tiles


@pytest.mark.parametrize("cfg", CONFIGS, ids=[f"{c[3]}x{c[4]}-{c[6]}" for c in CONFIGS])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_pixel_blend_random_tiles(cfg, out_dtype, cuda):
    B, C, Fo, hw, s, tiling, dt = cfg
    plan = make(cfg, out_dtype)
    rng = np.random.default_rng(hash((hw, s)) % 2**32)
    tiles = _tiles_random(cfg, rng)
    ref, mag = O.pixel_blend(tiles, hw, tiling, s)
    x = _pack(plan, tiles, dt).to(cuda)
    out = torch.full(ref.shape, float("nan"), device=cuda,
                     dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    note(f"pixel blend {hw} {s} {dt}->{out_dtype}")
    tdp.tdp_pixel_blend(plan, x, out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    tol = 2e-6 * mag + (4e-3 * np.abs(ref) if out_dtype == "bf16" else 0.0)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{bad.sum()} of {bad.size} elements out of tolerance"


@pytest.mark.parametrize("cfg", [c for c in CONFIGS if c[6] == "bf16"], ids=lambda c: f"{c[3]}x{c[4]}")
def test_pixel_blend_reassembles_image_bit_exact(cfg, cuda):
    B, C, Fo, hw, s, tiling, dt = cfg
    plan = make(cfg)
    rng = np.random.default_rng(7)
    img = torch.from_numpy(rng.standard_normal((B, C, Fo, hw[0] * s[0], hw[1] * s[1])).astype(np.float32))
    img = img.to(torch.bfloat16)
    ivs = [O.pixel_intervals(d, n, o, sc) for d, (n, o), sc in zip(hw, tiling, s)]
    tiles = [img[:, :, :, y0:y1, x0:x1].float().numpy() for (y0, y1) in ivs[0] for (x0, x1) in ivs[1]]
    x = _pack(plan, tiles, "bf16").to(cuda)
    out = torch.empty_like(img, device=cuda)
    note(f"pixel identity {hw} {s}")
    tdp.tdp_pixel_blend(plan, x, out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), img.view(torch.int16))


@pytest.mark.parametrize("seed", range(8))
def test_pixel_blend_random_configs(seed, cuda):
    from test_gpu_parity import _random_axis
    rng = np.random.default_rng(4000 + seed)
    (h, th), (w, tw) = _random_axis(rng, 10), _random_axis(rng, 14)
    dt = "f32" if rng.random() < 0.4 else "bf16"
    vec = 4 if dt == "f32" else 8
    cfg = (int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 3)), (h, w),
           (int(rng.integers(1, 6)), vec * int(rng.integers(1, 3))), (th, tw), dt)
    out_dtype = "bf16" if rng.random() < 0.5 else "f32"
    B, C, Fo, hw, s, tiling, _ = cfg
    plan = make(cfg, out_dtype)
    tiles = _tiles_random(cfg, rng)
    ref, mag = O.pixel_blend(tiles, hw, tiling, s)
    x = _pack(plan, tiles, dt).to(cuda)
    out = torch.full(ref.shape, float("nan"), device=cuda,
                     dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    note(f"pixel random {seed}: {cfg} -> {out_dtype}")
    tdp.tdp_pixel_blend(plan, x, out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    tol = 2e-6 * mag + (4e-3 * np.abs(ref) if out_dtype == "bf16" else 0.0)
    assert not (np.abs(got - ref) > tol).any()
