"""Host side of the pixel-tile blend: plan geometry against the oracle, errors."""
import numpy as np
import pytest

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp

CONFIGS = [
    # B, C, frames, latent (H, W), scale, tiling, dtype
    (1, 3, 2, (6, 10), (8, 8), ((2, 2), (3, 2)), "bf16"),
    (2, 4, 1, (5, 7), (3, 4), ((1, 0), (2, 1)), "f32"),
    (1, 3, 1, (68, 120), (32, 32), ((4, 8), (4, 16)), "bf16"),
    (1, 1, 3, (9, 9), (16, 16), ((3, 2), (1, 0)), "bf16"),
    (1, 3, 1, (8, 100), (8, 8), ((1, 0), (7, 6)), "bf16"),
]


def make(cfg, out_dtype=None):
    B, C, Fo, hw, s, tiling, dt = cfg
    return tdp.tdp_pixel_plan_create(tdp.make_pixel_config(B, C, Fo, hw, s, tiling, in_dtype=dt, out_dtype=out_dtype))


@pytest.mark.parametrize("cfg", CONFIGS)
def test_pixel_plan_matches_oracle_geometry(cfg):
    B, C, Fo, hw, s, tiling, _ = cfg
    plan = make(cfg)
    ivs = [O.pixel_intervals(d, n, o, sc) for d, (n, o), sc in zip(hw, tiling, s)]
    tile_elems, out_elems, T = tdp.tdp_pixel_plan_sizes(plan)
    assert T == len(ivs[0]) * len(ivs[1])
    assert out_elems == B * C * Fo * hw[0] * s[0] * hw[1] * s[1]
    offset = 0
    for t in range(T):
        info = tdp.tdp_pixel_plan_tile(plan, t)
        i, j = divmod(t, len(ivs[1]))
        (y0, y1), (x0, x1) = ivs[0][i], ivs[1][j]
        assert (info.grid[0], info.grid[1]) == (i, j)
        assert (info.origin[0], info.origin[1], info.shape[0], info.shape[1]) == (y0, x0, y1 - y0, x1 - x0)
        assert info.offset == offset
        assert info.elems == B * C * Fo * (y1 - y0) * (x1 - x0)
        offset += info.elems
    assert offset == tile_elems


@pytest.mark.parametrize("kw,status", [
    (dict(scale_hw=(8, 4)), tdp.TDP_ESHAPE),                    # bf16 needs width scale % 8 == 0
    (dict(scale_hw=(0, 8)), tdp.TDP_EINVAL),
    (dict(tiling_hw=((3, 3), (2, 2))), tdp.TDP_EGUARD),         # 3 * 4 > 10
    (dict(tiling_hw=((1, 1), (2, 2))), tdp.TDP_EGUARD),         # one tile needs overlap 0
    (dict(frames=0), tdp.TDP_EINVAL),
])
def test_pixel_plan_errors(kw, status):
    args = dict(batch=1, channels=3, frames=1, latent_hw=(10, 12), scale_hw=(8, 8), tiling_hw=((2, 1), (2, 2)))
    args.update(kw)
    with pytest.raises(tdp.TdpError) as ei:
        tdp.tdp_pixel_plan_create(tdp.make_pixel_config(**args))
    assert ei.value.status == status


@pytest.mark.device_abi
def test_pixel_blend_rejects_bad_pointers():
    import ctypes
    plan = make(CONFIGS[0])
    lib = tdp.load_library()
    null = ctypes.c_void_p(None)
    assert lib.tdp_pixel_blend(plan.handle, null, null, null) == tdp.TDP_EINVAL
    assert lib.tdp_pixel_blend(plan.handle, ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1000), null) == tdp.TDP_EINVAL
    assert lib.tdp_pixel_blend(None, null, null, null) == tdp.TDP_EINVAL


@pytest.mark.device_abi
def test_pixel_blend_refuses_launches_past_32_bit_work_items():
    """1024 channels of 64 frames of 64 x 128 cells at 32 pixels per cell:
    2^27 output rows of 4096 pixels, 2^23 row groups times 8 column strips
    of 256 threads = 2^34 work-items, more than one launch counts; refused
    on the host before any launch."""
    import ctypes
    plan = tdp.tdp_pixel_plan_create(tdp.make_pixel_config(1, 1024, 64, (64, 128), (32, 32), ((2, 8), (2, 16))))
    lib = tdp.load_library()
    al = ctypes.c_void_p(1 << 40)
    assert lib.tdp_pixel_blend(plan.handle, al, ctypes.c_void_p(1 << 41), ctypes.c_void_p(None)) == tdp.TDP_ESHAPE
    assert "work-items" in tdp.tdp_last_error()
