"""CPU oracle for the tiled extract/blend hot path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The product library never does; the two share
no code.  Parity unpinned: the remainder placement of ``split_by_count``.
"""
from .tdp_oracle import (  # noqa: F401
    AXES,
    bf16_bits_to_f32,
    blend,
    decoded_area_ratio,
    enumerate_tiles,
    extract,
    f32_to_bf16_bits,
    guard_holds,
    pixel_blend,
    pixel_intervals,
    rank_partial,
    round_robin_rank,
    split_by_count,
    tile_generated_tokens,
    tile_weights,
    tiling_quality,
    window_exact,
    window_f64,
    window_sums_exact,
)
