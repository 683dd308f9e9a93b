"""Seeded synthetic inputs shared by tests, smoke and bench (no method arithmetic)."""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    cond_positions,
    denoiser_params,
    grid_positions,
    make_inputs,
    random_tile_outputs,
    to_bf16_bits,
)
