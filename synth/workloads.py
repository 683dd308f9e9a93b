"""Seeded synthetic workloads for the tiled extract/blend path.

This module only draws inputs: latents, token positions, conditioning-token
intervals and the parameters of a stand-in denoiser.  It holds none of the
tiling method's arithmetic (no split, window, selection or blend), so the
oracle and the GPU library can both be fed from it without sharing code.

The shapes follow the workloads the pages name: LTX-2's ~6k-token stage
(512x768x121 video) and ~24k-token full-resolution call (1024x1536x121),
from the LTX-2 docs, "Sequence Parallelism (SP)", "Usage"; a 4K-class latent
(2176x3840 px at 32x spatial / 8x temporal compression); and the
conditioned case of TDP docs, "Shared negative (reference) positions".
No dataset or trained weights are involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    channels: int
    shape: tuple            # (F, H, W) latent grid
    tiling: tuple           # ((n_f, o_f), (n_h, o_h), (n_w, o_w))
    num_cond: int = 0
    num_ref: int = 0        # leading conditioning tokens with negative time
    dtype: str = "bf16"     # latent storage dtype: "bf16" or "f32"
    pos_scale: tuple = (8, 32, 32)   # position units per latent cell
    denoiser: str = "affine"         # "identity" or "affine"
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        F, H, W = self.shape
        return F * H * W


WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, (3, 8, 8), ((1, 0), (2, 2), (2, 2)),
                     dtype="f32", pos_scale=(1, 1, 1), denoiser="identity", seed=0,
                     note="3x8x8 fp32, 2x2 spatial tiles, identity denoiser"),
    "ltx": Workload("ltx", 1, 128, (16, 16, 24), ((1, 0), (2, 4), (2, 4)), seed=1,
                    note="LTX-2 stage-2-like, 6144 tokens (512x768x121)"),
    "fullres": Workload("fullres", 1, 128, (16, 32, 48), ((1, 0), (2, 8), (2, 8)), seed=2,
                        note="full-res, 24576 tokens (1024x1536x121)"),
    "4k": Workload("4k", 1, 128, (16, 68, 120), ((1, 0), (4, 8), (4, 16)), seed=3,
                   note="4K-class, 130560 tokens, 16 tiles"),
    "conditioned": Workload("conditioned", 2, 128, (16, 32, 48), ((2, 2), (3, 6), (3, 8)),
                            num_cond=1024, num_ref=256, seed=4,
                            note="B=2 plus 1024 conditioning tokens, 256 with negative time"),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store float32 samples as bf16 (torch's CPU conversion, round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def grid_positions(batch: int, shape, scale) -> np.ndarray:
    """[start, end) positions of a (F, H, W) token grid: cell i spans [i*s, (i+1)*s)."""
    F, H, W = shape
    f, h, w = np.meshgrid(np.arange(F), np.arange(H), np.arange(W), indexing="ij")
    coords = [f.reshape(-1), h.reshape(-1), w.reshape(-1)]
    pos = np.empty((batch, 3, F * H * W, 2), dtype=np.float32)
    for d in range(3):
        pos[:, d, :, 0] = coords[d] * scale[d]
        pos[:, d, :, 1] = (coords[d] + 1) * scale[d]
    return pos


def cond_positions(rng, batch: int, shape, scale, num_cond: int, num_ref: int) -> np.ndarray:
    """Random [start, end) intervals for appended conditioning tokens.

    Per axis: start cell u ~ U{0..D-1}, length L ~ U{1..4} cells, clipped to
    the grid.  The first ``num_ref`` tokens get a negative time interval
    [-8j, -8(j-1)), j ~ U{1..4} (reference tokens).  Identical across batch.
    """
    pos = np.empty((3, num_cond, 2), dtype=np.float32)
    for d in range(3):
        D, s = shape[d], scale[d]
        u = rng.integers(0, D, size=num_cond)
        L = rng.integers(1, 5, size=num_cond)
        pos[d, :, 0] = u * s
        pos[d, :, 1] = np.minimum(u + L, D) * s
    j = rng.integers(1, 5, size=num_ref)
    pos[0, :num_ref, 0] = -8.0 * j
    pos[0, :num_ref, 1] = -8.0 * (j - 1)
    return np.broadcast_to(pos, (batch, 3, num_cond, 2)).copy()


def denoiser_params(seed: int, num_tiles: int, kind: str):
    """Per-tile stand-in denoiser y = a_t * x + b_t, a_t and b_t exact in fp32.

    Each tile draws from its own stream seeded (seed, t), after the port's
    per-tile generator seeded from the tile index (mold #673, "Scope").
    """
    if kind == "identity":
        return np.ones(num_tiles, np.float32), np.zeros(num_tiles, np.float32)
    a = np.empty(num_tiles, np.float32)
    b = np.empty(num_tiles, np.float32)
    for t in range(num_tiles):
        z = np.random.default_rng([seed, t]).standard_normal(2)
        a[t] = np.float32(1.0 + 0.25 * z[0])
        b[t] = np.float32(0.25 * z[1])
    return a, b


def make_inputs(wl: Workload, seed: int | None = None):
    """Latent (B, N+Nc, C) and positions (B, 3, N+Nc, 2) for a workload.

    The latent is N(0, 1) drawn in float32, stored as bf16 bits (uint16) or
    float32.  Returns a dict with ``latent`` and ``pos`` as numpy arrays.
    """
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    N, Nc, B, C = wl.tokens, wl.num_cond, wl.batch, wl.channels
    x = rng.standard_normal((B, N + Nc, C), dtype=np.float32)
    latent = to_bf16_bits(x) if wl.dtype == "bf16" else x
    pos = np.empty((B, 3, N + Nc, 2), dtype=np.float32)
    pos[:, :, :N, :] = grid_positions(B, wl.shape, wl.pos_scale)
    if Nc:
        pos[:, :, N:, :] = cond_positions(rng, B, wl.shape, wl.pos_scale, Nc, wl.num_ref)
    return {"latent": latent, "pos": pos}


def random_tile_outputs(rng, batch: int, rows: int, channels: int, dtype: str) -> np.ndarray:
    """N(0,1) rows standing in for a denoiser's output, stored like the latent."""
    y = rng.standard_normal((batch, rows, channels), dtype=np.float32)
    return to_bf16_bits(y) if dtype == "bf16" else y
