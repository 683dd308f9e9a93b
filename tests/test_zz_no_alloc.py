"""tdp_extract_noalloc: the library's static per-GPU workspace in place of
the caller's.

GPU: two calls in a row through the C ABI, the second on a smaller plan, so
the second finds the first call's tables in the shared array; each call's
outputs must equal tdp_extract's (the same kernels with a caller workspace,
itself held to the oracle by the parity tests) bit for bit, and the second
is checked against the oracle as well.  A plan without conditioning tokens
(no workspace) follows.  CPU: a plan whose workspace exceeds the static
maximum is refused before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp
from harness import check_extract, note, plan_for, poisoned_buffers, to_device_latent
from synth import WORKLOADS, Workload, make_inputs

# workspace of 6912 bytes (16484 tokens), then 4096 (the conditioned
# workload), then none
CALLS = [
    ("cond_16k", Workload("cond_16k", 2, 128, (2, 12, 20), ((1, 0), (2, 2), (3, 3)), num_cond=16484,
                          num_ref=4121, dtype="bf16", seed=11)),
    ("conditioned", WORKLOADS["conditioned"]),
    ("fullres", WORKLOADS["fullres"]),
]

KEYS = ("tile_lat", "tile_pos", "tile_index", "tile_count", "cond_row", "cond_k")


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


@pytest.mark.gpu
def test_noalloc_matches_extract_on_successive_calls(cuda):
    sizes = [tdp.tdp_plan_sizes(plan_for(wl)).workspace_bytes for _, wl in CALLS]
    assert sizes[0] > sizes[1] > sizes[2] == 0 and sizes[0] <= tdp.TDP_STATIC_SCRATCH_BYTES
    for name, wl in CALLS:
        inp = make_inputs(wl)
        plan = plan_for(wl)
        lat = to_device_latent(inp["latent"], cuda)
        pos = torch.from_numpy(inp["pos"]).to(cuda)
        ref = poisoned_buffers(plan, cuda)
        note(f"extract {name} (caller workspace)")
        tdp.tdp_extract(plan, lat, pos, **ref)
        got = poisoned_buffers(plan, cuda)
        del got["workspace"]
        note(f"extract_noalloc {name} (static workspace)")
        tdp.tdp_extract_noalloc(plan, lat, pos, **got)
        torch.cuda.synchronize()
        for k in KEYS:
            assert np.array_equal(_bits(got[k]), _bits(ref[k])), f"{name}: {k} differs from tdp_extract"
        if name != "cond_16k":
            ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
            check_extract(plan, got, ex, wl.num_cond)


@pytest.mark.device_abi
def test_noalloc_refuses_plans_beyond_the_static_workspace():
    lib = tdp.load_library()
    wl = Workload("huge_cond", 1, 16, (1, 16, 16), ((1, 0), (4, 0), (4, 0)), num_cond=4_000_000, dtype="bf16")
    plan = plan_for(wl)
    assert tdp.tdp_plan_sizes(plan).workspace_bytes > tdp.TDP_STATIC_SCRATCH_BYTES
    al = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(None)
    #                               latent pos tile_lat tile_pos index count cond_row cond_k stream
    assert lib.tdp_extract_noalloc(plan.handle, al, al, al, al, al, al, al, al, null) == tdp.TDP_EINVAL
    assert "static" in tdp.tdp_last_error()
    # the shared checks come first
    assert lib.tdp_extract_noalloc(plan.handle, al, al, al, al, al, al, al, null, null) == tdp.TDP_EINVAL
    assert "cond_k" in tdp.tdp_last_error()
    assert lib.tdp_extract_noalloc(None, al, al, al, al, al, al, al, al, null) == tdp.TDP_EINVAL
