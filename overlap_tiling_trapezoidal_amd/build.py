"""Build libtdp.so (host planner + gfx950 kernels) in place with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtdp.so")
SOURCES = [os.path.join(HERE, "csrc", n) for n in ("plan.cpp", "quality.cpp", "kernels.hip", "pixel.hip")]
# memory-system ceilings for the measurement script (not the hot path)
CEILING_LIB = os.path.join(HERE, "libtdp_ceiling.so")
CEILING_SOURCES = [os.path.join(HERE, "csrc", "ceiling.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep fp32 division correctly rounded (window values must match the host plan)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(sources, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Build libtdp.so and libtdp_ceiling.so in place; returns libtdp.so's path."""
    _compile(SOURCES, LIB, verbose)
    _compile(CEILING_SOURCES, CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
