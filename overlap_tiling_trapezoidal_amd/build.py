"""Build libtdp.so (host planner + gfx950 kernels) in place with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtdp.so")
SOURCES = [os.path.join(HERE, "csrc", n) for n in (
    "plan.cpp", "quality.cpp", "pixel_plan.cpp", "kernels.hip", "pixel.hip")]
# memory-system ceilings for the measurement script (not the hot path)
CEILING_LIB = os.path.join(HERE, "libtdp_ceiling.so")
CEILING_SOURCES = [os.path.join(HERE, "csrc", "ceiling.hip")]

# the host planner alone, built with a host compiler under address and
# undefined-behaviour sanitizers (CPU tests only; no device entry points)
HOST_SAN_LIB = os.path.join(HERE, "libtdp_host_san.so")
HOST_SAN_SOURCES = [os.path.join(HERE, "csrc", n) for n in ("plan.cpp", "quality.cpp", "pixel_plan.cpp")]
HOST_SAN_FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all", "-fPIC", "-shared", "-Wall", "-I" + os.path.join(ROOT, "include")]

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


def build_host_sanitized(verbose: bool = False) -> str:
    """Build libtdp_host_san.so (host planner, ASan + UBSan) with g++."""
    tmp = HOST_SAN_LIB + ".tmp"
    cmd = [os.environ.get("CXX", "g++"), *HOST_SAN_FLAGS, *HOST_SAN_SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("g++ failed building libtdp_host_san.so")
    os.replace(tmp, HOST_SAN_LIB)
    return HOST_SAN_LIB


def host_sanitized_env(base=None) -> dict:
    """Environment for a Python process that loads libtdp_host_san.so: the
    address-sanitizer runtime preloaded ahead of the existing preload list,
    leak checks off (the interpreter never frees everything), stop at the
    first report (on stderr), and TDP_LIBRARY pointing at the build."""
    env = dict(os.environ if base is None else base)
    cxx = env.get("CXX", "g++")
    asan = subprocess.run([cxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not asan or not os.path.exists(asan):
        raise RuntimeError("the address-sanitizer runtime of the host compiler was not found")
    env["LD_PRELOAD"] = " ".join(x for x in (asan, env.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["TDP_LIBRARY"] = HOST_SAN_LIB
    return env


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv[1:]:
        print(build_host_sanitized(verbose=True))
    else:
        print(build(verbose=True))
