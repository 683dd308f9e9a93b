"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libtdp_host_san.so (plan.cpp, quality.cpp and pixel_plan.cpp with
g++ -fsanitize=address,undefined, stopping at the first report) and runs
the CPU tests in a child process that loads it through TDP_LIBRARY, with
the sanitizer runtime preloaded.  That build has no device entry points:
the tests of their host-side checks are skipped there and run against the
full library in the parent suite.
"""
import os
import subprocess
import sys

import pytest

import overlap_tiling_trapezoidal_amd as tdp
from overlap_tiling_trapezoidal_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(bool(os.environ.get("TDP_LIBRARY")), reason="already running on an override build")
def test_cpu_suite_clean_under_address_and_undefined_behaviour_sanitizers():
    lib = build.build_host_sanitized()
    env = build.host_sanitized_env()
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    probe = ("import overlap_tiling_trapezoidal_amd as t; t.load_library(); "
             "assert t.HOST_ONLY and t.LIB_PATH == %r; print('sanitized planner loaded')" % lib)
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "sanitized planner loaded" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    # -s: a report ends the process at once, so it must not sit in pytest's capture
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m", "not gpu", "-p", "no:cacheprovider",
           "--ignore", os.path.join(ROOT, "tests", "test_host_sanitizers.py"), os.path.join(ROOT, "tests")]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    for marker in ("runtime error", "AddressSanitizer"):
        i = out.find(marker)
        assert i < 0, out[max(0, i - 200): i + 4000]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout and " failed" not in r.stdout, r.stdout[-2000:]


def test_device_entry_list_matches_the_header():
    """The entry points a host-only build may lack are all declared ones."""
    assert set(tdp.DEVICE_FUNCTIONS) <= set(tdp.header_functions())
