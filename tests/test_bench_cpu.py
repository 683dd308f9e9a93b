"""bench.py's host-side pieces, on the CPU: the algorithmic byte counts the
metric divides by, the guard on the committed counter record, and the
one-GPU contract."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
import oracle as O
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _oracle_counts(wl):
    from synth import make_inputs
    inp = make_inputs(wl)
    ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
    return np.array([len(et["rows"]) for et in ex["tiles"]]), len(ex["tiles"])


def test_4k_compulsory_bytes():
    wl = WORKLOADS["4k"]
    counts, T = _oracle_counts(wl)
    ex, bl, S = bench.compulsory_bytes(wl, counts, T, 2, 2)
    # S = prod(dim + (n - 1) o) for a count-based split: 16 * 92 * 168
    assert S == 16 * (68 + 3 * 8) * (120 + 3 * 16) == 247296
    N, row = 16 * 68 * 120, 128 * 2
    assert ex == N * row + N * 24 + S * row + S * 24 + 4 * S + 4 * T
    assert bl == S * row + N * row
    assert (ex, bl) == (106788928, 96731136)


def test_4k_naive_bytes():
    # Per-tile gathers re-read the overlaps: 236.2 MB against 203.5 MB.
    wl = WORKLOADS["4k"]
    counts, T = _oracle_counts(wl)
    ex, bl, S = bench.compulsory_bytes(wl, counts, T, 2, 2)
    extra = bench.naive_bytes(wl, S, 2)
    assert extra == (247296 - 130560) * (256 + 24)
    assert round((ex + bl) / 1e6, 1) == 203.5 and round((ex + bl + extra) / 1e6, 1) == 236.2


def test_conditioned_counts_kept_rows():
    wl = WORKLOADS["conditioned"]
    counts, T = _oracle_counts(wl)
    ex, bl, S = bench.compulsory_bytes(wl, counts, T, 2, 2)
    gen = int(np.prod([d + (n - 1) * o for d, (n, o) in zip(wl.shape, wl.tiling)]))
    assert S > gen and S - gen >= 256 * T          # every reference token is kept by every tile
    rows, row = wl.tokens + wl.num_cond, wl.batch * wl.channels * 2
    sel = 4 * T * wl.num_cond + 4 * wl.num_cond
    assert bl == S * row + rows * row + sel


def test_latent_gather_bytes():
    # the per-latent gather reads the latent once and writes the tile rows:
    # at 4K the same bytes as the blend, which reads those rows and writes
    # the output
    wl = WORKLOADS["4k"]
    counts, T = _oracle_counts(wl)
    _, bl, S = bench.compulsory_bytes(wl, counts, T, 2, 2)
    assert bench.latent_bytes(wl, S, T, 2) == 130560 * 256 + 247296 * 256 == bl
    wl = WORKLOADS["conditioned"]
    counts, T = _oracle_counts(wl)
    S = int(sum(counts))
    rows, row = wl.tokens + wl.num_cond, wl.batch * wl.channels * 2
    assert bench.latent_bytes(wl, S, T, 2) == rows * row + S * row + 4 * T * wl.num_cond


def test_stream_bytes_formula():
    wl = WORKLOADS["4k"]
    S, B, C, rows = 247296, 1, 128, 130560
    got = bench.stream_bytes(wl, S, 2, 2)
    assert got == S * B * C * 2 + (2 * S - rows) * B * C * 4 + rows * B * C * (4 + 2)


def test_traffic_record_is_ignored_when_sources_change(monkeypatch):
    path = os.path.join(ROOT, bench.PMC_SUMMARY)
    rec = None
    for line in open(path):
        if line.strip().startswith("{") and '"traffic"' in line:
            rec = json.loads(line)
    assert rec is not None and rec["workload"] == "4k"
    monkeypatch.setattr(bench, "sources_hash", lambda: rec["sources_sha256_16"])
    for kernel in ("pipeline_kernel", "extract_kernel", "blend_kernel"):
        t = bench.measured_traffic("4k", kernel)
        assert t == rec["traffic"][kernel]["fetch_bytes"] + rec["traffic"][kernel]["write_bytes"]
    assert bench.measured_traffic("fullres", "pipeline_kernel") is None
    monkeypatch.setattr(bench, "sources_hash", lambda: "0" * 16)
    assert bench.measured_traffic("4k", "pipeline_kernel") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
