"""Throughput of the tiled extract + blend hot path on one MI355X.

One step = one extract and one blend of the same synthetic latent's size
(all tiles, run locally; the per-tile denoiser is not part of the path and
is the identity here), enqueued as one tdp_pipeline_step: the extract of
one buffer set and the blend of another, one launch for whole plans without
conditioning tokens.  The same steps as two calls each (tdp_extract, then
tdp_blend) are reported beside it (``two_calls``).  Inputs are resident in
HBM before the timed region starts.  With ``--step latent`` a step is
instead one tdp_pipeline_latent_step: the latent gather of one set and the
blend of another, with the selection tables of one positions set made
before the timed region (latents that share their positions), rated on the
gather's and the blend's compulsory bytes.

Caches: the 4K working set (~204 MB) fits the 256 MB Infinity Cache, so a
loop over one buffer set would time cache hits.  The bench rotates over
``--sets`` independent buffer sets (default R = 8) and pipelines them: step
i extracts set i mod R and blends set (i - R/2) mod R.  Extract then reads a
latent last touched R steps earlier (~1.6 GB of traffic at 4K) and blend
reads tile rows written R/2 steps earlier (~0.8 GB, three times the cache),
so no launch finds its inputs in the cache.

Timed region: the K pipelined steps are captured once in a HIP graph (the
form a serving loop runs; the entry points allocate nothing and are safe to
capture), replayed once untimed, then replayed between two events.  The
same K steps launched eagerly from Python are reported beside it.

Prints one JSON line (stdout): GB/s of compulsory bytes (each input read
once, each output written once; overlap re-reads not credited), the
fraction of the 8 TB/s HBM peak, a roofline entry for the dominant kernel,
the CPU oracle's rate on the same workload, the same step measured on each
of the five workloads (``workloads``, with the extract in two halves for
latents that share one positions set: the per-latent gather and its
pipelined step), the conditioned shape's extract and per-latent gather with
1024 to 16384 conditioning tokens (``selection_scaling``) and what plain hand-written streaming
kernels move on this GPU (``ceilings``, from libtdp_ceiling.so), also with
the extract's and the blend's own read:write mix at their own sizes
(``same_mix_ceilings``: a scatter writing each byte it reads twice, a
gather reading two bytes per byte written; ``frac_of_same_mix``).

Roofline: the dominant kernel is the one launch of a step (pipeline_kernel)
when the step is fused, else the longer of extract_kernel and blend_kernel.
Its average duration comes from a CUDA-graph replay of back-to-back launches
(rotating buffer sets) between two HIP events on the launch stream, so host
launch overhead does not enter it.  `traffic` is the HBM bytes per launch
that rocprofv3's FETCH_SIZE and WRITE_SIZE counters read for that kernel,
each scaled by what the counter reads for a device copy of known size; the
figures live in profiles/pipeline_kernel_4k_pmc.md with a hash of the kernel
sources, and are reported only while the sources still match that hash.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
KERNEL_SOURCES = ("overlap_tiling_trapezoidal_amd/csrc/kernels.hip", "overlap_tiling_trapezoidal_amd/csrc/plan.cpp",
                  "overlap_tiling_trapezoidal_amd/csrc/plan_internal.h",
                  "overlap_tiling_trapezoidal_amd/csrc/device_common.h", "include/tdp.h")
PMC_SUMMARY = "profiles/pipeline_kernel_4k_pmc.md"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def compulsory_bytes(wl, counts, num_tiles, e_in, e_out):
    """Algorithmic bytes of one extract and one blend.

    S = sum of used tile rows (generated + kept conditioning).
    extract: latent read B*(N+Nc)*C*e + positions read B*(N+Nc)*24
             + tile rows written S*B*C*e + tile positions S*B*24 + index 4*S
             + counts / selection tables (4*T + 4*T*Nc + 4*Nc)
    blend:   tile rows read S*B*C*e + output written B*(N+Nc)*C*e_out
             + selection tables read (4*T*Nc + 4*Nc)
    """
    B, C, Nc = wl.batch, wl.channels, wl.num_cond
    rows = wl.tokens + Nc
    S = int(sum(counts))
    sel = 4 * num_tiles * Nc + 4 * Nc
    extract = B * rows * C * e_in + B * rows * 24 + S * B * C * e_in + S * B * 24 + 4 * S + 4 * num_tiles + sel
    blend = S * B * C * e_in + B * rows * C * e_out + sel
    return extract, blend, S


def latent_bytes(wl, S, num_tiles, e_in):
    """Algorithmic bytes of one latent gather (tdp_extract_latent) from
    selection tables made once per positions set: latent read
    B*(N+Nc)*C*e + tile rows written S*B*C*e + cond_row read 4*T*Nc."""
    B, C, Nc = wl.batch, wl.channels, wl.num_cond
    return B * (wl.tokens + Nc) * C * e_in + S * B * C * e_in + 4 * num_tiles * Nc


def naive_bytes(wl, S, e_in):
    """Bytes a per-tile gather moves on top of the compulsory ones: every
    tile re-reads its own latent rows and positions, overlaps included."""
    rows = wl.tokens + wl.num_cond
    return (S - rows) * wl.batch * (wl.channels * e_in + 24)


def rank_share_rate(torch, tdp, dev, sets, wl, world, rank, reps):
    """One rank's round-robin share: extract of its tiles and its full-size
    fp32 partial buffer (the all_reduce input), on the rotating input sets.
    Algorithmic bytes: extract reads the latent rows and positions the
    rank's tiles cover (each once) and writes its tile rows, positions and
    index map; blend reads its tile rows and writes the whole fp32 buffer."""
    import numpy as np
    cfg = tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond,
                          in_dtype=wl.dtype, out_dtype="f32")
    plan = tdp.tdp_plan_create_rank(cfg, world, rank)
    held = tdp.held_tiles(plan)
    cover = np.zeros(wl.shape, dtype=bool)
    S_r = 0
    for t in held:
        inf = tdp.tdp_plan_tile(plan, t)
        (f0, h0, w0), (sf, sh, sw) = tuple(inf.origin), tuple(inf.shape)
        cover[f0:f0 + sf, h0:h0 + sh, w0:w0 + sw] = True
        S_r += inf.gen_tokens
    assert wl.num_cond == 0, "the rank-share figure is taken on workloads without conditioning"
    e_in = 2 if wl.dtype == "bf16" else 4
    B, C = wl.batch, wl.channels
    U = int(cover.sum())
    ex_bytes = U * B * (C * e_in + 24) + S_r * B * (C * e_in + 24) + 4 * S_r + 4 * len(held)
    bl_bytes = S_r * B * C * e_in + B * wl.tokens * C * 4
    rs = [{"bufs": tdp.allocate_extract_outputs(plan, dev), "out": tdp.allocate_output(plan, dev)}
          for _ in range(len(sets))]
    gstream = torch.cuda.Stream(dev)

    def ex(i):
        s, b = sets[i % len(sets)], rs[i % len(sets)]["bufs"]
        tdp.tdp_extract(plan, s["latent"], s["pos"], b["tile_lat"], b["tile_pos"], b["tile_index"],
                        b["tile_count"], b["cond_row"], b["cond_k"], b["workspace"], gstream)

    def bl(i):
        r = rs[i % len(sets)]
        tdp.tdp_blend(plan, r["bufs"]["tile_lat"], r["bufs"]["cond_row"], r["bufs"]["cond_k"], r["out"], gstream)

    n = len(sets)

    def step_fn(i):  # the rank's pipelined step: extract set i, partial blend of set i - n/2
        s, b, q = sets[i % n], rs[i % n]["bufs"], rs[(i - n // 2) % n]
        tdp.tdp_pipeline_step(plan, s["latent"], s["pos"], b["tile_lat"], b["tile_pos"], b["tile_index"],
                              b["tile_count"], b["cond_row"], b["cond_k"], b["workspace"],
                              tile_out=q["bufs"]["tile_lat"], out=q["out"], stream=gstream)

    ex_ms = graph_time_ms(torch, gstream, ex, reps)
    bl_ms = graph_time_ms(torch, gstream, bl, reps)
    st_ms = graph_time_ms(torch, gstream, step_fn, reps)
    step = ex_ms + bl_ms
    return {"world": world, "rank": rank, "tiles": held, "tile_rows": S_r, "covered_rows": U,
            "step_ms": round(st_ms, 5), "step_gbs": round((ex_bytes + bl_bytes) / (st_ms * 1e-3) / 1e9, 1),
            "extract_ms": round(ex_ms, 5), "extract_bytes": ex_bytes,
            "extract_gbs": round(ex_bytes / (ex_ms * 1e-3) / 1e9, 1),
            "partial_blend_ms": round(bl_ms, 5), "partial_blend_bytes": bl_bytes,
            "partial_blend_gbs": round(bl_bytes / (bl_ms * 1e-3) / 1e9, 1),
            "gbs": round((ex_bytes + bl_bytes) / (step * 1e-3) / 1e9, 1),
            "note": "partial buffer in fp32 over the whole latent; the all_reduce itself is not run; "
                    "gbs: extract and partial blend as separate launches, step_gbs: the rank's "
                    "tdp_pipeline_step (one launch)"}


def stream_bytes(wl, S, e_in, e_out):
    """Algorithmic bytes of the streaming blend of all tiles plus the rounding:
    tile rows read once, the fp32 accumulator written for every tile row and
    read for every row but a voxel's first, then read once and rounded."""
    B, C = wl.batch, wl.channels
    rows = wl.tokens + wl.num_cond
    tiles = S * B * C * e_in
    acc = S * B * C * 4 + (S - rows) * B * C * 4
    finish = rows * B * C * 4 + rows * B * C * e_out
    return tiles + acc + finish


def pixel_rate(torch, tdp, dev, stream, sets=2, reps=8):
    """Blend of decoded pixel tiles for a 4K frame sequence: 8 RGB frames of
    2176 x 3840 bf16 from the 16-tile 4K latent tiling at 32 pixels per cell.
    Algorithmic bytes: every tile read once plus the output written once.
    The best of three graph-timed passes (the first in a process runs slower)."""
    cfg = tdp.make_pixel_config(1, 3, 8, (68, 120), (32, 32), ((4, 8), (4, 16)), in_dtype="bf16")
    plan = tdp.tdp_pixel_plan_create(cfg)
    tile_elems, out_elems, T = tdp.tdp_pixel_plan_sizes(plan)
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    bufs = [(torch.randn(tile_elems, device=dev, generator=g).to(torch.bfloat16),
             torch.empty(out_elems, device=dev, dtype=torch.bfloat16)) for _ in range(sets)]

    def run(i):
        x, out = bufs[i % sets]
        tdp.tdp_pixel_blend(plan, x, out, stream)

    ms = min(graph_time_ms(torch, stream, run, reps) for _ in range(3))
    nbytes = 2 * (tile_elems + out_elems)
    return {"workload": "8 frames RGB 2176x3840 bf16, 16 tiles (4x4), overlap 256/512 px", "tiles": T,
            "ms": round(ms, 4), "bytes": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def sources_hash():
    """First 16 hex digits of the SHA-256 over the kernel sources, in order."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when there is none for this workload or the sources changed."""
    path = os.path.join(ROOT, PMC_SUMMARY)
    if not os.path.exists(path):
        return None
    for line in open(path):
        line = line.strip()
        if line.startswith("{") and '"traffic"' in line:
            rec = json.loads(line)
            if rec.get("sources_sha256_16") != sources_hash() or rec.get("workload") != workload:
                return None
            t = rec["traffic"].get(kernel)
            return None if t is None else int(t["fetch_bytes"] + t["write_bytes"])
    return None


def graph_time_ms(torch, stream, fn, reps):
    """Average duration of fn(i) over `reps` back-to-back launches, from a
    CUDA-graph replay bracketed by two events on `stream`."""
    with torch.cuda.stream(stream):
        for i in range(reps):
            fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def workload_rates(torch, tdp, dev, wl, sets_n=8, steps=64):
    """Extract, blend and pipelined step (tdp_pipeline_step) of one workload,
    each timed as a graph replay of `steps` launches over `sets_n` rotating
    buffer sets (the blend `sets_n // 2` steps behind the extract), with the
    GB/s of its compulsory bytes.  Also the extract in two halves for
    latents that share one positions set: tdp_extract_positions (once per
    set), the per-latent gather tdp_extract_latent, and the pipelined step
    tdp_pipeline_latent_step (gather + blend), with the gather's own
    compulsory bytes."""
    import numpy as np
    from synth import make_inputs
    inp = make_inputs(wl)
    cfg = tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond,
                          in_dtype=wl.dtype, out_dtype=wl.dtype)
    plan = tdp.tdp_plan_create(cfg)
    T = tdp.tdp_plan_num_tiles(plan)

    def to_dev(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) if x.dtype == np.uint16 \
            else torch.from_numpy(x).to(dev)

    sets = [{"latent": to_dev(inp["latent"]), "pos": torch.from_numpy(inp["pos"]).to(dev),
             "bufs": tdp.allocate_extract_outputs(plan, dev), "out": tdp.allocate_output(plan, dev)}
            for _ in range(sets_n)]
    stream = torch.cuda.Stream(dev)
    lag = sets_n // 2

    def ex(i):
        s = sets[i % sets_n]
        tdp.tdp_extract(plan, s["latent"], s["pos"], stream=stream, **s["bufs"])

    def bl(i):
        s = sets[i % sets_n]
        b = s["bufs"]
        tdp.tdp_blend(plan, b["tile_lat"], b["cond_row"], b["cond_k"], s["out"], stream)

    def step(i):
        s, q = sets[i % sets_n], sets[(i - lag) % sets_n]
        tdp.tdp_pipeline_step(plan, s["latent"], s["pos"], stream=stream, **s["bufs"], tile_out=q["bufs"]["tile_lat"],
                              blend_cond_row=q["bufs"]["cond_row"], blend_cond_k=q["bufs"]["cond_k"], out=q["out"])

    # the two halves: every set has the same positions, so set 0's tables
    # (written by its extract) serve every latent
    tab = sets[0]["bufs"]

    def positions(i):
        b = sets[i % sets_n]["bufs"]
        tdp.tdp_extract_positions(plan, sets[i % sets_n]["pos"], b["tile_pos"], b["tile_index"], b["tile_count"],
                                  b["cond_row"], b["cond_k"], b["workspace"], stream=stream)

    def gather(i):
        s = sets[i % sets_n]
        tdp.tdp_extract_latent(plan, s["latent"], tab["cond_row"], s["bufs"]["tile_lat"], stream=stream)

    def latent_step(i):
        s, q = sets[i % sets_n], sets[(i - lag) % sets_n]
        tdp.tdp_pipeline_latent_step(plan, s["latent"], tab["cond_row"], s["bufs"]["tile_lat"],
                                     tile_out=q["bufs"]["tile_lat"], blend_cond_row=tab["cond_row"],
                                     blend_cond_k=tab["cond_k"], out=q["out"], stream=stream)

    with torch.cuda.stream(stream):
        for i in range(sets_n):
            ex(i)
    torch.cuda.synchronize()
    counts = sets[0]["bufs"]["tile_count"].cpu().numpy()
    e = 2 if wl.dtype == "bf16" else 4
    ex_b, bl_b, S = compulsory_bytes(wl, counts, T, e, e)
    ex_ms = graph_time_ms(torch, stream, ex, steps)
    bl_ms = graph_time_ms(torch, stream, bl, steps)
    st_ms = graph_time_ms(torch, stream, step, steps)
    gbs = (ex_b + bl_b) / (st_ms * 1e-3) / 1e9
    pos_ms = graph_time_ms(torch, stream, positions, steps)
    ga_ms = graph_time_ms(torch, stream, gather, steps)
    ls_ms = graph_time_ms(torch, stream, latent_step, steps)
    ga_b = latent_bytes(wl, S, T, e)
    return {
        "config": f"B={wl.batch} C={wl.channels} (F,H,W)={wl.shape} {wl.dtype}, tiles "
                  f"{tuple(n for n, _ in wl.tiling)} overlap {tuple(o for _, o in wl.tiling)}, {T} tiles, "
                  f"{wl.num_cond} conditioning tokens",
        "tile_rows": S,
        "extract_us": round(ex_ms * 1e3, 3), "extract_bytes": ex_b,
        "extract_gbs": round(ex_b / (ex_ms * 1e-3) / 1e9, 1),
        "blend_us": round(bl_ms * 1e3, 3), "blend_bytes": bl_b,
        "blend_gbs": round(bl_b / (bl_ms * 1e-3) / 1e9, 1),
        "step_us": round(st_ms * 1e3, 3), "bytes_per_step": ex_b + bl_b,
        "gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "positions_us": round(pos_ms * 1e3, 3),
        "latent_us": round(ga_ms * 1e3, 3), "latent_bytes": ga_b,
        "latent_gbs": round(ga_b / (ga_ms * 1e-3) / 1e9, 1),
        "latent_step_us": round(ls_ms * 1e3, 3), "latent_step_bytes": ga_b + bl_b,
        "latent_step_gbs": round((ga_b + bl_b) / (ls_ms * 1e-3) / 1e9, 1),
    }


def selection_scaling(torch, tdp, dev, counts=(1024, 4096, 16384), sets_n=8, steps=32):
    """Extract of the conditioned shape (B=2, 18 tiles) with more and more
    conditioning tokens (a quarter of them at negative time, as in the
    conditioned workload): microseconds and GB/s of its compulsory bytes,
    graph-timed over rotating buffer sets as the workloads are."""
    import numpy as np
    from synth import WORKLOADS, Workload, make_inputs
    base = WORKLOADS["conditioned"]
    out = []
    for nc in counts:
        wl = Workload(f"conditioned_{nc}", base.batch, base.channels, base.shape, base.tiling, num_cond=nc,
                      num_ref=nc // 4, dtype=base.dtype, seed=base.seed)
        inp = make_inputs(wl)
        plan = tdp.tdp_plan_create(tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, nc,
                                                   in_dtype=wl.dtype, out_dtype=wl.dtype))
        T = tdp.tdp_plan_num_tiles(plan)
        lat = torch.from_numpy(inp["latent"].view(np.int16)).view(torch.bfloat16).to(dev)
        pos = torch.from_numpy(inp["pos"]).to(dev)
        sets = [(lat.clone(), pos.clone(), tdp.allocate_extract_outputs(plan, dev)) for _ in range(sets_n)]
        stream = torch.cuda.Stream(dev)

        def ex(i):
            la, po, b = sets[i % sets_n]
            tdp.tdp_extract(plan, la, po, stream=stream, **b)

        def gather(i):
            la, _, b = sets[i % sets_n]
            tdp.tdp_extract_latent(plan, la, sets[0][2]["cond_row"], b["tile_lat"], stream=stream)
        ms = graph_time_ms(torch, stream, ex, steps)
        ga_ms = graph_time_ms(torch, stream, gather, steps)
        counts_t = sets[0][2]["tile_count"].cpu().numpy()
        ex_b, _, S = compulsory_bytes(wl, counts_t, T, 2, 2)
        ga_b = latent_bytes(wl, S, T, 2)
        out.append({"num_cond": nc, "tile_rows": S, "extract_us": round(ms * 1e3, 3), "extract_bytes": ex_b,
                    "extract_gbs": round(ex_b / (ms * 1e-3) / 1e9, 1), "latent_us": round(ga_ms * 1e3, 3),
                    "latent_bytes": ga_b, "latent_gbs": round(ga_b / (ga_ms * 1e-3) / 1e9, 1)})
        del sets
    return out


def ceiling_rates(torch, dev, nbytes=256 << 20, passes=12):
    """GB/s of plain hand-written streaming kernels (libtdp_ceiling.so):
    copies with non-temporal or device-scope stores, a read, a write, a
    gather (two reads per write) and a scatter (two writes per read).  Each
    pass uses a buffer pair the previous pass did not touch (at least 1 GB
    of traffic between two uses of a buffer)."""
    from overlap_tiling_trapezoidal_amd import ceiling
    bufs = [torch.empty(2 * nbytes, dtype=torch.uint8, device=dev) for _ in range(4)]
    for b in bufs:
        b.fill_(1)
    sink = torch.empty(4096, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(dev)
    out = {"bytes_per_pass": nbytes}
    for mode in ceiling.MODES:
        def run(i, mode=mode):
            ceiling.run(mode, bufs[(2 * i) % 4], bufs[(2 * i + 1) % 4], sink, nbytes, stream)
        ms = graph_time_ms(torch, stream, run, passes)
        out[mode + "_gbs"] = round(ceiling.MOVED[mode] * nbytes / (ms * 1e-3) / 1e9, 1)
    del bufs
    return out


def same_mix_ceilings(torch, dev, extract_read, blend_write, sets=8, passes=32):
    """The hand-written scatter and gather at the sizes of this workload's
    extract (reads `extract_read` bytes, writes twice that) and blend
    (writes `blend_write`, reads twice that), over `sets` rotating buffer
    sets as the bench rotates its own: GB/s and microseconds per pass."""
    from overlap_tiling_trapezoidal_amd import ceiling
    sink = torch.empty(4096, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(dev)
    out = {}
    for op, mode, nb in (("extract", "scatter", extract_read), ("blend", "gather", blend_write)):
        nb = max(8192, nb // 8192 * 8192)
        small = [torch.ones(nb, dtype=torch.uint8, device=dev) for _ in range(sets)]
        large = [torch.ones(2 * nb, dtype=torch.uint8, device=dev) for _ in range(sets)]
        src, dst = (small, large) if mode == "scatter" else (large, small)

        def run(i, mode=mode, nb=nb, src=src, dst=dst):
            ceiling.run(mode, src[i % sets], dst[i % sets], sink, nb, stream)
        ms = graph_time_ms(torch, stream, run, passes)
        moved = ceiling.MOVED[mode] * nb
        out[op] = {"mode": mode, "bytes": moved, "us": round(ms * 1e3, 3),
                   "gbs": round(moved / (ms * 1e-3) / 1e9, 1)}
        del small, large, src, dst
    return out


def cpu_baseline(wl, inp, extract_bytes, blend_bytes, budget_s=12.0):
    """The oracle (numpy, fp64 blend) on the same workload, repeated ~budget_s."""
    import numpy as np
    import oracle as O
    wall = cpu = 0.0
    reps = 0
    while wall < budget_s or reps == 0:
        c0, t0 = time.process_time(), time.perf_counter()
        ex = O.extract(inp["latent"], inp["pos"], wl.shape, wl.tiling, wl.num_cond)
        ys = [O.bf16_bits_to_f32(et["latent"]) if et["latent"].dtype == np.uint16 else et["latent"]
              for et in ex["tiles"]]
        O.blend(ys, ex, wl.shape, wl.tiling, wl.num_cond)
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        reps += 1
    per = wall / reps
    return {
        "value": round((extract_bytes + blend_bytes) / per / 1e9, 4),
        "unit": "GB/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"full {wl.name} workload, oracle extract+blend x{reps} ({wall:.1f} s wall, "
                  f"{per * 1e3:.0f} ms per step); host has {os.cpu_count()} CPUs, "
                  f"{len(os.sched_getaffinity(0))} in affinity",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1, help="GPUs (one: every tile runs locally)")
    ap.add_argument("--steps", type=int, default=500, help="timed pipelined steps K")
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps before the timed ones")
    ap.add_argument("--workload", default="4k", choices=("tiny", "ltx", "fullres", "4k", "conditioned"),
                    help="the workload the headline line times")
    ap.add_argument("--sets", type=int, default=8, help="rotating buffer sets (cache-cold launches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-normalize", action="store_true",
                    help="plan without TDP_NORMALIZE_POSITIONS (positions copied unshifted)")
    ap.add_argument("--no-workloads", action="store_true", help="skip the per-workload table")
    ap.add_argument("--step", choices=("full", "latent"), default="full",
                    help="full: tdp_pipeline_step (the whole extract and a blend); latent: "
                         "tdp_pipeline_latent_step over latents that share one positions set (the "
                         "latent gather and a blend; tables from one tdp_extract_positions call)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the tiled hot path has no cross-GPU step here "
              "(every tile runs locally). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import overlap_tiling_trapezoidal_amd as tdp
    from synth import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    wl = WORKLOADS[args.workload]
    inp = make_inputs(wl)
    cfg = tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond,
                          in_dtype=wl.dtype, out_dtype=wl.dtype, normalize=not args.no_normalize)
    plan = tdp.tdp_plan_create(cfg)
    T = tdp.tdp_plan_num_tiles(plan)
    R = max(4, args.sets)
    D = R // 2  # blend runs D steps behind extract

    def to_dev_latent(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    sets = []
    for r in range(R):
        bufs = tdp.allocate_extract_outputs(plan, dev)
        sets.append({
            "latent": to_dev_latent(inp["latent"]),
            "pos": torch.from_numpy(inp["pos"]).to(dev),
            "bufs": bufs,
            "out": tdp.allocate_output(plan, dev),
        })
    stream = torch.cuda.current_stream(dev)

    def extract(s, st=None):
        b = s["bufs"]
        tdp.tdp_extract(plan, s["latent"], s["pos"], b["tile_lat"], b["tile_pos"], b["tile_index"],
                        b["tile_count"], b["cond_row"], b["cond_k"], b["workspace"], st or stream)

    def blend(s, st=None):
        b = s["bufs"]
        tdp.tdp_blend(plan, b["tile_lat"], b["cond_row"], b["cond_k"], s["out"], st or stream)

    latent_steps = args.step == "latent"
    tables = sets[0]["bufs"]  # every set has the same positions: one set's selection serves all

    def step(i, st=None):
        """Pipelined step i: extract set i mod R and blend set (i - D) mod R,
        one tdp_pipeline_step (one launch where the plan allows); with
        --step latent, the latent gather of set i and the blend of set i - D,
        one tdp_pipeline_latent_step."""
        s, q = sets[i % R], sets[(i - D) % R]
        b = s["bufs"]
        if latent_steps:
            tdp.tdp_pipeline_latent_step(plan, s["latent"], tables["cond_row"], b["tile_lat"],
                                         tile_out=q["bufs"]["tile_lat"], blend_cond_row=tables["cond_row"],
                                         blend_cond_k=tables["cond_k"], out=q["out"], stream=st or stream)
            return
        tdp.tdp_pipeline_step(plan, s["latent"], s["pos"], b["tile_lat"], b["tile_pos"], b["tile_index"],
                              b["tile_count"], b["cond_row"], b["cond_k"], b["workspace"],
                              tile_out=q["bufs"]["tile_lat"], blend_cond_row=q["bufs"]["cond_row"],
                              blend_cond_k=q["bufs"]["cond_k"], out=q["out"], stream=st or stream)

    def step_two_calls(i, st=None):
        if latent_steps:
            s = sets[i % R]
            tdp.tdp_extract_latent(plan, s["latent"], tables["cond_row"], s["bufs"]["tile_lat"], st or stream)
        else:
            extract(sets[i % R], st)
        blend(sets[(i - D) % R], st)

    # prime every set, then warm up the pipeline
    for s in sets:
        extract(s)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    counts = sets[0]["bufs"]["tile_count"].cpu().numpy()
    e_in = 2 if wl.dtype == "bf16" else 4
    ex_bytes, bl_bytes, S = compulsory_bytes(wl, counts, T, e_in, e_in)
    ga_bytes = latent_bytes(wl, S, T, e_in)
    step_bytes = (ga_bytes if latent_steps else ex_bytes) + bl_bytes

    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # eager: exactly K steps launched from Python between two events
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        step(i)
    stop.record(stream)
    enqueue = time.perf_counter() - wall0
    torch.cuda.synchronize()
    eager_ms_per_step = start.elapsed_time(stop) / K

    # spread over steps: K more eager steps, each between events of its own
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    evs[0].record(stream)
    for i in range(K):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(K))
    pct = {f"p{q}": round(per_step[min(K - 1, round(q / 100 * (K - 1)))], 5) for q in (10, 50, 90)}

    # timed region: the same K steps captured once in a HIP graph (the form a
    # serving loop runs), replayed once untimed, then replayed between two
    # events on the capture stream
    pstream = torch.cuda.Stream(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=pstream):
        for i in range(K):
            step(i, pstream)
    with torch.cuda.stream(pstream):
        graph.replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    with torch.cuda.stream(pstream):
        start.record(pstream)
        graph.replay()
        stop.record(pstream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(stop) / K
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    del graph
    # the same K steps as two calls each (tdp_extract, then tdp_blend)
    two_ms = graph_time_ms(torch, pstream, lambda i: step_two_calls(i, pstream), K)
    fused = latent_steps or wl.num_cond == 0  # one launch per step

    # per-operation launch durations (graph replay, launch stream)
    gstream = torch.cuda.Stream(dev)
    reps = max(16, min(K, 64))

    def extract_g(i):
        b = sets[i % R]["bufs"]
        s = sets[i % R]
        tdp.tdp_extract(plan, s["latent"], s["pos"], b["tile_lat"], b["tile_pos"], b["tile_index"],
                        b["tile_count"], b["cond_row"], b["cond_k"], b["workspace"], gstream)

    def blend_g(i):
        s = sets[i % R]
        tdp.tdp_blend(plan, s["bufs"]["tile_lat"], s["bufs"]["cond_row"], s["bufs"]["cond_k"], s["out"], gstream)

    ex_ms = graph_time_ms(torch, gstream, extract_g, reps)
    bl_ms = graph_time_ms(torch, gstream, blend_g, reps)

    # streaming blend: tile by tile into an fp32 accumulator, then rounding
    accs = [tdp.allocate_accumulator(plan, dev) for _ in range(2)]
    infos = [tdp.tdp_plan_tile(plan, t) for t in range(T)]
    tile_elems = [wl.batch * inf.capacity * wl.channels for inf in infos]
    views = [[s["bufs"]["tile_lat"][inf.lat_offset: inf.lat_offset + n] for inf, n in zip(infos, tile_elems)]
             for s in sets]

    def stream_g(i):
        s = sets[i % R]
        acc = accs[i % 2]
        for t in range(T):
            tdp.tdp_blend_tile(plan, t, views[i % R][t], s["bufs"]["cond_row"], s["bufs"]["cond_k"], acc, gstream)
        tdp.tdp_blend_finish(plan, acc, s["out"], gstream)

    st_ms = graph_time_ms(torch, gstream, stream_g, max(8, reps // 4))
    st_bytes = stream_bytes(wl, S, e_in, e_in)
    del accs, views
    pix = pixel_rate(torch, tdp, dev, gstream)
    share = rank_share_rate(torch, tdp, dev, sets, wl, 4, 0, reps) if wl.num_cond == 0 else None

    # torch's device copy of the same size, for reference
    nbytes = 256 << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(3)]
    for d in dst:
        d.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record(stream)
    for i in range(12):
        dst[i % 3].copy_(src if i % 2 == 0 else dst[(i + 1) % 3])
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 12 * 2 * nbytes / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    ceilings = ceiling_rates(torch, dev)
    best_copy = max(ceilings["copy_nt_gbs"], ceilings["copy_device_scope_gbs"])
    e_in_b = 2 if wl.dtype == "bf16" else 4
    rows = wl.tokens + wl.num_cond
    mix = same_mix_ceilings(torch, dev, wl.batch * rows * (wl.channels * e_in_b + 3 * 8),
                            wl.batch * rows * wl.channels * e_in_b)

    # the same step on every workload (this run's own figures for its workload)
    table = {}
    scaling = None
    if not args.no_workloads:
        for name, w in WORKLOADS.items():
            log(f"[bench] workload {name}")
            table[name] = workload_rates(torch, tdp, dev, w)
        log("[bench] selection scaling")
        scaling = selection_scaling(torch, tdp, dev)

    if latent_steps:  # the step is one launch: that kernel is the dominant one
        dom = ("latent gather + blend, one launch", step_bytes, ms_per_step,
               "pipeline_latent_kernel; in one-wave workgroups, pipeline_latent_wave_kernel, for plans without "
               "conditioning tokens and more than 16 blend units per compute unit")
    elif fused:
        dom = ("extract + blend, one launch", step_bytes, ms_per_step, "pipeline_kernel")
    else:
        dom = ("extract", ex_bytes, ex_ms, "extract_kernel") if ex_ms >= bl_ms else \
              ("blend", bl_bytes, bl_ms, "blend_kernel")
    achieved = dom[1] / (dom[2] * 1e-3) / 1e9
    traffic = measured_traffic(wl.name, dom[3]) if not args.no_normalize else None
    result = {
        "metric": "tiled extract+blend GB/s on 1 MI355X; fraction of HBM peak",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) latent, grid positions)",
        "config": {
            "workload": f"{wl.name}: B={wl.batch} C={wl.channels} (F,H,W)={wl.shape} {wl.dtype}, "
                        f"tiles {tuple(n for n, _ in wl.tiling)} overlap {tuple(o for _, o in wl.tiling)}, "
                        f"{T} tiles, {wl.num_cond} conditioning tokens",
            "tokens": wl.tokens,
            "tile_rows": S,
            "bytes_per_step": step_bytes,
            "naive_bytes_per_step": step_bytes + naive_bytes(wl, S, e_in),
            "buffer_sets": R,
            "normalize_positions": not args.no_normalize,
            "step": args.step,
        },
        "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "step_call": ("tdp_pipeline_latent_step (one launch; tables from one tdp_extract_positions)"
                      if latent_steps else "tdp_pipeline_step (one launch)" if fused
                      else "tdp_pipeline_step (extents with the blend, then selection, positions and latent rows)"),
        "two_calls": {"ms_per_step": round(two_ms, 5), "value": round(step_bytes / (two_ms * 1e-3) / 1e9, 2),
                      "note": ("the same K steps as tdp_extract_latent + tdp_blend" if latent_steps else
                               "the same K steps as tdp_extract + tdp_blend") + ", two calls each"},
        "ops": {
            "extract_ms": round(ex_ms, 5), "extract_bytes": ex_bytes,
            "extract_gbs": round(ex_bytes / (ex_ms * 1e-3) / 1e9, 1),
            "blend_ms": round(bl_ms, 5), "blend_bytes": bl_bytes,
            "blend_gbs": round(bl_bytes / (bl_ms * 1e-3) / 1e9, 1),
            "graph_launches": reps,
            "stream_blend_ms": round(st_ms, 5), "stream_blend_bytes": st_bytes,
            "stream_blend_gbs": round(st_bytes / (st_ms * 1e-3) / 1e9, 1),
        },
        "pixel_blend": pix,
        "rank_share": share,
        "torch_copy_gbs": round(copy_gbs, 1),
        "ceilings": ceilings,
        "frac_of_best_copy": round(gbs / best_copy, 4),
        "same_mix_ceilings": mix,
        "frac_of_same_mix": {
            "extract": round((ex_bytes / (ex_ms * 1e-3) / 1e9) / mix["extract"]["gbs"], 4),
            "blend": round((bl_bytes / (bl_ms * 1e-3) / 1e9) / mix["blend"]["gbs"], 4),
        },
        "target": "70% of the 8 TB/s peak on the 4K-class latent (5600 GB/s, 36.3 us per step)",
        "meets_target": bool(wl.name == "4k" and gbs >= 0.7 * HBM_PEAK_GBS),
        "workloads": table,
        "selection_scaling": scaling,
        "roofline": {
            "bound": "hbm",
            "kernel": f"{dom[0]} ({dom[3]})",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": dom[1],
            "avg_launch_us": round(dom[2] * 1e3, 3),
            "traffic_source": PMC_SUMMARY if traffic is not None else None,
        },
        "wall_s_timed_region": round(wall, 4),
        "timing": "HIP graph of the K steps, replayed between two events",
        "eager_ms_per_step": round(eager_ms_per_step, 5),
        "eager_step_ms_percentiles": pct,
        "eager_value": round(step_bytes / (eager_ms_per_step * 1e-3) / 1e9, 2),
        "eager_enqueue_s": round(enqueue, 4),
        "sources_sha256_16": sources_hash(),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(wl, inp, ex_bytes, bl_bytes, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
