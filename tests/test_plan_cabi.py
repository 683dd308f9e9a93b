"""Host-side tests of the C-ABI library (no GPU needed).

The library loads and exports every function include/tdp.h declares; the
host planner agrees bit for bit with the oracle on intervals, windows, tile
enumeration and slot layout; every error path returns its status and a
message naming the limit.  No device function is called here.
"""
import ctypes
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import overlap_tiling_trapezoidal_amd as tdp
from synth import WORKLOADS


@pytest.fixture(scope="module")
def lib():
    return tdp.load_library()


def plan_for(wl, **kw):
    cfg = tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond,
                          in_dtype=wl.dtype, **kw)
    return tdp.tdp_plan_create(cfg)


def test_exports_the_host_planner(lib):
    """Every declared function but the device entry points, in any build."""
    names = [n for n in tdp.header_functions() if n not in tdp.DEVICE_FUNCTIONS]
    assert len(names) >= 19
    for name in names:
        assert hasattr(lib, name), name


@pytest.mark.device_abi
def test_exports_every_declared_symbol(lib):
    names = tdp.header_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


@pytest.mark.device_abi
def test_ceiling_library_exports_and_rejects_bad_arguments():
    """The measurement library loads, exports what include/tdp_ceiling.h
    declares and refuses bad arguments on the host (nothing enqueued)."""
    from overlap_tiling_trapezoidal_amd import ceiling
    clib = ceiling.load_library()
    names = ceiling.header_functions()
    assert names == ["tdp_ceiling_run"]
    for name in names:
        assert ctypes.cast(getattr(clib, name), ctypes.c_void_p).value
    al, null = ctypes.c_void_p(0x1000), ctypes.c_void_p(None)
    assert clib.tdp_ceiling_run(6, al, al, al, 8192, null) == -1        # mode
    assert clib.tdp_ceiling_run(0, al, al, null, 8000, null) == -1      # size
    assert clib.tdp_ceiling_run(0, null, al, null, 8192, null) == -1    # src
    assert clib.tdp_ceiling_run(2, al, null, null, 8192, null) == -1    # sink
    assert clib.tdp_ceiling_run(0, ctypes.c_void_p(0x1008), al, null, 8192, null) == -1  # alignment


def fp32_rne(q: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational (ties to even)."""
    f = np.float32(float(q))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - q)
        if best is None or err < best[0] or (err == best[0] and (int(cand.view(np.uint32)) & 1) == 0):
            best = (err, cand)
    return best[1]


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_plan_matches_oracle(name):
    wl = WORKLOADS[name]
    plan = plan_for(wl)
    ivs = [O.split_by_count(d, n, o) for d, (n, o) in zip(wl.shape, wl.tiling)]
    for d in range(3):
        assert tdp.tdp_plan_intervals(plan, d) == ivs[d]
        for i in range(len(ivs[d])):
            got = tdp.tdp_plan_window(plan, d, i)
            want = np.array([fp32_rne(w) for w in O.window_exact(ivs[d], i, wl.tiling[d][1])], np.float32)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    tiles = O.enumerate_tiles(wl.shape, wl.tiling)
    assert tdp.tdp_plan_num_tiles(plan) == len(tiles)
    lat_off = pos_off = idx_off = 0
    for t, tile in enumerate(tiles):
        info = tdp.tdp_plan_tile(plan, t)
        assert info.index == t
        assert tuple(info.grid) == tile["grid"]
        assert tuple(info.origin) == tile["origin"]
        assert tuple(info.shape) == tile["size"]
        gen = int(np.prod(tile["size"]))
        assert info.gen_tokens == gen
        assert info.capacity == gen + wl.num_cond
        # slots are packed back to back in tile order
        assert (info.lat_offset, info.pos_offset, info.index_offset) == (lat_off, pos_off, idx_off)
        lat_off += wl.batch * info.capacity * wl.channels
        pos_off += wl.batch * info.capacity * 6
        idx_off += info.capacity
        assert tdp.tdp_plan_tile_rank(plan, t, 4) == O.round_robin_rank(t, 4)
    s = tdp.tdp_plan_sizes(plan)
    assert (s.tile_lat_elems, s.tile_pos_floats, s.tile_index_ints) == (lat_off, pos_off, idx_off)
    assert s.cond_row_ints == len(tiles) * wl.num_cond
    assert s.cond_k_ints == wl.num_cond
    assert (s.workspace_bytes > 0) == (wl.num_cond > 0)
    assert s.out_elems == wl.batch * (wl.tokens + wl.num_cond) * wl.channels


def test_plan_matches_oracle_random_guarded():
    rng = np.random.default_rng(11)
    done = 0
    while done < 300:
        shape = tuple(int(x) for x in rng.integers(1, 70, size=3))
        tiling = []
        for dim in shape:
            n = int(rng.integers(1, 7))
            o = 0 if n == 1 else int(rng.integers(0, dim // (n + 1) + 1))
            if dim - o < n:
                n, o = 1, 0
            tiling.append((n, o))
        cfg = tdp.make_config(1, 8, shape, tiling, in_dtype="bf16")
        plan = tdp.tdp_plan_create(cfg)
        for d in range(3):
            assert tdp.tdp_plan_intervals(plan, d) == O.split_by_count(shape[d], *tiling[d])
        assert tdp.tdp_plan_num_tiles(plan) == len(O.enumerate_tiles(shape, tiling))
        done += 1


def test_unguarded_window_sums_reproduce_table():
    # The 1-D table of mold #673 through the library: dim 21, overlap 8.
    for n, want_max in [(2, 1.0), (3, 1.074), (4, 1.161)]:
        cfg = tdp.make_config(1, 8, (1, 1, 21), ((1, 0), (1, 0), (n, 8)), unguarded=True)
        plan = tdp.tdp_plan_create(cfg)
        sums = np.zeros(21, np.float32)   # fp32 sums, as a blend would form them
        for i, (a, b) in enumerate(tdp.tdp_plan_intervals(plan, 2)):
            sums[a:b] += tdp.tdp_plan_window(plan, 2, i)
        assert abs(float(sums.max()) - want_max) <= 1e-3
        if n == 2:
            assert np.all(sums == np.float32(1.0))


def test_fp32_ramps_sum_to_one():
    # Complementary ramps (j+1)/(o+1) and (o-j)/(o+1) add to exactly 1 in fp32.
    for o in range(1, 300):
        dim = 3 * o + 3
        cfg = tdp.make_config(1, 8, (1, 1, dim), ((1, 0), (1, 0), (2, o)))
        plan = tdp.tdp_plan_create(cfg)
        (a0, b0), (a1, b1) = tdp.tdp_plan_intervals(plan, 2)
        w0, w1 = tdp.tdp_plan_window(plan, 2, 0), tdp.tdp_plan_window(plan, 2, 1)
        s = np.zeros(dim, np.float32)
        s[a0:b0] += w0
        s[a1:b1] += w1
        assert np.all(s == np.float32(1.0)), o


@pytest.mark.parametrize("kw,status,fragment", [
    (dict(tiling=((1, 0), (2, 8), (1, 0)), shape=(4, 21, 8)), tdp.TDP_EGUARD, "reduce overlap on height to <= 7"),
    (dict(tiling=((1, 1), (1, 0), (1, 0))), tdp.TDP_EGUARD, "untiled axis"),
    (dict(tiling=((0, 0), (1, 0), (1, 0))), tdp.TDP_EINVAL, "num_tiles"),
    (dict(tiling=((1, 0), (2, -1), (1, 0))), tdp.TDP_EINVAL, "overlap must be >= 0"),
    (dict(tiling=((1, 0), (1, 0), (9, 0)), shape=(4, 8, 8)), tdp.TDP_ESHAPE, "stride below one cell"),
    (dict(tiling=((1, 0), (1, 0), (33, 0)), shape=(4, 8, 100)), tdp.TDP_ESHAPE, "limit of 32"),
    (dict(channels=12), tdp.TDP_ESHAPE, "multiple of 16 bytes"),
    (dict(channels=1024), tdp.TDP_ESHAPE, "at most 1024"),
    (dict(batch=0), tdp.TDP_EINVAL, ">= 1"),
    (dict(num_cond=-1), tdp.TDP_EINVAL, "num_cond"),
    (dict(in_dtype=7), tdp.TDP_EINVAL, "in_dtype"),
    (dict(shape=(4, 8, 5000)), tdp.TDP_ESHAPE, "width 5000"),
    (dict(shape=(1024, 1024, 4096), num_cond=0), tdp.TDP_ESHAPE, "int32"),
])
def test_plan_errors(kw, status, fragment):
    args = dict(batch=1, channels=128, shape=(4, 8, 8), tiling=((1, 0), (1, 0), (1, 0)), num_cond=0,
                in_dtype="bf16")
    args.update(kw)
    cfg = tdp.make_config(args["batch"], args["channels"], args["shape"], args["tiling"], args["num_cond"],
                          in_dtype=args["in_dtype"])
    with pytest.raises(tdp.TdpError) as ei:
        tdp.tdp_plan_create(cfg)
    assert ei.value.status == status
    assert fragment in str(ei.value), str(ei.value)


def test_unknown_flags_and_nulls(lib):
    cfg = tdp.make_config(1, 128, (4, 8, 8), ((1, 0),) * 3)
    cfg.flags = 0x80
    with pytest.raises(tdp.TdpError) as ei:
        tdp.tdp_plan_create(cfg)
    assert ei.value.status == tdp.TDP_EINVAL
    assert lib.tdp_plan_create(None, None) == tdp.TDP_EINVAL
    assert lib.tdp_plan_num_tiles(None, None) == tdp.TDP_EINVAL
    assert lib.tdp_status_string(tdp.TDP_EGUARD).startswith(b"TDP_EGUARD")


@pytest.mark.device_abi
def test_device_calls_reject_bad_plans_before_launch(lib):
    # Validation happens on the host before anything is enqueued, so these
    # run without a GPU.
    cfg = tdp.make_config(1, 8, (1, 1, 21), ((1, 0), (1, 0), (3, 8)), unguarded=True)
    plan = tdp.tdp_plan_create(cfg)
    null = ctypes.c_void_p(None)
    assert lib.tdp_extract(plan.handle, *([null] * 10)) == tdp.TDP_EGUARD
    assert lib.tdp_blend(plan.handle, *([null] * 5)) == tdp.TDP_EGUARD
    good = tdp.tdp_plan_create(tdp.make_config(1, 128, (4, 8, 8), ((1, 0), (2, 2), (2, 2))))
    assert lib.tdp_extract(good.handle, *([null] * 10)) == tdp.TDP_EINVAL
    assert "null" in tdp.tdp_last_error()
    assert lib.tdp_blend(good.handle, *([null] * 5)) == tdp.TDP_EINVAL
    assert lib.tdp_extract(None, *([null] * 10)) == tdp.TDP_EINVAL
    # misaligned pointers are refused too
    odd = ctypes.c_void_p(0x1002)
    al = ctypes.c_void_p(0x1000)
    assert lib.tdp_extract(good.handle, odd, al, al, al, al, al, null, null, null, null) == tdp.TDP_EINVAL
    assert "aligned" in tdp.tdp_last_error()


@pytest.mark.device_abi
@pytest.mark.parametrize("case", ["rank_zero_fill", "whole_latent_units", "whole_conditioned"])
def test_device_calls_refuse_launches_past_32_bit_work_items(case, lib):
    """Plans inside every planner limit whose launches would need more
    work-items than one HIP launch counts (2^32 - 1) are refused with
    TDP_ESHAPE by every device call, on the host and before the first
    launch, so no call leaves partial output.
    - rank_zero_fill: a rank's blend zero-fills 8192 * 8192 lines, one
      256-thread workgroup each (2^34 work-items);
    - whole_latent_units: 2^27 one-row lines of 1024-byte rows, one wave
      each (2^33);
    - whole_conditioned: the same with conditioning tokens (the selection
      and conditioning blend parts add to the sum)."""
    null = ctypes.c_void_p(None)
    if case == "rank_zero_fill":
        cfg = tdp.make_config(1, 8, (8192, 8192, 1), ((1, 0), (2, 8), (1, 0)))
        plan = tdp.tdp_plan_create_rank(cfg, 2, 0)
    else:
        nc = 4096 if case == "whole_conditioned" else 0
        plan = tdp.tdp_plan_create(tdp.make_config(1, 512, (8192, 16384, 1), ((1, 0), (2, 8), (1, 0)), nc))
    b = [ctypes.c_void_p((i + 1) << 40) for i in range(16)]   # distinct, aligned, never dereferenced
    calls = {
        "tdp_extract": lambda: lib.tdp_extract(plan.handle, *b[:9], null),
        "tdp_extract_noalloc": lambda: lib.tdp_extract_noalloc(plan.handle, *b[:8], null),
        "tdp_extract_positions": lambda: lib.tdp_extract_positions(plan.handle, *b[:7], null),
        "tdp_extract_latent": lambda: lib.tdp_extract_latent(plan.handle, *b[:3], null),
        "tdp_blend": lambda: lib.tdp_blend(plan.handle, *b[:4], null),
        "tdp_pipeline_step": lambda: lib.tdp_pipeline_step(plan.handle, *b[:13], null),
        "tdp_pipeline_latent_step": lambda: lib.tdp_pipeline_latent_step(plan.handle, *b[:7], null),
    }
    for name, call in calls.items():
        assert call() == tdp.TDP_ESHAPE, name
        assert "work-items" in tdp.tdp_last_error(), (name, tdp.tdp_last_error())
    if case != "rank_zero_fill":
        # the streaming blend: its finish pass (one thread per four floats of
        # a 2^27-row, 512-channel accumulator) is refused at the first tile
        assert lib.tdp_blend_tile(plan.handle, 0, *b[:3], b[3], null) == tdp.TDP_ESHAPE
        assert "work-items" in tdp.tdp_last_error()
        assert lib.tdp_blend_finish(plan.handle, b[0], b[1], null) == tdp.TDP_ESHAPE


@pytest.mark.device_abi
def test_pipeline_step_refuses_before_launch(lib):
    """Bad and overlapping arguments are refused on the host (no GPU call)."""
    plan = plan_for(WORKLOADS["4k"])
    s = tdp.tdp_plan_sizes(plan)
    null = ctypes.c_void_p(None)
    base = {k: ctypes.c_void_p((i + 1) << 36) for i, k in enumerate(
        ("latent", "pos", "tile_lat", "tile_pos", "index", "count", "tile_out", "out"))}

    def call(**over):
        a = dict(base, **over)
        return lib.tdp_pipeline_step(plan.handle, a["latent"], a["pos"], a["tile_lat"], a["tile_pos"], a["index"],
                                     a["count"], null, null, null, a["tile_out"], null, null, a["out"], null)
    assert call(tile_out=base["tile_lat"]) == tdp.TDP_EINVAL
    assert "reads a buffer the extract writes" in tdp.tdp_last_error()
    inside = ctypes.c_void_p(base["tile_lat"].value + (s.tile_lat_elems * 2 // 32) * 16)
    assert call(tile_out=inside) == tdp.TDP_EINVAL           # starts inside tile_lat
    assert call(out=base["tile_pos"]) == tdp.TDP_EINVAL
    assert "writes a buffer the extract writes" in tdp.tdp_last_error()
    assert call(out=ctypes.c_void_p(base["latent"].value + 4096)) == tdp.TDP_EINVAL
    assert "writes a buffer the extract reads" in tdp.tdp_last_error()
    assert call(out=null) == tdp.TDP_EINVAL
    assert call(tile_out=ctypes.c_void_p(base["tile_out"].value + 8)) == tdp.TDP_EINVAL   # misaligned
    assert lib.tdp_pipeline_step(None, *([null] * 14)) == tdp.TDP_EINVAL


@pytest.mark.device_abi
def test_split_extract_refuses_before_launch(lib):
    """tdp_extract_positions, tdp_extract_latent and tdp_pipeline_latent_step
    refuse null, misaligned and overlapping arguments on the host (no GPU
    call); with conditioning tokens cond_row (and for the positions call
    cond_k and the workspace) are required."""
    wl = WORKLOADS["conditioned"]
    plan = plan_for(wl)
    s = tdp.tdp_plan_sizes(plan)
    null = ctypes.c_void_p(None)
    b = {k: ctypes.c_void_p((i + 1) << 36) for i, k in enumerate(
        ("latent", "pos", "tile_lat", "tile_pos", "index", "count", "cond_row", "cond_k", "ws", "tile_out", "out",
         "bcond_row", "bcond_k"))}

    def positions(**over):
        a = dict(b, **over)
        return lib.tdp_extract_positions(plan.handle, a["pos"], a["tile_pos"], a["index"], a["count"], a["cond_row"],
                                         a["cond_k"], a["ws"], null)

    def gather(**over):
        a = dict(b, **over)
        return lib.tdp_extract_latent(plan.handle, a["latent"], a["cond_row"], a["tile_lat"], null)

    def step(**over):
        a = dict(b, **over)
        return lib.tdp_pipeline_latent_step(plan.handle, a["latent"], a["cond_row"], a["tile_lat"], a["tile_out"],
                                            a["bcond_row"], a["bcond_k"], a["out"], null)
    for key in ("pos", "tile_pos", "index", "count", "cond_row", "cond_k", "ws"):
        assert positions(**{key: null}) == tdp.TDP_EINVAL, key
    assert "workspace" in (positions(ws=null), tdp.tdp_last_error())[1]
    assert positions(pos=ctypes.c_void_p(b["pos"].value + 4)) == tdp.TDP_EINVAL      # pairs need 8 bytes
    assert positions(ws=ctypes.c_void_p(b["ws"].value + 8)) == tdp.TDP_EINVAL        # workspace needs 16
    for key in ("latent", "cond_row", "tile_lat"):
        assert gather(**{key: null}) == tdp.TDP_EINVAL, key
    assert "cond_row is required" in (gather(cond_row=null), tdp.tdp_last_error())[1]
    assert gather(latent=ctypes.c_void_p(b["latent"].value + 8)) == tdp.TDP_EINVAL
    assert gather(cond_row=ctypes.c_void_p(b["cond_row"].value + 2)) == tdp.TDP_EINVAL
    assert step(tile_out=b["tile_lat"]) == tdp.TDP_EINVAL
    assert "which the gather writes" in tdp.tdp_last_error()
    assert step(bcond_row=ctypes.c_void_p(b["tile_lat"].value + (s.tile_lat_elems * 2 // 32) * 16)) == tdp.TDP_EINVAL
    assert step(out=ctypes.c_void_p(b["latent"].value + 4096)) == tdp.TDP_EINVAL
    assert "writes a buffer the gather reads" in tdp.tdp_last_error()
    assert step(out=b["cond_row"]) == tdp.TDP_EINVAL
    assert step(bcond_k=null) == tdp.TDP_EINVAL
    assert step(out=ctypes.c_void_p(b["out"].value + 8)) == tdp.TDP_EINVAL
    for f, n in ((lib.tdp_extract_positions, 8), (lib.tdp_extract_latent, 4), (lib.tdp_pipeline_latent_step, 8)):
        assert f(None, *([null] * n)) == tdp.TDP_EINVAL


@pytest.mark.device_abi
def test_lookback_polls_setting(lib):
    assert lib.tdp_set_lookback_polls(-1) == tdp.TDP_EINVAL
    assert "polls" in tdp.tdp_last_error()
    for polls in (0, 1, 256):
        tdp.tdp_set_lookback_polls(polls)


@pytest.mark.device_abi
def test_cond_k_and_workspace_arguments(lib):
    """With conditioning tokens, tdp_extract needs cond_row, cond_k and the
    workspace, and tdp_blend / tdp_blend_tile need cond_row and cond_k; null
    and misaligned ones are refused on the host, before any launch."""
    wl = WORKLOADS["conditioned"]
    plan = plan_for(wl)
    s = tdp.tdp_plan_sizes(plan)
    T = len(O.enumerate_tiles(wl.shape, wl.tiling))
    assert s.cond_k_ints == wl.num_cond
    # at least one extent part per tile and one look-back word per (tile, 64 tokens)
    assert s.workspace_bytes >= T * wl.batch * 3 * 8 + T * (-(-wl.num_cond // 64)) * 4 and s.workspace_bytes % 256 == 0
    assert tdp.tdp_plan_sizes(plan_for(WORKLOADS["4k"])).workspace_bytes == 0
    null = ctypes.c_void_p(None)
    al = ctypes.c_void_p(0x1000)
    odd4 = ctypes.c_void_p(0x1002)   # not 4-byte aligned
    odd16 = ctypes.c_void_p(0x1008)  # 8- but not 16-byte aligned
    #                      latent pos tile_lat tile_pos index count cond_row cond_k workspace stream
    assert lib.tdp_extract(plan.handle, al, al, al, al, al, al, al, null, al, null) == tdp.TDP_EINVAL
    assert "cond_k" in tdp.tdp_last_error()
    assert lib.tdp_extract(plan.handle, al, al, al, al, al, al, null, al, al, null) == tdp.TDP_EINVAL
    assert "cond_row" in tdp.tdp_last_error()
    assert lib.tdp_extract(plan.handle, al, al, al, al, al, al, al, al, null, null) == tdp.TDP_EINVAL
    assert "workspace" in tdp.tdp_last_error()
    assert lib.tdp_extract(plan.handle, al, al, al, al, al, al, al, odd4, al, null) == tdp.TDP_EINVAL
    assert "align" in tdp.tdp_last_error()
    assert lib.tdp_extract(plan.handle, al, al, al, al, al, al, al, al, odd16, null) == tdp.TDP_EINVAL
    assert "workspace" in tdp.tdp_last_error()
    #                    tile_out cond_row cond_k out stream
    assert lib.tdp_blend(plan.handle, al, al, null, al, null) == tdp.TDP_EINVAL
    assert "cond_k" in tdp.tdp_last_error()
    assert lib.tdp_blend(plan.handle, al, al, odd4, al, null) == tdp.TDP_EINVAL
    assert lib.tdp_blend_tile(plan.handle, 0, al, al, null, al, null) == tdp.TDP_EINVAL
    assert "cond_k" in tdp.tdp_last_error()
    assert lib.tdp_blend_tile(plan.handle, 0, al, al, odd4, al, null) == tdp.TDP_EINVAL
    # without conditioning tokens none of the three is needed: the null
    # pointers pass validation (the launch itself needs a GPU, so it is not
    # reached here: a null latent is refused first)
    plain = plan_for(WORKLOADS["fullres"])
    assert lib.tdp_extract(plain.handle, null, al, al, al, al, al, null, null, null, null) == tdp.TDP_EINVAL
    assert "null device pointer" in tdp.tdp_last_error()


def test_4k_sizes():
    plan = plan_for(WORKLOADS["4k"])
    s = tdp.tdp_plan_sizes(plan)
    assert s.num_slots == 16
    assert s.tile_index_ints == 247296
    assert s.tile_lat_elems == 247296 * 128
    assert s.tile_pos_floats == 247296 * 6
    assert s.cond_row_ints == 0


# --- rank plans: one rank's round-robin share -----------------------------

@pytest.mark.parametrize("name", ["tiny", "conditioned", "4k"])
@pytest.mark.parametrize("world", [1, 2, 3, 4, 7, 40])
def test_rank_plan_layout(name, world):
    wl = WORKLOADS[name]
    cfg = tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond, in_dtype=wl.dtype)
    tiles = O.enumerate_tiles(wl.shape, wl.tiling)
    T = len(tiles)
    whole = tdp.tdp_plan_create(cfg)
    gen_max = max(int(np.prod(t["size"])) for t in tiles)
    for rank in range(world):
        plan = tdp.tdp_plan_create_rank(cfg, world, rank)
        mine = [t for t in range(T) if O.round_robin_rank(t, world) == rank]
        assert tdp.tdp_plan_local_tiles(plan) == (world, rank, len(mine))
        assert tdp.held_tiles(plan) == mine
        assert tdp.tdp_plan_num_tiles(plan) == T
        s = tdp.tdp_plan_sizes(plan)
        assert s.num_slots == len(mine)
        assert s.cond_row_ints == T * wl.num_cond          # k counts every rank's tiles
        assert s.out_elems == wl.batch * (wl.tokens + wl.num_cond) * wl.channels
        if world == 1:
            sw = tdp.tdp_plan_sizes(whole)
            assert (s.tile_lat_elems, s.tile_pos_floats, s.tile_index_ints) == \
                   (sw.tile_lat_elems, sw.tile_pos_floats, sw.tile_index_ints)
            for t in range(T):
                a, b = tdp.tdp_plan_tile(plan, t), tdp.tdp_plan_tile(whole, t)
                assert (a.lat_offset, a.pos_offset, a.index_offset) == (b.lat_offset, b.pos_offset, b.index_offset)
            continue
        cap = gen_max + wl.num_cond                        # uniform slots
        assert s.tile_index_ints == len(mine) * cap
        assert s.tile_lat_elems == len(mine) * cap * wl.batch * wl.channels
        assert s.tile_pos_floats == len(mine) * cap * wl.batch * 6
        for t in range(T):
            info = tdp.tdp_plan_tile(plan, t)
            assert tuple(info.origin) == tiles[t]["origin"] and tuple(info.shape) == tiles[t]["size"]
            assert info.capacity == int(np.prod(tiles[t]["size"])) + wl.num_cond
            if t in mine:
                j = mine.index(t)
                assert info.index_offset == j * cap
                assert info.lat_offset == j * cap * wl.batch * wl.channels
                assert info.pos_offset == j * cap * wl.batch * 6
            else:
                assert (info.lat_offset, info.pos_offset, info.index_offset) == (-1, -1, -1)


def test_rank_plan_errors(lib):
    cfg = tdp.make_config(1, 128, (4, 8, 8), ((1, 0), (2, 2), (2, 2)))
    for world, rank in [(0, 0), (-1, 0), (2, 2), (2, -1), (3, 5)]:
        with pytest.raises(tdp.TdpError) as ei:
            tdp.tdp_plan_create_rank(cfg, world, rank)
        assert ei.value.status == tdp.TDP_EINVAL
    assert lib.tdp_plan_create_rank(None, 2, 0, None) == tdp.TDP_EINVAL
    bad = tdp.make_config(1, 128, (4, 8, 8), ((1, 0), (2, 5), (2, 2)))   # guard: 5 * 3 > 8
    with pytest.raises(tdp.TdpError) as ei:
        tdp.tdp_plan_create_rank(bad, 2, 0)
    assert ei.value.status == tdp.TDP_EGUARD


@pytest.mark.device_abi
def test_rank_plan_device_call_errors(lib):
    # the streaming blend is for whole plans; refused before any launch
    cfg = tdp.make_config(1, 128, (4, 8, 8), ((1, 0), (2, 2), (2, 2)))
    plan = tdp.tdp_plan_create_rank(cfg, 2, 1)
    al = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(None)
    assert lib.tdp_blend_tile(plan.handle, 1, al, null, null, al, null) == tdp.TDP_EINVAL
    assert "rank plans" in tdp.tdp_last_error()
    assert lib.tdp_blend_finish(plan.handle, al, al, null) == tdp.TDP_EINVAL
    # a rank that holds tiles still needs its tile buffers
    assert lib.tdp_extract(plan.handle, al, al, null, null, null, null, null, null, null, null) == tdp.TDP_EINVAL
    assert lib.tdp_blend(plan.handle, null, null, null, al, null) == tdp.TDP_EINVAL


def _brute_cover(ivs, x):
    return [i for i, (a, b) in enumerate(ivs) if a <= x < b]


def test_cell_tiles_match_brute_force():
    rng = np.random.default_rng(5)
    checked = 0
    for _ in range(400):
        dim = int(rng.integers(1, 300))
        n = int(rng.integers(1, min(32, dim) + 1))
        o = 0 if n == 1 else int(rng.integers(0, dim // (n + 1) + 1))
        if dim - o < n:
            continue
        plan = tdp.tdp_plan_create(tdp.make_config(1, 8, (1, 1, dim), ((1, 0), (1, 0), (n, o))))
        ivs = O.split_by_count(dim, n, o)
        for x in range(dim):
            assert tdp.tdp_plan_cell_tiles(plan, 2, x) == _brute_cover(ivs, x), (dim, n, o, x)
        checked += 1
    assert checked > 300


def test_large_axes_near_limit():
    # Products i*(dim-o) and (x+1)*n reach 2^31 at TDP_MAX_AXIS cells and 32
    # tiles with no overlap (the first case); they are formed in uint32.
    limit = 1 << 26
    rng = np.random.default_rng(9)
    for dim, n, o in [(limit, 32, 0), (limit, 32, None), (limit - 7, 31, None), (limit // 3 + 1, 17, None),
                      (123457, 32, None)]:
        if o is None:
            o = int(rng.integers(0, dim // (n + 1) + 1))
        plan = tdp.tdp_plan_create(tdp.make_config(1, 8, (dim, 1, 1), ((n, o), (1, 0), (1, 0))))
        ivs = O.split_by_count(dim, n, o)
        assert tdp.tdp_plan_intervals(plan, 0) == ivs
        for x in list(rng.integers(0, dim, 200)) + [0, dim - 1] + [a for a, _ in ivs] + [b - 1 for _, b in ivs]:
            assert tdp.tdp_plan_cell_tiles(plan, 0, int(x)) == _brute_cover(ivs, int(x))
    with pytest.raises(tdp.TdpError) as ei:
        tdp.tdp_plan_create(tdp.make_config(1, 8, (limit + 1, 1, 1), ((1, 0),) * 3))
    assert ei.value.status == tdp.TDP_ESHAPE
    # positions are addressed with 32-bit byte offsets: fewer than 2^29 rows
    tdp.tdp_plan_create(tdp.make_config(1, 8, (limit, 7, 1), ((1, 0),) * 3, num_cond=limit - 1))
    with pytest.raises(tdp.TdpError) as ei:
        tdp.tdp_plan_create(tdp.make_config(1, 8, (limit, 7, 1), ((1, 0),) * 3, num_cond=limit))
    assert ei.value.status == tdp.TDP_ESHAPE
    assert "2^29" in str(ei.value) or str(1 << 29) in str(ei.value)


# --------------------------------------------------------------------------
# Plan quality: library figures against the oracle's
# --------------------------------------------------------------------------

def _same_quality(lib_q, ref):
    for k in ("total_cells", "grid_cells", "largest_cells", "seams", "max_rank_cells", "rank_cells"):
        assert lib_q[k] == ref[k], k
    for k in ("area_ratio", "largest_fraction", "imbalance"):
        assert lib_q[k] == pytest.approx(float(ref[k]), rel=1e-15, abs=1e-15), k


def test_quality_distvae_strips_matches_oracle():
    dims, ivs = (128, 128), [[(0, 43), (32, 75), (64, 107), (96, 128)], [(0, 128)]]
    for world in (1, 2, 3, 4, 5, 8):
        _same_quality(tdp.tdp_tiling_quality(dims, ivs, world), O.tiling_quality(dims, ivs, world))
    q = tdp.tdp_tiling_quality(dims, ivs, 4)
    assert (q["seams"], round(q["area_ratio"], 2), round(100 * q["imbalance"], 1)) == (3, 1.26, 6.8)


def test_quality_random_tilings_match_oracle():
    rng = np.random.default_rng(21)
    for _ in range(60):
        nd = int(rng.integers(1, 4))
        dims = [int(x) for x in rng.integers(1, 40, nd)]
        ivs = []
        for d in dims:
            k = int(rng.integers(1, 5))
            a = sorted(int(x) for x in rng.integers(0, d, k))
            ivs.append([(s, int(rng.integers(s + 1, d + 1))) for s in a])   # arbitrary, may overlap or leave gaps
        world = int(rng.integers(1, 9))
        _same_quality(tdp.tdp_tiling_quality(dims, ivs, world), O.tiling_quality(dims, ivs, world))


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_plan_quality_matches_oracle(name):
    wl = WORKLOADS[name]
    plan = tdp.tdp_plan_create(tdp.make_config(wl.batch, wl.channels, wl.shape, wl.tiling, wl.num_cond,
                                               in_dtype=wl.dtype))
    ivs = [O.split_by_count(d, n, o) for d, (n, o) in zip(wl.shape, wl.tiling)]
    for world in (1, 2, 4, 8):
        _same_quality(tdp.tdp_plan_quality(plan, world), O.tiling_quality(wl.shape, ivs, world))
    assert tdp.tdp_plan_quality(plan, 1)["area_ratio"] == pytest.approx(O.decoded_area_ratio(wl.shape, wl.tiling))


def test_quality_errors():
    with pytest.raises(tdp.TdpError):
        tdp.tdp_tiling_quality((10,), [[(3, 3)]], 1)          # empty interval
    with pytest.raises(tdp.TdpError):
        tdp.tdp_tiling_quality((10,), [[(0, 11)]], 1)         # past the axis
    with pytest.raises(tdp.TdpError):
        tdp.tdp_tiling_quality((10,), [[(0, 5)]], 0)          # no ranks
    with pytest.raises(tdp.TdpError):
        tdp.tdp_tiling_quality((10,) * 9, [[(0, 5)]] * 9, 1)  # too many axes
    lib = tdp.load_library()
    q = tdp.tdp_quality()
    assert lib.tdp_plan_quality(None, 1, ctypes.byref(q), None) == tdp.TDP_EINVAL
