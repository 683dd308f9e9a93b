"""Python binding of libtdp: tiled-data-parallel latent tiling on MI355X.

Thin ctypes layer over the C ABI declared in ``include/tdp.h``: the names are
the C names, and every step of the hot path runs in the library's HIP
kernels.  This module only marshals arguments: it checks tensors (device,
dtype, contiguity and size against the plan) before any pointer reaches the
library, so a wrong buffer raises here instead of reaching a kernel.

PyTorch supplies device memory and streams; nothing here computes.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB_PATH = os.path.join(_HERE, "libtdp.so")
# TDP_LIBRARY names another build to load instead, e.g. the host-only planner
# built with address and undefined-behaviour sanitizers for the CPU tests
# (build.py --host-sanitized); such a build may lack the device entry points.
LIB_PATH = os.environ.get("TDP_LIBRARY") or DEFAULT_LIB_PATH
DEVICE_FUNCTIONS = ("tdp_extract", "tdp_extract_noalloc", "tdp_set_lookback_polls", "tdp_pipeline_step",
                    "tdp_extract_positions", "tdp_extract_latent", "tdp_pipeline_latent_step", "tdp_blend",
                    "tdp_blend_tile", "tdp_blend_finish", "tdp_pixel_blend")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tdp.h")

# ---- constants (mirror include/tdp.h) --------------------------------------
TDP_OK = 0
TDP_EINVAL = -1
TDP_EGUARD = -2
TDP_ESHAPE = -3
TDP_EHIP = -4
TDP_F32 = 0
TDP_BF16 = 1
TDP_NORMALIZE_POSITIONS = 0x1
TDP_UNGUARDED = 0x2
TDP_MAX_TILES_PER_AXIS = 32
TDP_STATIC_SCRATCH_BYTES = 1 << 20

_DTYPES = {"f32": TDP_F32, "float32": TDP_F32, "bf16": TDP_BF16, "bfloat16": TDP_BF16}


class tdp_axis_tiling(ctypes.Structure):
    _fields_ = [("num_tiles", ctypes.c_int32), ("overlap", ctypes.c_int32)]


class tdp_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("channels", ctypes.c_int32),
        ("frames", ctypes.c_int32),
        ("height", ctypes.c_int32),
        ("width", ctypes.c_int32),
        ("num_cond", ctypes.c_int32),
        ("axis", tdp_axis_tiling * 3),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class tdp_tile_info(ctypes.Structure):
    _fields_ = [
        ("index", ctypes.c_int32),
        ("grid", ctypes.c_int32 * 3),
        ("origin", ctypes.c_int32 * 3),
        ("shape", ctypes.c_int32 * 3),
        ("gen_tokens", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("lat_offset", ctypes.c_int64),
        ("pos_offset", ctypes.c_int64),
        ("index_offset", ctypes.c_int64),
    ]


class tdp_sizes(ctypes.Structure):
    _fields_ = [
        ("num_slots", ctypes.c_int32),
        ("tile_lat_elems", ctypes.c_int64),
        ("tile_pos_floats", ctypes.c_int64),
        ("tile_index_ints", ctypes.c_int64),
        ("cond_row_ints", ctypes.c_int64),
        ("cond_k_ints", ctypes.c_int64),
        ("out_elems", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
    ]


class tdp_pixel_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("channels", ctypes.c_int32),
        ("frames", ctypes.c_int32),
        ("height", ctypes.c_int32),
        ("width", ctypes.c_int32),
        ("scale", ctypes.c_int32 * 2),
        ("axis", tdp_axis_tiling * 2),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
    ]


class tdp_pixel_tile(ctypes.Structure):
    _fields_ = [
        ("index", ctypes.c_int32),
        ("grid", ctypes.c_int32 * 2),
        ("origin", ctypes.c_int32 * 2),
        ("shape", ctypes.c_int32 * 2),
        ("offset", ctypes.c_int64),
        ("elems", ctypes.c_int64),
    ]


class tdp_quality(ctypes.Structure):
    _fields_ = [
        ("total_cells", ctypes.c_int64),
        ("grid_cells", ctypes.c_int64),
        ("largest_cells", ctypes.c_int64),
        ("seams", ctypes.c_int64),
        ("max_rank_cells", ctypes.c_int64),
        ("area_ratio", ctypes.c_double),
        ("largest_fraction", ctypes.c_double),
        ("imbalance", ctypes.c_double),
    ]


class TdpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [{status}]")
        self.status = status


_lib = None
HOST_ONLY = False  # the loaded build has the host planner only (no device entry points)


def load_library(path: str = LIB_PATH):
    """Load libtdp.so; raises ImportError when it has not been built."""
    global _lib, HOST_ONLY
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libtdp.so not found at {path}: build it first "
                          "(python overlap_tiling_trapezoidal_amd/build.py)")
    lib = ctypes.CDLL(path)
    vp, i32, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
    sig = {
        "tdp_plan_create": (ctypes.c_int, [ctypes.POINTER(tdp_config), ctypes.POINTER(vp)]),
        "tdp_plan_create_rank": (ctypes.c_int, [ctypes.POINTER(tdp_config), i32, i32, ctypes.POINTER(vp)]),
        "tdp_plan_local_tiles": (ctypes.c_int, [vp, i32p, i32p, i32p]),
        "tdp_plan_destroy": (None, [vp]),
        "tdp_plan_num_tiles": (ctypes.c_int, [vp, i32p]),
        "tdp_plan_intervals": (ctypes.c_int, [vp, ctypes.c_int, i32p, i32p]),
        "tdp_plan_window": (ctypes.c_int, [vp, ctypes.c_int, i32, ctypes.POINTER(ctypes.c_float)]),
        "tdp_plan_tile": (ctypes.c_int, [vp, i32, ctypes.POINTER(tdp_tile_info)]),
        "tdp_plan_cell_tiles": (ctypes.c_int, [vp, ctypes.c_int, i32, i32p, i32p]),
        "tdp_plan_sizes": (ctypes.c_int, [vp, ctypes.POINTER(tdp_sizes)]),
        "tdp_plan_tile_rank": (ctypes.c_int, [vp, i32, i32, i32p]),
        "tdp_tiling_quality": (ctypes.c_int, [i32, i32p, i32p, i32p, i32p, i32, ctypes.POINTER(tdp_quality),
                                              ctypes.POINTER(ctypes.c_int64)]),
        "tdp_plan_quality": (ctypes.c_int, [vp, i32, ctypes.POINTER(tdp_quality), ctypes.POINTER(ctypes.c_int64)]),
        "tdp_extract": (ctypes.c_int, [vp] * 11),
        "tdp_extract_noalloc": (ctypes.c_int, [vp] * 10),
        "tdp_set_lookback_polls": (ctypes.c_int, [i32]),
        "tdp_pipeline_step": (ctypes.c_int, [vp] * 15),
        "tdp_extract_positions": (ctypes.c_int, [vp] * 9),
        "tdp_extract_latent": (ctypes.c_int, [vp] * 5),
        "tdp_pipeline_latent_step": (ctypes.c_int, [vp] * 9),
        "tdp_blend": (ctypes.c_int, [vp] * 6),
        "tdp_blend_tile": (ctypes.c_int, [vp, i32, vp, vp, vp, vp, vp]),
        "tdp_blend_finish": (ctypes.c_int, [vp] * 4),
        "tdp_pixel_plan_create": (ctypes.c_int, [ctypes.POINTER(tdp_pixel_config), ctypes.POINTER(vp)]),
        "tdp_pixel_plan_destroy": (None, [vp]),
        "tdp_pixel_plan_tile": (ctypes.c_int, [vp, i32, ctypes.POINTER(tdp_pixel_tile)]),
        "tdp_pixel_plan_sizes": (ctypes.c_int, [vp, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                                i32p]),
        "tdp_pixel_blend": (ctypes.c_int, [vp] * 4),
        "tdp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "tdp_last_error": (ctypes.c_char_p, []),
    }
    missing = [name for name in sig if not hasattr(lib, name)]
    if missing and (path == DEFAULT_LIB_PATH or any(m not in DEVICE_FUNCTIONS for m in missing)):
        raise ImportError(f"{path} does not export {', '.join(missing)}")
    for name, (res, args) in sig.items():
        if name in missing:
            continue
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    HOST_ONLY = bool(missing)
    _lib = lib
    return lib


def _header_functions_in(path: str) -> list[str]:
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tdp_[a-z_]+)\s*\(", text)))


def header_functions(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/tdp.h declares."""
    return _header_functions_in(path)


def _check(status: int):
    if status != TDP_OK:
        lib = load_library()
        raise TdpError(status, lib.tdp_last_error().decode())


# ---- plan -----------------------------------------------------------------

def make_config(batch, channels, shape, tiling, num_cond=0, in_dtype="bf16", out_dtype=None,
                normalize=True, unguarded=False) -> tdp_config:
    """Fill a tdp_config.  ``shape`` = (F, H, W); ``tiling`` = ((n, o),) * 3."""
    cfg = tdp_config()
    cfg.batch, cfg.channels = batch, channels
    cfg.frames, cfg.height, cfg.width = shape
    cfg.num_cond = num_cond
    for d, (n, o) in enumerate(tiling):
        cfg.axis[d].num_tiles, cfg.axis[d].overlap = n, o
    cfg.in_dtype = _DTYPES[in_dtype] if isinstance(in_dtype, str) else in_dtype
    out_dtype = in_dtype if out_dtype is None else out_dtype
    cfg.out_dtype = _DTYPES[out_dtype] if isinstance(out_dtype, str) else out_dtype
    cfg.flags = (TDP_NORMALIZE_POSITIONS if normalize else 0) | (TDP_UNGUARDED if unguarded else 0)
    return cfg


class Plan:
    """Owns a tdp_plan handle (host memory only)."""

    def __init__(self, handle: int, cfg: tdp_config):
        self._h = ctypes.c_void_p(handle)
        self.cfg = cfg

    @property
    def handle(self):
        if not self._h:
            raise ValueError("plan was destroyed")
        return self._h

    def destroy(self):
        if self._h:
            load_library().tdp_plan_destroy(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    # derived geometry
    @property
    def shape(self):
        return (self.cfg.frames, self.cfg.height, self.cfg.width)

    @property
    def tokens(self):
        F, H, W = self.shape
        return F * H * W


def tdp_plan_create(cfg: tdp_config) -> Plan:
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.tdp_plan_create(ctypes.byref(cfg), ctypes.byref(h)))
    return Plan(h.value, cfg)


def tdp_plan_create_rank(cfg: tdp_config, world: int, rank: int) -> Plan:
    """Plan of rank ``rank``'s round-robin share of the tiles over ``world`` ranks."""
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.tdp_plan_create_rank(ctypes.byref(cfg), world, rank, ctypes.byref(h)))
    return Plan(h.value, cfg)


def tdp_plan_local_tiles(plan: Plan) -> tuple[int, int, int]:
    """(world, rank, number of tiles the plan holds)."""
    w, r, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().tdp_plan_local_tiles(plan.handle, ctypes.byref(w), ctypes.byref(r), ctypes.byref(n)))
    return w.value, r.value, n.value


def held_tiles(plan: Plan) -> list[int]:
    """Tile indices the plan holds, in slot order (t = rank + slot * world)."""
    world, rank, n = tdp_plan_local_tiles(plan)
    return [rank + j * world for j in range(n)]


def tdp_plan_destroy(plan: Plan):
    plan.destroy()


def tdp_plan_num_tiles(plan: Plan) -> int:
    n = ctypes.c_int32()
    _check(load_library().tdp_plan_num_tiles(plan.handle, ctypes.byref(n)))
    return n.value


def tdp_plan_intervals(plan: Plan, axis: int) -> list[tuple[int, int]]:
    n = plan.cfg.axis[axis].num_tiles if 0 <= axis < 3 else 1
    starts = (ctypes.c_int32 * max(n, 1))()
    ends = (ctypes.c_int32 * max(n, 1))()
    _check(load_library().tdp_plan_intervals(plan.handle, axis, starts, ends))
    return [(starts[i], ends[i]) for i in range(n)]


def tdp_plan_window(plan: Plan, axis: int, i: int):
    import numpy as np
    ivs = tdp_plan_intervals(plan, axis)
    if not 0 <= i < len(ivs):
        raise IndexError(i)
    size = ivs[i][1] - ivs[i][0]
    buf = (ctypes.c_float * size)()
    _check(load_library().tdp_plan_window(plan.handle, axis, i, buf))
    return np.ctypeslib.as_array(buf).copy()


def tdp_plan_cell_tiles(plan: Plan, axis: int, x: int) -> list[int]:
    tiles = (ctypes.c_int32 * 2)()
    n = ctypes.c_int32()
    _check(load_library().tdp_plan_cell_tiles(plan.handle, axis, x, tiles, ctypes.byref(n)))
    return [tiles[i] for i in range(n.value)]


def tdp_plan_tile(plan: Plan, t: int) -> tdp_tile_info:
    info = tdp_tile_info()
    _check(load_library().tdp_plan_tile(plan.handle, t, ctypes.byref(info)))
    return info


def tdp_plan_sizes(plan: Plan) -> tdp_sizes:
    s = tdp_sizes()
    _check(load_library().tdp_plan_sizes(plan.handle, ctypes.byref(s)))
    return s


def tdp_plan_tile_rank(plan: Plan, t: int, world: int) -> int:
    r = ctypes.c_int32()
    _check(load_library().tdp_plan_tile_rank(plan.handle, t, world, ctypes.byref(r)))
    return r.value


def tdp_status_string(status: int) -> str:
    return load_library().tdp_status_string(status).decode()


def tdp_last_error() -> str:
    return load_library().tdp_last_error().decode()


# ---- device buffers (torch) ----------------------------------------------

def _torch_dtype(code: int):
    import torch
    return torch.bfloat16 if code == TDP_BF16 else torch.float32


def _ptr(t, name, dtype, numel, device):
    """Pointer of a CUDA tensor after checking it can hold ``numel`` elements."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on {device or 'a GPU'}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _quality_dict(q: tdp_quality, ranks) -> dict:
    d = {name: getattr(q, name) for name, _ in tdp_quality._fields_}
    d["rank_cells"] = list(ranks)
    return d


def tdp_tiling_quality(dims, intervals, world: int) -> dict:
    """Cost figures of a tiling given per-axis [start, end) intervals."""
    nd = len(dims)
    arr = lambda xs: (ctypes.c_int32 * max(1, len(xs)))(*xs)  # noqa: E731
    starts = [a for ivs in intervals for a, _ in ivs]
    ends = [b for ivs in intervals for _, b in ivs]
    q = tdp_quality()
    ranks = (ctypes.c_int64 * max(1, world))()
    _check(load_library().tdp_tiling_quality(nd, arr(list(dims)), arr([len(v) for v in intervals]), arr(starts),
                                              arr(ends), world, ctypes.byref(q), ranks))
    return _quality_dict(q, ranks[:world])


def tdp_plan_quality(plan: Plan, world: int) -> dict:
    """Cost figures of a plan's tiles on ``world`` round-robin ranks."""
    q = tdp_quality()
    ranks = (ctypes.c_int64 * max(1, world))()
    _check(load_library().tdp_plan_quality(plan.handle, world, ctypes.byref(q), ranks))
    return _quality_dict(q, ranks[:world])


def allocate_extract_outputs(plan: Plan, device="cuda"):
    """Caller-owned buffers for tdp_extract / tdp_blend, sized by the plan
    (the keys are tdp_extract's argument names)."""
    import torch
    s = tdp_plan_sizes(plan)
    dev = torch.device(device)
    return {
        "tile_lat": torch.empty(s.tile_lat_elems, dtype=_torch_dtype(plan.cfg.in_dtype), device=dev),
        "tile_pos": torch.empty(s.tile_pos_floats, dtype=torch.float32, device=dev),
        "tile_index": torch.empty(s.tile_index_ints, dtype=torch.int32, device=dev),
        "tile_count": torch.empty(max(s.num_slots, 1), dtype=torch.int32, device=dev),
        "cond_row": torch.empty(max(s.cond_row_ints, 1), dtype=torch.int32, device=dev),
        "cond_k": torch.empty(max(s.cond_k_ints, 1), dtype=torch.int32, device=dev),
        "workspace": torch.empty(max(s.workspace_bytes, 1), dtype=torch.uint8, device=dev),
    }


def allocate_output(plan: Plan, device="cuda"):
    import torch
    s = tdp_plan_sizes(plan)
    c = plan.cfg
    return torch.empty(s.out_elems, dtype=_torch_dtype(c.out_dtype),
                       device=torch.device(device)).view(c.batch, plan.tokens + c.num_cond, c.channels)


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _extract_args(plan: Plan, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k):
    import torch
    c = plan.cfg
    s = tdp_plan_sizes(plan)
    rows = plan.tokens + c.num_cond
    dev = latent.device
    none = ctypes.c_void_p(None)
    return [
        plan.handle,
        _ptr(latent, "latent", _torch_dtype(c.in_dtype), c.batch * rows * c.channels, dev),
        _ptr(pos, "pos", torch.float32, c.batch * 3 * rows * 2, dev),
        _ptr(tile_lat, "tile_lat", _torch_dtype(c.in_dtype), s.tile_lat_elems, dev),
        _ptr(tile_pos, "tile_pos", torch.float32, s.tile_pos_floats, dev),
        _ptr(tile_index, "tile_index", torch.int32, s.tile_index_ints, dev),
        _ptr(tile_count, "tile_count", torch.int32, s.num_slots, dev),
        _ptr(cond_row, "cond_row", torch.int32, s.cond_row_ints, dev) if c.num_cond else none,
        _ptr(cond_k, "cond_k", torch.int32, s.cond_k_ints, dev) if c.num_cond else none,
    ]


def tdp_extract(plan: Plan, latent, pos, tile_lat, tile_pos, tile_index, tile_count,
                cond_row=None, cond_k=None, workspace=None, stream=None):
    """Enqueue the tile gather on ``stream`` (default: torch's current stream)."""
    import torch
    s = tdp_plan_sizes(plan)
    dev = latent.device
    args = _extract_args(plan, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k)
    args.append(_ptr(workspace, "workspace", torch.uint8, s.workspace_bytes, dev) if s.workspace_bytes
                else ctypes.c_void_p(None))
    args.append(_stream_handle(stream, dev))
    _check(load_library().tdp_extract(*args))


def tdp_set_lookback_polls(polls: int):
    """Reads of an unpublished look-back flag before a conditioning selection
    wave counts that chunk itself (process-wide; results do not depend on it)."""
    _check(load_library().tdp_set_lookback_polls(int(polls)))


def tdp_extract_noalloc(plan: Plan, latent, pos, tile_lat, tile_pos, tile_index, tile_count,
                        cond_row=None, cond_k=None, stream=None):
    """tdp_extract with the library's static per-GPU workspace in place of a
    caller's (for callers that cannot allocate device memory; calls that
    overlap on one GPU race)."""
    args = _extract_args(plan, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k)
    args.append(_stream_handle(stream, latent.device))
    _check(load_library().tdp_extract_noalloc(*args))


def tdp_blend(plan: Plan, tile_out, cond_row, cond_k, out, stream=None):
    """Enqueue the blend of tile outputs into ``out`` on ``stream``
    (``cond_row`` and ``cond_k`` from tdp_extract; ignored when Nc == 0)."""
    import torch
    c = plan.cfg
    s = tdp_plan_sizes(plan)
    dev = tile_out.device
    none = ctypes.c_void_p(None)
    args = [
        plan.handle,
        _ptr(tile_out, "tile_out", _torch_dtype(c.in_dtype), s.tile_lat_elems, dev),
        _ptr(cond_row, "cond_row", torch.int32, s.cond_row_ints, dev) if c.num_cond else none,
        _ptr(cond_k, "cond_k", torch.int32, s.cond_k_ints, dev) if c.num_cond else none,
        _ptr(out, "out", _torch_dtype(c.out_dtype), s.out_elems, dev),
        _stream_handle(stream, dev),
    ]
    _check(load_library().tdp_blend(*args))


def tdp_pipeline_step(plan: Plan, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row=None,
                      cond_k=None, workspace=None, *, tile_out, blend_cond_row=None, blend_cond_k=None, out,
                      stream=None):
    """Enqueue tdp_extract of ``latent`` and tdp_blend of ``tile_out`` (an
    earlier latent's tile outputs, none of this extract's buffers) as one
    step, one launch where the plan allows."""
    import torch
    c = plan.cfg
    s = tdp_plan_sizes(plan)
    dev = latent.device
    none = ctypes.c_void_p(None)
    args = _extract_args(plan, latent, pos, tile_lat, tile_pos, tile_index, tile_count, cond_row, cond_k)
    args.append(_ptr(workspace, "workspace", torch.uint8, s.workspace_bytes, dev) if s.workspace_bytes else none)
    args += [
        _ptr(tile_out, "tile_out", _torch_dtype(c.in_dtype), s.tile_lat_elems, dev),
        _ptr(blend_cond_row, "blend_cond_row", torch.int32, s.cond_row_ints, dev) if c.num_cond else none,
        _ptr(blend_cond_k, "blend_cond_k", torch.int32, s.cond_k_ints, dev) if c.num_cond else none,
        _ptr(out, "out", _torch_dtype(c.out_dtype), s.out_elems, dev),
        _stream_handle(stream, dev),
    ]
    _check(load_library().tdp_pipeline_step(*args))


def tdp_extract_positions(plan: Plan, pos, tile_pos, tile_index, tile_count, cond_row=None, cond_k=None,
                          workspace=None, stream=None):
    """Enqueue what tdp_extract writes except the latent rows (tile positions,
    index map, counts, cond_row, cond_k): once per positions set."""
    import torch
    c = plan.cfg
    s = tdp_plan_sizes(plan)
    rows = plan.tokens + c.num_cond
    dev = pos.device
    none = ctypes.c_void_p(None)
    args = [
        plan.handle,
        _ptr(pos, "pos", torch.float32, c.batch * 3 * rows * 2, dev),
        _ptr(tile_pos, "tile_pos", torch.float32, s.tile_pos_floats, dev),
        _ptr(tile_index, "tile_index", torch.int32, s.tile_index_ints, dev),
        _ptr(tile_count, "tile_count", torch.int32, s.num_slots, dev),
        _ptr(cond_row, "cond_row", torch.int32, s.cond_row_ints, dev) if c.num_cond else none,
        _ptr(cond_k, "cond_k", torch.int32, s.cond_k_ints, dev) if c.num_cond else none,
        _ptr(workspace, "workspace", torch.uint8, s.workspace_bytes, dev) if s.workspace_bytes else none,
        _stream_handle(stream, dev),
    ]
    _check(load_library().tdp_extract_positions(*args))


def _gather_args(plan: Plan, latent, cond_row, tile_lat):
    import torch
    c = plan.cfg
    s = tdp_plan_sizes(plan)
    rows = plan.tokens + c.num_cond
    dev = latent.device
    return [
        plan.handle,
        _ptr(latent, "latent", _torch_dtype(c.in_dtype), c.batch * rows * c.channels, dev),
        _ptr(cond_row, "cond_row", torch.int32, s.cond_row_ints, dev) if c.num_cond else ctypes.c_void_p(None),
        _ptr(tile_lat, "tile_lat", _torch_dtype(c.in_dtype), s.tile_lat_elems, dev),
    ]


def tdp_extract_latent(plan: Plan, latent, cond_row, tile_lat, stream=None):
    """Enqueue the latent rows of every held tile into ``tile_lat``, at the
    slot rows ``cond_row`` (from tdp_extract_positions) gives."""
    args = _gather_args(plan, latent, cond_row, tile_lat)
    args.append(_stream_handle(stream, latent.device))
    _check(load_library().tdp_extract_latent(*args))


def tdp_pipeline_latent_step(plan: Plan, latent, cond_row, tile_lat, *, tile_out, blend_cond_row=None,
                             blend_cond_k=None, out, stream=None):
    """Enqueue tdp_extract_latent of ``latent`` and tdp_blend of ``tile_out``
    as one step (one launch for whole plans)."""
    import torch
    c = plan.cfg
    s = tdp_plan_sizes(plan)
    dev = latent.device
    none = ctypes.c_void_p(None)
    args = _gather_args(plan, latent, cond_row, tile_lat)
    args += [
        _ptr(tile_out, "tile_out", _torch_dtype(c.in_dtype), s.tile_lat_elems, dev),
        _ptr(blend_cond_row, "blend_cond_row", torch.int32, s.cond_row_ints, dev) if c.num_cond else none,
        _ptr(blend_cond_k, "blend_cond_k", torch.int32, s.cond_k_ints, dev) if c.num_cond else none,
        _ptr(out, "out", _torch_dtype(c.out_dtype), s.out_elems, dev),
        _stream_handle(stream, dev),
    ]
    _check(load_library().tdp_pipeline_latent_step(*args))


def allocate_accumulator(plan: Plan, device="cuda"):
    """fp32 (B, N+Nc, C) accumulator for the streaming blend."""
    import torch
    c = plan.cfg
    return torch.empty((c.batch, plan.tokens + c.num_cond, c.channels), dtype=torch.float32,
                       device=torch.device(device))


def tdp_blend_tile(plan: Plan, t: int, tile_out, cond_row, cond_k, acc, stream=None):
    """Enqueue the streaming blend of tile t's slot ``tile_out`` into ``acc``."""
    import torch
    c = plan.cfg
    info = tdp_plan_tile(plan, t)
    dev = acc.device
    rows = plan.tokens + c.num_cond
    none = ctypes.c_void_p(None)
    _check(load_library().tdp_blend_tile(
        plan.handle, t,
        _ptr(tile_out, "tile_out", _torch_dtype(c.in_dtype), c.batch * info.capacity * c.channels, dev),
        _ptr(cond_row, "cond_row", torch.int32, c.num_cond * tdp_plan_num_tiles(plan), dev) if c.num_cond else none,
        _ptr(cond_k, "cond_k", torch.int32, c.num_cond, dev) if c.num_cond else none,
        _ptr(acc, "acc", torch.float32, c.batch * rows * c.channels, dev),
        _stream_handle(stream, dev)))


def tdp_blend_finish(plan: Plan, acc, out, stream=None):
    """Enqueue the rounding of ``acc`` to the output dtype into ``out``."""
    import torch
    c = plan.cfg
    n = c.batch * (plan.tokens + c.num_cond) * c.channels
    dev = acc.device
    _check(load_library().tdp_blend_finish(plan.handle, _ptr(acc, "acc", torch.float32, n, dev),
                                           _ptr(out, "out", _torch_dtype(c.out_dtype), n, dev),
                                           _stream_handle(stream, dev)))


def tile_views(plan: Plan, buffers, counts=None):
    """Per-slot torch views into the tile-major buffers (every tile, or a
    rank plan's own tiles in slot order).

    ``counts`` (host list of tile_count) trims each view to its used rows;
    without it the views span the whole slot.  Returns a list of dicts with
    ``lat`` (B, rows, C), ``pos`` (B, 3, rows, 2), ``index`` (rows,) and
    ``info`` (its ``index`` is the tile).
    """
    c = plan.cfg
    views = []
    for j, t in enumerate(held_tiles(plan)):
        info = tdp_plan_tile(plan, t)
        cap = info.capacity
        used = cap if counts is None else int(counts[j])
        lat = buffers["tile_lat"][info.lat_offset: info.lat_offset + c.batch * cap * c.channels]
        pos = buffers["tile_pos"][info.pos_offset: info.pos_offset + c.batch * 6 * cap]
        idx = buffers["tile_index"][info.index_offset: info.index_offset + cap]
        views.append({
            "lat": lat.view(c.batch, cap, c.channels)[:, :used],
            "pos": pos.view(c.batch, 3, cap, 2)[:, :, :used],
            "index": idx[:used],
            "info": info,
        })
    return views


# ---------------------------------------------------------------------------
# Spatial blend of decoded pixel tiles
# ---------------------------------------------------------------------------

def make_pixel_config(batch, channels, frames, latent_hw, scale_hw, tiling_hw, in_dtype="bf16",
                      out_dtype=None) -> tdp_pixel_config:
    """Fill a tdp_pixel_config; ``tiling_hw`` = ((n_h, o_h), (n_w, o_w)) in latent cells."""
    cfg = tdp_pixel_config()
    cfg.batch, cfg.channels, cfg.frames = batch, channels, frames
    cfg.height, cfg.width = latent_hw
    for a in range(2):
        cfg.scale[a] = scale_hw[a]
        cfg.axis[a].num_tiles, cfg.axis[a].overlap = tiling_hw[a]
    code = lambda d: _DTYPES[d] if isinstance(d, str) else d  # noqa: E731
    cfg.in_dtype = code(in_dtype)
    cfg.out_dtype = code(in_dtype if out_dtype is None else out_dtype)
    return cfg


class PixelPlan:
    """Owning handle of a tdp_pixel_plan."""

    def __init__(self, handle, cfg):
        self.handle, self.cfg = handle, cfg

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.tdp_pixel_plan_destroy(self.handle)
            self.handle = None


def tdp_pixel_plan_create(cfg: tdp_pixel_config) -> PixelPlan:
    h = ctypes.c_void_p()
    _check(load_library().tdp_pixel_plan_create(ctypes.byref(cfg), ctypes.byref(h)))
    return PixelPlan(h, cfg)


def tdp_pixel_plan_tile(plan: PixelPlan, t: int) -> tdp_pixel_tile:
    info = tdp_pixel_tile()
    _check(load_library().tdp_pixel_plan_tile(plan.handle, t, ctypes.byref(info)))
    return info


def tdp_pixel_plan_sizes(plan: PixelPlan):
    """(tile buffer elements, output elements, tile count)."""
    a, b, n = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(load_library().tdp_pixel_plan_sizes(plan.handle, ctypes.byref(a), ctypes.byref(b), ctypes.byref(n)))
    return a.value, b.value, n.value


def tdp_pixel_blend(plan: PixelPlan, tiles, out, stream=None):
    """Enqueue the blend of packed pixel tiles into ``out`` (B, C, frames, H*s_h, W*s_w)."""
    c = plan.cfg
    tile_elems, out_elems, _ = tdp_pixel_plan_sizes(plan)
    dev = out.device
    _check(load_library().tdp_pixel_blend(plan.handle, _ptr(tiles, "tiles", _torch_dtype(c.in_dtype), tile_elems, dev),
                                          _ptr(out, "out", _torch_dtype(c.out_dtype), out_elems, dev),
                                          _stream_handle(stream, dev)))
