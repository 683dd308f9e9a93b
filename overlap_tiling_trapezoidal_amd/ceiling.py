"""ctypes binding of libtdp_ceiling.so (declared in include/tdp_ceiling.h):
HBM ceilings of plain hand-written streaming kernels, for the measurement
script.  Not part of the tiled hot path."""
from __future__ import annotations

import ctypes
import os

from . import _header_functions_in

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtdp_ceiling.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tdp_ceiling.h")

MODES = {"copy_nt": 0, "copy_device_scope": 1, "read": 2, "write": 3, "gather": 4, "scatter": 5}
# bytes one pass moves, as a multiple of its `nbytes` argument
MOVED = {"copy_nt": 2, "copy_device_scope": 2, "read": 1, "write": 1, "gather": 3, "scatter": 3}
_lib = None


def load_library(path: str = LIB_PATH):
    """Load libtdp_ceiling.so; raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libtdp_ceiling.so not found at {path}: build it first "
                          "(python overlap_tiling_trapezoidal_amd/build.py)")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.tdp_ceiling_run.restype = ctypes.c_int
    lib.tdp_ceiling_run.argtypes = [ctypes.c_int, vp, vp, vp, ctypes.c_size_t, vp]
    _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH) -> list[str]:
    return _header_functions_in(path)


def run(mode: str, src, dst, sink, nbytes: int, stream) -> None:
    """Enqueue one pass of `mode` over `nbytes` on `stream` (torch tensors)."""
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else None)  # noqa: E731
    st = load_library().tdp_ceiling_run(MODES[mode], ptr(src), ptr(dst), ptr(sink), nbytes,
                                        ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise RuntimeError(f"tdp_ceiling_run({mode}) failed with status {st}")
