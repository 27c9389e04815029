"""ctypes declarations for libgsraster.so (the C ABI in include/gsraster.h).

The library is built in-tree by ``differentiable_tile_rasterization_amd.build``;
loading fails with an ImportError-like RuntimeError if it is missing. There is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgsraster.so")

GS_OK = 0
GS_ERR_INVALID_ARG = 1
GS_ERR_CAPACITY = 2
GS_ERR_HIP = 3
GS_ERR_UNSUPPORTED = 4
GS_FLAG_ACCUM_WEIGHT = 1
GS_FLAG_WALK_ADD = 2
GS_FLAG_WALK_STORE = 4
GS_FLAG_WALK_DEFER = 8

STATUS_NAMES = {0: "GS_OK", 1: "GS_ERR_INVALID_ARG", 2: "GS_ERR_CAPACITY", 3: "GS_ERR_HIP",
                4: "GS_ERR_UNSUPPORTED"}

# Every symbol include/gsraster.h declares.
EXPORTS = ["gs_last_error", "gs_version", "gs_bin_tiles_workspace_size", "gs_bin_tiles",
           "gs_rasterize_fwd_workspace_size", "gs_rasterize_fwd", "gs_rasterize_fwd_depth",
           "gs_rasterize_bwd_workspace_size", "gs_rasterize_bwd", "gs_rasterize_bwd_depth",
           "gs_rasterize_bwd_timed", "gs_rasterize_bwd_noalloc_capacity", "gs_rasterize_bwd_noalloc"]

_lib = None


def load() -> ctypes.CDLL:
    """Load libgsraster.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m differentiable_tile_rasterization_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    i64 = ctypes.c_int64
    u32 = ctypes.c_uint32
    sz = ctypes.c_size_t
    lib.gs_last_error.argtypes = []
    lib.gs_last_error.restype = ctypes.c_char_p
    lib.gs_version.argtypes = []
    lib.gs_version.restype = ctypes.c_int
    lib.gs_bin_tiles_workspace_size.argtypes = [i32, i64, i32, i32]
    lib.gs_bin_tiles_workspace_size.restype = sz
    lib.gs_bin_tiles.argtypes = [i32, P, P, P, P, P, i32, i32, i64, P, P, P, ctypes.POINTER(i64),
                                 ctypes.POINTER(i64), P, sz, P]
    lib.gs_bin_tiles.restype = ctypes.c_int
    lib.gs_rasterize_fwd_workspace_size.argtypes = [i32]
    lib.gs_rasterize_fwd_workspace_size.restype = sz
    lib.gs_rasterize_fwd.argtypes = [i32, P, P, P, P, P, i32, i32, P, P, i64, P, P, P, P, P, sz, P]
    lib.gs_rasterize_fwd.restype = ctypes.c_int
    lib.gs_rasterize_fwd_depth.argtypes = [i32, P, P, P, P, P, P, i32, i32, P, P, i64, P, P, P, P, P, P, P,
                                           P, sz, P]
    lib.gs_rasterize_fwd_depth.restype = ctypes.c_int
    lib.gs_rasterize_bwd_workspace_size.argtypes = [i32, i64, i32, i32]
    lib.gs_rasterize_bwd_workspace_size.restype = sz
    lib.gs_rasterize_bwd.argtypes = [i32, P, P, P, P, P, P, i32, i32, P, P, P, i64, i64, P, P, P,
                                     P, P, P, P, P, u32, P, sz, P]
    lib.gs_rasterize_bwd.restype = ctypes.c_int
    lib.gs_rasterize_bwd_depth.argtypes = [i32, P, P, P, P, P, P, P, i32, i32, P, P, P, i64, i64, P, P, P, P,
                                           P, P, P, P, P, P, P, P, P, u32, P, sz, P]
    lib.gs_rasterize_bwd_depth.restype = ctypes.c_int
    lib.gs_rasterize_bwd_timed.argtypes = lib.gs_rasterize_bwd.argtypes + [ctypes.POINTER(P)]
    lib.gs_rasterize_bwd_timed.restype = ctypes.c_int
    lib.gs_rasterize_bwd_noalloc_capacity.argtypes = []
    lib.gs_rasterize_bwd_noalloc_capacity.restype = sz
    lib.gs_rasterize_bwd_noalloc.argtypes = lib.gs_rasterize_bwd.argtypes[:23] + [P]
    lib.gs_rasterize_bwd_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


class GsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != GS_OK:
        raise GsError(status, load().gs_last_error().decode(errors="replace"))
