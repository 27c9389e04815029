"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before any device work (these
paths never touch a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from differentiable_tile_rasterization_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsraster.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*]+\s+\**(gs_\w+)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", out, re.M))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version():
    assert _lib.load().gs_version() >= 100


def test_workspace_size_grows_with_capacity():
    lib = _lib.load()
    a = lib.gs_bin_tiles_workspace_size(1000, 0, 64, 64)
    b = lib.gs_bin_tiles_workspace_size(1000, 100000, 64, 64)
    assert 0 < a < b
    assert lib.gs_bin_tiles_workspace_size(-1, 0, 64, 64) == 0


def _fwd(lib, n=1, w=64, h=64, ptr=1, nul=None, ws=256, wsb=1 << 20, n_isect=0):
    p = ctypes.c_void_p(ptr)
    return lib.gs_rasterize_fwd(n, p, p, p, p, nul, w, h, p, p, n_isect, p, p, p, nul, ctypes.c_void_p(ws), wsb, None)


def test_fwd_rejects_bad_arguments():
    lib = _lib.load()
    assert _fwd(lib, n=-1) == _lib.GS_ERR_INVALID_ARG
    assert b"n = -1" in lib.gs_last_error()
    assert _fwd(lib, w=0) == _lib.GS_ERR_INVALID_ARG
    assert _fwd(lib, h=40000) == _lib.GS_ERR_INVALID_ARG
    assert _fwd(lib, ptr=0) == _lib.GS_ERR_INVALID_ARG
    assert _fwd(lib, n=10, wsb=lib.gs_rasterize_fwd_workspace_size(10) - 1) == _lib.GS_ERR_INVALID_ARG
    assert b"workspace" in lib.gs_last_error()
    assert _fwd(lib, ws=128) == _lib.GS_ERR_INVALID_ARG
    assert _fwd(lib, n_isect=-1) == _lib.GS_ERR_INVALID_ARG
    assert b"n_isect" in lib.gs_last_error()
    assert _fwd(lib, n_isect=1 << 31) == _lib.GS_ERR_INVALID_ARG
    p = ctypes.c_void_p(1)
    # a pair count with no pair list
    assert lib.gs_rasterize_fwd(1, p, p, p, p, None, 8, 8, p, None, 5, p, p, p, None, ctypes.c_void_p(256),
                                1 << 20, None) == _lib.GS_ERR_INVALID_ARG
    assert b"sorted_ids" in lib.gs_last_error()
    assert lib.gs_rasterize_fwd_workspace_size(1000) >= 48 * 1000


def test_bwd_rejects_bad_arguments():
    lib = _lib.load()
    p = ctypes.c_void_p(1)

    def call(n=1, w=8, h=8, flags=0, aw=None, grad=p, n_isect=0, n_slots=None, ws=None, wsb=0):
        n_slots = n_isect if n_slots is None else n_slots
        return lib.gs_rasterize_bwd(n, p, p, p, p, p, None, w, h, p, p, p, n_isect, n_slots, p, p, p, grad, grad,
                                    grad, grad, aw, flags, ws, wsb, None)
    assert call(n=-5) == _lib.GS_ERR_INVALID_ARG
    assert call(flags=0x80) == _lib.GS_ERR_INVALID_ARG
    assert b"unknown flags" in lib.gs_last_error()
    for two in (_lib.GS_FLAG_WALK_ADD | _lib.GS_FLAG_WALK_STORE, _lib.GS_FLAG_WALK_ADD | _lib.GS_FLAG_WALK_DEFER,
                _lib.GS_FLAG_WALK_STORE | _lib.GS_FLAG_WALK_DEFER):
        assert call(flags=two) == _lib.GS_ERR_INVALID_ARG
        assert b"more than one walk flag" in lib.gs_last_error()
    assert call(flags=0x10) == _lib.GS_ERR_INVALID_ARG
    assert call(flags=_lib.GS_FLAG_ACCUM_WEIGHT, aw=None) == _lib.GS_ERR_INVALID_ARG
    assert b"accum_weight" in lib.gs_last_error()
    assert call(grad=ctypes.c_void_p(0)) == _lib.GS_ERR_INVALID_ARG
    assert call(w=-3) == _lib.GS_ERR_INVALID_ARG
    assert call(n_isect=-1) == _lib.GS_ERR_INVALID_ARG
    assert call(n_isect=1 << 31) == _lib.GS_ERR_INVALID_ARG
    # the slot count: at least the pair count, at most 2^31 - 1
    assert call(n_isect=10, n_slots=9) == _lib.GS_ERR_INVALID_ARG
    assert b"n_slots" in lib.gs_last_error()
    assert call(n_isect=10, n_slots=1 << 31) == _lib.GS_ERR_INVALID_ARG
    assert b"n_slots" in lib.gs_last_error()
    need = lib.gs_rasterize_bwd_workspace_size(1, 100, 8, 8)
    assert need >= 100 * 49 + 64
    assert call(n_isect=100, ws=None, wsb=need) == _lib.GS_ERR_INVALID_ARG
    assert b"workspace" in lib.gs_last_error()
    assert call(n_isect=100, ws=ctypes.c_void_p(256), wsb=need - 1) == _lib.GS_ERR_INVALID_ARG
    assert call(n_isect=100, ws=ctypes.c_void_p(300), wsb=need) == _lib.GS_ERR_INVALID_ARG
    assert b"aligned" in lib.gs_last_error()
    # the workspace is sized by the slots, not the pairs
    assert call(n_isect=10, n_slots=100, ws=ctypes.c_void_p(256),
                wsb=lib.gs_rasterize_bwd_workspace_size(1, 10, 8, 8)) == _lib.GS_ERR_INVALID_ARG
    assert b"workspace" in lib.gs_last_error()


def test_bwd_timed_rejects_bad_arguments():
    lib = _lib.load()
    p = ctypes.c_void_p(1)

    def call(events, n=-5):
        return lib.gs_rasterize_bwd_timed(n, p, p, p, p, p, None, 8, 8, p, p, p, 0, 0, p, p, p, p, p, p, p, None,
                                          0, None, 0, None, events)
    assert call(None) == _lib.GS_ERR_INVALID_ARG
    assert b"events" in lib.gs_last_error()
    # the plain argument checks come first, before any event is recorded
    assert call((ctypes.c_void_p * 4)(1, 1, 1, 1)) == _lib.GS_ERR_INVALID_ARG
    assert b"n = -5" in lib.gs_last_error()


def test_bin_rejects_bad_arguments():
    lib = _lib.load()
    p = ctypes.c_void_p(256)
    cnt = ctypes.c_int64(0)
    def call(n=4, w=64, h=64, cap=16, ws=p, wsb=1 << 20, ncnt=True, offs=p, conics=p, opac=p):
        return lib.gs_bin_tiles(n, p, conics, opac, p, p, w, h, cap, p, p, offs, ctypes.byref(cnt) if ncnt else None,
                                None, ws, wsb, None)
    assert call(n=-1) == _lib.GS_ERR_INVALID_ARG
    assert call(w=0) == _lib.GS_ERR_INVALID_ARG
    assert call(cap=-1) == _lib.GS_ERR_INVALID_ARG
    assert call(ncnt=False) == _lib.GS_ERR_INVALID_ARG
    assert call(offs=None) == _lib.GS_ERR_INVALID_ARG
    assert b"splat_offsets" in lib.gs_last_error()
    for kw in ({"conics": None}, {"opac": None}):   # the culling ellipse's inputs
        assert call(**kw) == _lib.GS_ERR_INVALID_ARG
        assert b"NULL splat array" in lib.gs_last_error()
    assert call(wsb=16) == _lib.GS_ERR_INVALID_ARG
    assert b"workspace" in lib.gs_last_error()
    assert call(ws=ctypes.c_void_p(257)) == _lib.GS_ERR_INVALID_ARG
    assert b"aligned" in lib.gs_last_error()


def test_error_string_is_thread_local():
    import threading
    lib = _lib.load()
    assert _fwd(lib, n=-7) == _lib.GS_ERR_INVALID_ARG
    seen = {}

    def other():
        seen["msg"] = lib.gs_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert b"n = -7" in lib.gs_last_error()
    assert b"n = -7" not in seen["msg"]


def test_binding_pair_count_never_exceeds_the_list():
    """The binding hands the kernels a pair count no larger than the entries
    sorted_ids holds (the forward and backward clamp tile ranges to it)."""
    import torch
    import differentiable_tile_rasterization_amd as gsr
    ids = torch.zeros(10, dtype=torch.int32)
    assert gsr._pair_count(ids, None) == 10
    assert gsr._pair_count(ids, 7) == 7
    for bad in (11, -1):
        with pytest.raises(ValueError):
            gsr._pair_count(ids, bad)
    with pytest.raises(ValueError):
        gsr._pair_count(torch.zeros((2, 5), dtype=torch.int32), None)


def test_noalloc_rejects_sizes_beyond_its_scratch_before_any_device_call():
    """The allocation-free backward checks the scene's size against its fixed
    scratch on the host first: an oversized call returns GS_ERR_CAPACITY (and
    bad sizes GS_ERR_INVALID_ARG) without touching a device."""
    lib = _lib.load()
    cap = lib.gs_rasterize_bwd_noalloc_capacity()
    assert cap == 64 << 20
    p = ctypes.c_void_p(1)

    def call(n=1000, n_isect=0, n_slots=None, w=64, h=64):
        n_slots = n_isect if n_slots is None else n_slots
        return lib.gs_rasterize_bwd_noalloc(n, p, p, p, p, p, None, w, h, p, p, p, n_isect, n_slots, p, p, p, p, p,
                                            p, p, None, 0, None)
    assert call(n_isect=2_000_000) == _lib.GS_ERR_CAPACITY
    assert b"scratch" in lib.gs_last_error()
    assert call(n_isect=1000, n_slots=2_000_000) == _lib.GS_ERR_CAPACITY   # sized by the slots
    assert call(n=-1) == _lib.GS_ERR_INVALID_ARG
    assert call(w=0) == _lib.GS_ERR_INVALID_ARG
    assert lib.gs_rasterize_bwd_workspace_size(1000, 1_000_000, 64, 64) <= cap


def test_depth_entry_points_reject_bad_arguments():
    """The depth variants check their extra arguments on the host, before any
    device work, and refuse the depth terms on the walks that lack them."""
    lib = _lib.load()
    p = ctypes.c_void_p(1)
    ws = ctypes.c_void_p(256)

    def fwd(depths=p, totals=p, med=None, pos=None):
        return lib.gs_rasterize_fwd_depth(4, p, p, p, p, depths, None, 64, 64, p, p, 0, p, p, p, None, totals, med,
                                          pos, ws, 1 << 20, None)
    assert fwd(depths=None) == _lib.GS_ERR_INVALID_ARG
    assert b"depths" in lib.gs_last_error()
    assert fwd(depths=None, totals=None, pos=p) == _lib.GS_ERR_INVALID_ARG

    def bwd(depths=p, totals=p, pos=p, gd=p, gm=None, dz=p, flags=0):
        return lib.gs_rasterize_bwd_depth(1, p, p, p, p, depths, p, None, 8, 8, p, p, p, 0, 0, p, p, totals, pos, p,
                                          gd, gm, p, p, p, p, dz, None, flags, None, 0, None)
    assert bwd(depths=None) == _lib.GS_ERR_INVALID_ARG
    assert bwd(dz=None) == _lib.GS_ERR_INVALID_ARG
    assert b"dL_ddepths" in lib.gs_last_error()
    assert bwd(pos=None) == _lib.GS_ERR_INVALID_ARG
    assert b"median_pos" in lib.gs_last_error()
    assert bwd(totals=None) == _lib.GS_ERR_INVALID_ARG
    assert b"dist_totals" in lib.gs_last_error()
    # the median term needs no totals: the call gets as far as the workspace check
    assert bwd(totals=None, gd=None, gm=p) == _lib.GS_ERR_INVALID_ARG
    assert b"workspace" in lib.gs_last_error()
    for walk in (_lib.GS_FLAG_WALK_ADD, _lib.GS_FLAG_WALK_STORE):
        assert bwd(flags=walk) == _lib.GS_ERR_UNSUPPORTED
        assert b"deferred walk" in lib.gs_last_error()
        assert bwd(gd=None, gm=p, flags=walk) == _lib.GS_ERR_UNSUPPORTED
    assert bwd(flags=0x80) == _lib.GS_ERR_INVALID_ARG


def test_splat_count_limit_is_checked_everywhere():
    """n up to 2^29 (per-splat int32 offsets such as 3 n stay in range); one
    more is refused by every entry point before any device work, and the
    workspace queries return 0 for it."""
    lib = _lib.load()
    big = (1 << 29) + 1
    p = ctypes.c_void_p(256)
    cnt = ctypes.c_int64(0)
    assert lib.gs_bin_tiles_workspace_size(big, 0, 64, 64) == 0
    assert lib.gs_rasterize_fwd_workspace_size(big) == 0
    assert lib.gs_rasterize_bwd_workspace_size(big, 0, 64, 64) == 0
    assert lib.gs_rasterize_fwd_workspace_size(1 << 29) >= 48 * (1 << 29)
    assert lib.gs_bin_tiles(big, p, p, p, p, p, 64, 64, 16, p, p, p, ctypes.byref(cnt), None, p, 1 << 20,
                            None) == _lib.GS_ERR_INVALID_ARG
    assert b"outside 0..536870912" in lib.gs_last_error()
    assert _fwd(lib, n=big) == _lib.GS_ERR_INVALID_ARG
    assert b"outside 0..536870912" in lib.gs_last_error()
    q = ctypes.c_void_p(1)
    assert lib.gs_rasterize_bwd(big, q, q, q, q, q, None, 8, 8, q, q, q, 0, 0, q, q, q, q, q, q, q, None, 0,
                                None, 0, None) == _lib.GS_ERR_INVALID_ARG
    assert b"outside 0..536870912" in lib.gs_last_error()
    assert lib.gs_rasterize_bwd_noalloc(big, q, q, q, q, q, None, 8, 8, q, q, q, 0, 0, q, q, q, q, q, q, q,
                                        None, 0, None) == _lib.GS_ERR_INVALID_ARG
