"""libgsraster: tile-based Gaussian-splat rasterization (binning, forward,
backward) as hand-written HIP kernels for the AMD Instinct MI355X (gfx950).

This module is a thin binding over the C ABI of include/gsraster.h. The
functions carry the C entry points' names; they check and marshal torch
tensors (device memory, the current HIP stream) into the C call and allocate
the outputs. Every step of the computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import GS_FLAG_ACCUM_WEIGHT, GsError

__all__ = ["gs_bin_tiles", "gs_rasterize_fwd", "gs_rasterize_fwd_depth", "gs_rasterize_bwd",
           "gs_rasterize_bwd_depth", "gs_rasterize_bwd_workspace_size", "gs_rasterize_fwd_workspace_size",
           "gs_rasterize_bwd_noalloc", "gs_rasterize_bwd_noalloc_capacity", "gs_version", "GsError",
           "GS_FLAG_ACCUM_WEIGHT", "TILE", "tile_grid", "Bins"]

TILE = 16


def tile_grid(width: int, height: int) -> tuple[int, int]:
    return (width + TILE - 1) // TILE, (height + TILE - 1) // TILE


def gs_version() -> int:
    return int(_lib.load().gs_version())


def _ptr(t):
    if t is None:
        return None
    if t.numel() == 0:
        # an empty view reports a NULL data pointer; pass its allocation instead
        return ctypes.c_void_p(t.untyped_storage().data_ptr() or None)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, dev):
    """The caller's stream, or the current stream of the tensors' device; a
    stream of another device is refused (its kernels would address memory of
    the wrong GPU)."""
    s = torch.cuda.current_stream(dev) if stream is None else stream
    if s.device != dev:
        raise ValueError(f"stream is on {s.device}, the tensors on {dev}")
    return ctypes.c_void_p(s.cuda_stream)


def _same_device(dev, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, means2d on {dev}: all tensors must share one device")


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _pair_count(sorted_ids, n_isect) -> int:
    """The pair count the kernels clamp tile ranges to: every entry of
    sorted_ids by default, never more than it holds."""
    if sorted_ids.dim() != 1:
        raise ValueError(f"sorted_ids must be one-dimensional, got shape {tuple(sorted_ids.shape)}")
    held = int(sorted_ids.numel())
    if n_isect is None:
        return held
    n_isect = int(n_isect)
    if n_isect < 0 or n_isect > held:
        raise ValueError(f"n_isect = {n_isect}, but sorted_ids holds {held} entries")
    return n_isect


class Bins:
    """Result of gs_bin_tiles: sorted_ids [n_isect] int32, tile_ranges
    [GX*GY, 2] int32, splat_offsets [n+1] int32 (the numbering of the tiles of
    each splat's rectangle that the backward uses for its accumulation slots)
    and n_slots, the number of those slots (splat_offsets[n]; when not given,
    the larger of that and n_isect, read from the device)."""

    def __init__(self, sorted_ids, tile_ranges, splat_offsets, n_isect, width, height, n_slots=None):
        self.sorted_ids = sorted_ids
        self.tile_ranges = tile_ranges
        self.splat_offsets = splat_offsets
        self.n_isect = n_isect
        self.width = width
        self.height = height
        if n_slots is None:
            n_slots = max(int(n_isect), int(splat_offsets[-1].item()) if splat_offsets.numel() else 0)
        self.n_slots = int(n_slots)


def _aligned_workspace(nbytes, dev):
    """A uint8 device buffer and a 256-byte aligned pointer into it."""
    ws = torch.empty((nbytes + 256,), dtype=torch.uint8, device=dev)
    return ws, ctypes.c_void_p((ws.data_ptr() + 255) & ~255)


def _workspace(ws, nbytes, dev):
    """Use the caller's uint8 buffer (checked) or allocate one."""
    if ws is None:
        return _aligned_workspace(nbytes, dev)
    _need(ws, "workspace", torch.uint8)
    if ws.numel() < nbytes + 256:
        raise ValueError(f"workspace holds {ws.numel()} bytes, need {nbytes + 256}")
    return ws, ctypes.c_void_p((ws.data_ptr() + 255) & ~255)


def gs_bin_tiles(means2d, conics, opacities, radii, depths, width: int, height: int, capacity: int | None = None,
                 stream=None) -> Bins:
    """Bin splats into 16x16 tiles (each splat only where its alpha >= 1/255
    ellipse can reach) and sort each tile's list by depth.

    Allocates sorted_ids with ``capacity`` entries (default: 4 per splat) and,
    if the count read back exceeds it, reallocates and calls again."""
    n = int(means2d.shape[0])
    _need(means2d, "means2d", torch.float32, (n, 2))
    _need(conics, "conics", torch.float32, (n, 3))
    _need(opacities, "opacities", torch.float32, (n,))
    _need(radii, "radii", torch.int32, (n,))
    _need(depths, "depths", torch.float32, (n,))
    lib = _lib.load()
    dev = means2d.device
    _same_device(dev, conics=conics, opacities=opacities, radii=radii, depths=depths)
    GX, GY = tile_grid(width, height)
    cap = int(capacity) if capacity is not None else max(4 * n, 1)
    ranges = torch.empty((GX * GY, 2), dtype=torch.int32, device=dev)
    offsets = torch.empty((n + 1,), dtype=torch.int32, device=dev)
    st = _stream(stream, dev)
    for _attempt in range(2):
        ids = torch.empty((max(cap, 1),), dtype=torch.int32, device=dev)
        ws_bytes = int(lib.gs_bin_tiles_workspace_size(n, cap, width, height))
        ws, wsp = _aligned_workspace(ws_bytes, dev)
        n_isect, n_slots = ctypes.c_int64(0), ctypes.c_int64(0)
        with torch.cuda.device(dev):
            status = lib.gs_bin_tiles(n, _ptr(means2d), _ptr(conics), _ptr(opacities), _ptr(radii), _ptr(depths),
                                      width, height, cap, _ptr(ids), _ptr(ranges), _ptr(offsets),
                                      ctypes.byref(n_isect), ctypes.byref(n_slots), wsp, ws_bytes, st)
        if status == _lib.GS_ERR_CAPACITY:
            cap = int(n_isect.value)
            continue
        _lib.check(status)
        I = int(n_isect.value)
        return Bins(ids[:I], ranges, offsets, I, width, height, n_slots=int(n_slots.value))
    raise GsError(_lib.GS_ERR_CAPACITY, "binning capacity still too small after reallocation")


def gs_rasterize_fwd(means2d, conics, colors, opacities, background, width: int, height: int,
                     tile_ranges, sorted_ids, max_weight: bool = False, workspace=None, stream=None,
                     n_isect: int | None = None):
    """Forward composite. Returns (image [H,W,3], final_T [H,W], n_contrib [H,W]),
    and with ``max_weight`` also each splat's largest compositing weight
    alpha T over the pixels that composite it ([n], 0 if none).
    ``workspace`` may pass a uint8 device buffer of at least
    gs_rasterize_fwd_workspace_size(n) + 256 bytes. ``n_isect`` (default:
    every entry of ``sorted_ids``) is the pair count the tile ranges are
    clamped to; it may not exceed the entries sorted_ids holds."""
    n = int(means2d.shape[0])
    _need(means2d, "means2d", torch.float32, (n, 2))
    _need(conics, "conics", torch.float32, (n, 3))
    _need(colors, "colors", torch.float32, (n, 3))
    _need(opacities, "opacities", torch.float32, (n,))
    if background is not None:
        _need(background, "background", torch.float32, (3,))
    GX, GY = tile_grid(width, height)
    _need(tile_ranges, "tile_ranges", torch.int32, (GX * GY, 2))
    _need(sorted_ids, "sorted_ids", torch.int32)
    n_pairs = _pair_count(sorted_ids, n_isect)
    dev = means2d.device
    _same_device(dev, conics=conics, colors=colors, opacities=opacities, background=background,
                 tile_ranges=tile_ranges, sorted_ids=sorted_ids, workspace=workspace)
    image = torch.empty((height, width, 3), dtype=torch.float32, device=dev)
    final_T = torch.empty((height, width), dtype=torch.float32, device=dev)
    n_contrib = torch.empty((height, width), dtype=torch.int32, device=dev)
    mw = torch.empty((n,), dtype=torch.float32, device=dev) if max_weight else None
    lib = _lib.load()
    ws_bytes = int(lib.gs_rasterize_fwd_workspace_size(n))
    workspace, wsp = _workspace(workspace, ws_bytes, dev)
    st = _stream(stream, dev)
    with torch.cuda.device(dev):
        _lib.check(lib.gs_rasterize_fwd(
            n, _ptr(means2d), _ptr(conics), _ptr(colors), _ptr(opacities), _ptr(background), width, height,
            _ptr(tile_ranges), _ptr(sorted_ids), n_pairs, _ptr(image), _ptr(final_T), _ptr(n_contrib), _ptr(mw), wsp,
            ws_bytes, st))
    if max_weight:
        return image, final_T, n_contrib, mw
    return image, final_T, n_contrib


def gs_rasterize_fwd_depth(means2d, conics, colors, opacities, depths, background, width: int, height: int,
                           tile_ranges, sorted_ids, distortion: bool = True, median: bool = True,
                           max_weight: bool = False, workspace=None, stream=None, n_isect: int | None = None):
    """gs_rasterize_fwd with the depth outputs. Returns a dict: image, final_T,
    n_contrib, [max_weight]; with ``distortion`` dist_totals [H,W,4] = (A, B,
    C, D): A = sum alpha T, B and C the first two moments of depth about the
    median, D = sum over composited pairs i < j of w_i w_j (z_i - z_j)^2; with
    ``median`` median_depth [H,W] (depth of the last composited splat whose
    transmittance before it is > 1/2, 0 if none); median_pos [H,W] int32
    (that splat's list position + 1, 0 if none) with either, since the
    backward's depth terms need it."""
    n = int(means2d.shape[0])
    _need(means2d, "means2d", torch.float32, (n, 2))
    _need(conics, "conics", torch.float32, (n, 3))
    _need(colors, "colors", torch.float32, (n, 3))
    _need(opacities, "opacities", torch.float32, (n,))
    _need(depths, "depths", torch.float32, (n,))
    if background is not None:
        _need(background, "background", torch.float32, (3,))
    GX, GY = tile_grid(width, height)
    _need(tile_ranges, "tile_ranges", torch.int32, (GX * GY, 2))
    _need(sorted_ids, "sorted_ids", torch.int32)
    n_pairs = _pair_count(sorted_ids, n_isect)
    dev = means2d.device
    _same_device(dev, conics=conics, colors=colors, opacities=opacities, depths=depths, background=background,
                 tile_ranges=tile_ranges, sorted_ids=sorted_ids, workspace=workspace)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"image": torch.empty((height, width, 3), **f32), "final_T": torch.empty((height, width), **f32),
           "n_contrib": torch.empty((height, width), dtype=torch.int32, device=dev)}
    if max_weight:
        out["max_weight"] = torch.empty((n,), **f32)
    if distortion:
        out["dist_totals"] = torch.empty((height, width, 4), **f32)
    if median:
        out["median_depth"] = torch.empty((height, width), **f32)
    if distortion or median:
        out["median_pos"] = torch.empty((height, width), dtype=torch.int32, device=dev)
    lib = _lib.load()
    ws_bytes = int(lib.gs_rasterize_fwd_workspace_size(n))
    workspace, wsp = _workspace(workspace, ws_bytes, dev)
    st = _stream(stream, dev)
    g = out.get
    with torch.cuda.device(dev):
        _lib.check(lib.gs_rasterize_fwd_depth(
            n, _ptr(means2d), _ptr(conics), _ptr(colors), _ptr(opacities), _ptr(depths), _ptr(background), width,
            height, _ptr(tile_ranges), _ptr(sorted_ids), n_pairs, _ptr(out["image"]), _ptr(out["final_T"]),
            _ptr(out["n_contrib"]), _ptr(g("max_weight")), _ptr(g("dist_totals")), _ptr(g("median_depth")),
            _ptr(g("median_pos")), wsp, ws_bytes, st))
    return out


def _check_bwd_args(means2d, conics, colors, opacities, radii, background, width, height, bins, final_T,
                    n_contrib, dL_dimage, workspace):
    n = int(means2d.shape[0])
    _need(means2d, "means2d", torch.float32, (n, 2))
    _need(conics, "conics", torch.float32, (n, 3))
    _need(colors, "colors", torch.float32, (n, 3))
    _need(opacities, "opacities", torch.float32, (n,))
    _need(radii, "radii", torch.int32, (n,))
    if background is not None:
        _need(background, "background", torch.float32, (3,))
    GX, GY = tile_grid(width, height)
    _need(bins.tile_ranges, "tile_ranges", torch.int32, (GX * GY, 2))
    _need(bins.sorted_ids, "sorted_ids", torch.int32)
    _need(bins.splat_offsets, "splat_offsets", torch.int32, (n + 1,))
    _pair_count(bins.sorted_ids, bins.n_isect)
    _need(final_T, "final_T", torch.float32, (height, width))
    _need(n_contrib, "n_contrib", torch.int32, (height, width))
    _need(dL_dimage, "dL_dimage", torch.float32, (height, width, 3))
    _same_device(means2d.device, conics=conics, colors=colors, opacities=opacities, radii=radii,
                 background=background, tile_ranges=bins.tile_ranges, sorted_ids=bins.sorted_ids,
                 splat_offsets=bins.splat_offsets, final_T=final_T, n_contrib=n_contrib, dL_dimage=dL_dimage,
                 workspace=workspace)


def _output_shapes(n, accum_weight):
    shapes = {"dL_dmeans2d": (n, 2), "dL_dconics": (n, 3), "dL_dcolors": (n, 3), "dL_dopacities": (n,)}
    if accum_weight:
        shapes["accum_weight"] = (n,)
    return shapes


def _check_outputs(out, n, accum_weight, dev):
    """The kernels write every element: shapes, dtype and device are checked like the inputs."""
    if out is None:
        raise ValueError("out: a dict of preallocated outputs is required")
    for k, v in _output_shapes(n, accum_weight).items():
        if k not in out:
            raise ValueError(f"out lacks {k!r}")
        _need(out[k], k, torch.float32, v)
        _same_device(dev, **{k: out[k]})


def _bwd_args(means2d, conics, colors, opacities, radii, background, width, height, bins, final_T, n_contrib,
              dL_dimage, out, accum_weight, walk):
    """The C arguments up to and including flags."""
    n = int(means2d.shape[0])
    flags = GS_FLAG_ACCUM_WEIGHT if accum_weight else 0
    if walk is not None:
        walks = {"add": _lib.GS_FLAG_WALK_ADD, "store": _lib.GS_FLAG_WALK_STORE, "defer": _lib.GS_FLAG_WALK_DEFER}
        if walk not in walks:
            raise ValueError(f"walk: None, 'add', 'store' or 'defer', not {walk!r}")
        flags |= walks[walk]
    return (n, _ptr(means2d), _ptr(conics), _ptr(colors), _ptr(opacities), _ptr(radii), _ptr(background), width,
            height, _ptr(bins.tile_ranges), _ptr(bins.sorted_ids), _ptr(bins.splat_offsets), bins.n_isect,
            bins.n_slots, _ptr(final_T), _ptr(n_contrib), _ptr(dL_dimage), _ptr(out["dL_dmeans2d"]), _ptr(out["dL_dconics"]),
            _ptr(out["dL_dcolors"]), _ptr(out["dL_dopacities"]),
            _ptr(out.get("accum_weight") if accum_weight else None), flags)


def gs_rasterize_bwd(means2d, conics, colors, opacities, radii, background, width: int, height: int, bins: Bins,
                     final_T, n_contrib, dL_dimage, accum_weight: bool = False, out=None, workspace=None,
                     stream=None, events=None, walk=None):
    """Backward. Returns dict with dL_dmeans2d [n,2], dL_dconics [n,3],
    dL_dcolors [n,3], dL_dopacities [n] and, with ``accum_weight``, the
    per-splat accumulated weight [n]. ``walk``: None (the library's default,
    the deferred walk), "defer", "add" or "store" (GS_FLAG_WALK_DEFER /
    GS_FLAG_WALK_ADD / GS_FLAG_WALK_STORE). ``out`` may pass preallocated outputs
    (same dict keys) and ``workspace`` a uint8 device buffer of at least
    gs_rasterize_bwd_workspace_size(n, bins.n_slots, width, height) + 256 bytes, to keep
    allocation out of timed loops. ``events``: four torch.cuda.Event objects
    (timing enabled, already recorded once) to be recorded at the call's
    stage boundaries (gs_rasterize_bwd_timed)."""
    n = int(means2d.shape[0])
    dev = means2d.device
    _check_bwd_args(means2d, conics, colors, opacities, radii, background, width, height, bins, final_T,
                    n_contrib, dL_dimage, workspace)
    lib = _lib.load()
    if out is None:
        out = {k: torch.empty(v, dtype=torch.float32, device=dev) for k, v in _output_shapes(n, accum_weight).items()}
    else:
        _check_outputs(out, n, accum_weight, dev)
    ws_bytes = int(lib.gs_rasterize_bwd_workspace_size(n, bins.n_slots, width, height))
    workspace, wsp = _workspace(workspace, ws_bytes, dev)
    args = _bwd_args(means2d, conics, colors, opacities, radii, background, width, height, bins, final_T,
                     n_contrib, dL_dimage, out, accum_weight, walk) + (wsp, ws_bytes, _stream(stream, dev))
    if events is not None and len(events) != 4:
        raise ValueError("events: four torch.cuda.Event objects")
    with torch.cuda.device(dev):
        if events is None:
            _lib.check(lib.gs_rasterize_bwd(*args))
        else:
            handles = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(int(e.cuda_event)) for e in events])
            _lib.check(lib.gs_rasterize_bwd_timed(*args, handles))
    return out


def gs_rasterize_bwd_depth(means2d, conics, colors, opacities, depths, radii, background, width: int,
                           height: int, bins: Bins, final_T, n_contrib, median_pos, dL_dimage, dist_totals=None,
                           dL_ddist=None, dL_dmedian=None, accum_weight: bool = False, out=None, workspace=None,
                           stream=None, walk=None):
    """gs_rasterize_bwd with the depth terms: also the gradients of
    sum dL_ddist * D + dL_dmedian * median_depth (either upstream may be
    None; dist_totals and median_pos as gs_rasterize_fwd_depth returned
    them). Returns gs_rasterize_bwd's dict plus dL_ddepths [n]."""
    n = int(means2d.shape[0])
    dev = means2d.device
    _check_bwd_args(means2d, conics, colors, opacities, radii, background, width, height, bins, final_T,
                    n_contrib, dL_dimage, workspace)
    _need(depths, "depths", torch.float32, (n,))
    _need(median_pos, "median_pos", torch.int32, (height, width))
    if dL_ddist is not None:
        _need(dL_ddist, "dL_ddist", torch.float32, (height, width))
        if dist_totals is None:
            raise ValueError("dL_ddist needs dist_totals (from gs_rasterize_fwd_depth)")
    if dist_totals is not None:
        _need(dist_totals, "dist_totals", torch.float32, (height, width, 4))
    if dL_dmedian is not None:
        _need(dL_dmedian, "dL_dmedian", torch.float32, (height, width))
    _same_device(dev, depths=depths, median_pos=median_pos, dist_totals=dist_totals, dL_ddist=dL_ddist,
                 dL_dmedian=dL_dmedian)
    lib = _lib.load()
    shapes = dict(_output_shapes(n, accum_weight), dL_ddepths=(n,))
    if out is None:
        out = {k: torch.empty(v, dtype=torch.float32, device=dev) for k, v in shapes.items()}
    else:
        for k, v in shapes.items():
            if k not in out:
                raise ValueError(f"out lacks {k!r}")
            _need(out[k], k, torch.float32, v)
            _same_device(dev, **{k: out[k]})
    a = _bwd_args(means2d, conics, colors, opacities, radii, background, width, height, bins, final_T,
                  n_contrib, dL_dimage, out, accum_weight, walk)
    ws_bytes = int(lib.gs_rasterize_bwd_workspace_size(n, bins.n_slots, width, height))
    workspace, wsp = _workspace(workspace, ws_bytes, dev)
    # gs_rasterize_bwd's arguments with the depth inputs and output spliced in
    args = (a[:5] + (_ptr(depths),) + a[5:16] + (_ptr(dist_totals), _ptr(median_pos), a[16], _ptr(dL_ddist),
                                                 _ptr(dL_dmedian)) + a[17:21] + (_ptr(out["dL_ddepths"]),) + a[21:]
            + (wsp, ws_bytes, _stream(stream, dev)))
    with torch.cuda.device(dev):
        _lib.check(lib.gs_rasterize_bwd_depth(*args))
    return out


def gs_rasterize_bwd_noalloc(means2d, conics, colors, opacities, radii, background, width: int, height: int,
                             bins: Bins, final_T, n_contrib, dL_dimage, out, accum_weight: bool = False,
                             stream=None, walk=None):
    """gs_rasterize_bwd with its workspace in the library's fixed device
    array (no allocation by the library; ``out`` holds the caller's
    preallocated outputs, the keys of gs_rasterize_bwd's result). Raises
    GsError (GS_ERR_CAPACITY) when the scene needs more than
    gs_rasterize_bwd_noalloc_capacity() bytes. Calls that overlap on one GPU
    share that array and race."""
    n = int(means2d.shape[0])
    dev = means2d.device
    _check_bwd_args(means2d, conics, colors, opacities, radii, background, width, height, bins, final_T,
                    n_contrib, dL_dimage, None)
    _check_outputs(out, n, accum_weight, dev)
    lib = _lib.load()
    args = _bwd_args(means2d, conics, colors, opacities, radii, background, width, height, bins, final_T,
                     n_contrib, dL_dimage, out, accum_weight, walk)
    with torch.cuda.device(dev):
        _lib.check(lib.gs_rasterize_bwd_noalloc(*args, _stream(stream, dev)))
    return out


def gs_rasterize_bwd_noalloc_capacity() -> int:
    return int(_lib.load().gs_rasterize_bwd_noalloc_capacity())


def gs_rasterize_bwd_workspace_size(n: int, n_slots: int, width: int, height: int) -> int:
    return int(_lib.load().gs_rasterize_bwd_workspace_size(n, n_slots, width, height))


def gs_rasterize_fwd_workspace_size(n: int) -> int:
    return int(_lib.load().gs_rasterize_fwd_workspace_size(n))
