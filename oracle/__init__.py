"""CPU float64 oracle for tile-based Gaussian-splat rasterization.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package. The product path (the
HIP library and its Python binding) never touches it, and it shares no code,
header, table or helper with that path. The seeded input generators in
``scenes`` are the only module both sides use; they hold none of the method's
arithmetic.

Contents, each following the pages' problem statement (the pages print no
formulas; see gs_oracle.c for the compositing reading):

* :func:`bin_tiles` -- which 16x16 tiles each splat covers, and each tile's
  list ordered by depth. The binning / radix-sort / tile-range stages appear
  as ``emit_pairs``, ``radix_hist``, ``radix_scatter`` and ``extract_offsets``
  in the timing table of page "Phase 5 step 30b — kernel-by-kernel timing"
  (section 計測結果). Written out as one library sort (numpy.lexsort) of all
  (splat, tile) pairs by (tile, depth bits, id).
* :func:`rasterize_fwd` / :func:`rasterize_bwd` -- per-pixel front-to-back
  composite and the exact gradient of L = sum <dL/dImage, image> (C core,
  float64, OpenMP over tiles).
* :func:`rasterize_fwd_depth` / :func:`rasterize_bwd_depth` -- the
  distortion and median-depth terms (the optional features of
  rasterize_bwd_2d on the Spirula Studio page, section 机制拆解, which gives
  no formula; the reading is stated there) and their exact gradients.
* :func:`composite_bruteforce` / :func:`depth_terms_bruteforce` -- the same
  composite (and depth terms, as a full double sum) with no tiles at all:
  every pixel walks every splat in (depth, id) order. Used to pin the tiled
  oracle.

Binning is the only integer decision driven by floating point here, and it is
taken in float32 exactly like the kernels take it (the tile rectangle from
mean +- radius, scaled by 1/16 and floored), so binning parity is bit-exact.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

TILE = 16
ALPHA_MIN = 1.0 / 255.0
ALPHA_MAX = 0.99
T_MIN = 1e-4

_lib = None


def _load():
    global _lib
    if _lib is None:
        # GS_ORACLE_LIB: another build of this C core (the tests' mutation
        # checks point the pins at deliberately broken copies)
        path = os.environ.get("GS_ORACLE_LIB") or _build.OUT
        if path == _build.OUT and (not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
            _build.build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.gso_forward.argtypes = [i32, i32, P, P, P, P, P, P, P, P, i32, P, P, P, P]
        lib.gso_forward.restype = i32
        lib.gso_backward.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, P, P, i32, P, P]
        lib.gso_backward.restype = i32
        lib.gso_max_weight.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, P, i32, P, P, P]
        lib.gso_max_weight.restype = i32
        lib.gso_pixel_outcomes.argtypes = [i32, i32, P, P, P, P, P, P, P, i32, P, P, i32, P, P, P, P]
        lib.gso_pixel_outcomes.restype = i32
        lib.gso_forward_depth.argtypes = [i32, i32, P, P, P, P, P, P, P, P, P, i32, P, P, P, P]
        lib.gso_forward_depth.restype = i32
        lib.gso_backward_depth.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, i32, P, P]
        lib.gso_backward_depth.restype = i32
        lib.gso_threads.argtypes = []
        lib.gso_threads.restype = i32
        lib.gso_set_threads.argtypes = [i32]
        lib.gso_set_threads.restype = None
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the C core runs on."""
    return int(_load().gso_threads())


def set_threads(n: int) -> None:
    """Run the C core's parallel loops on ``n`` threads from now on."""
    _load().gso_set_threads(int(n))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def grid(width: int, height: int) -> tuple[int, int]:
    return (width + TILE - 1) // TILE, (height + TILE - 1) // TILE


# ----------------------------------------------------------------------------
# Binning
# ----------------------------------------------------------------------------

def tile_rects(means2d: np.ndarray, radii: np.ndarray, depths: np.ndarray, width: int, height: int):
    """Per-splat tile rectangle [tx0, tx1) x [ty0, ty1), float32 arithmetic.

    A splat is culled (empty rectangle) if radius <= 0, depth is not > 0, or
    its mean is not finite."""
    GX, GY = grid(width, height)
    f = np.float32
    m = np.asarray(means2d, dtype=f)
    r = np.asarray(radii, dtype=np.int32).astype(f)
    inv = f(1.0 / TILE)
    with np.errstate(invalid="ignore", over="ignore"):
        x0 = np.floor((m[:, 0] - r) * inv)
        x1 = np.floor((m[:, 0] + r) * inv) + f(1.0)
        y0 = np.floor((m[:, 1] - r) * inv)
        y1 = np.floor((m[:, 1] + r) * inv) + f(1.0)
    tx0 = np.clip(x0, 0, GX).astype(np.int64)
    tx1 = np.clip(x1, 0, GX).astype(np.int64)
    ty0 = np.clip(y0, 0, GY).astype(np.int64)
    ty1 = np.clip(y1, 0, GY).astype(np.int64)
    d = np.asarray(depths, dtype=f)
    live = (np.asarray(radii) > 0) & (d > 0) & np.isfinite(m[:, 0]) & np.isfinite(m[:, 1])
    live &= (tx1 > tx0) & (ty1 > ty0)
    tx1 = np.where(live, tx1, tx0)
    ty1 = np.where(live, ty1, ty0)
    return tx0, tx1, ty0, ty1


def cull_ellipses(means2d, conics, opacities):
    """Per-splat constants of the binning's culling ellipse, float32.

    A splat can reach alpha >= 1/255 only where its quadratic form
    Q(d) = a dx^2 + 2 b dx dy + c dy^2 <= 2 ln(255 o). The binning keeps a
    tile only if the ellipse {Q <= T} meets the tile's pixel-centre rectangle,
    with T an upper bound on 2 ln(255 o) taken with basic float32 operations
    only (each rounded once, in a fixed order, so that any IEEE float32
    implementation decides every tile identically): with 255 o = m2 * 2^e2,
    m2 in [1, 2), ln(255 o) <= e2 ln 2 + (m2 - 1) / sqrt(m2) (the bound
    ln x <= (x - 1)/sqrt(x) for x >= 1), then T = 2 lnb (1 + 2^-10) + 2^-10.
    Q is taken through the Cholesky factors of the conic: Q = (l11 u + l21 v)^2
    + (l22 v)^2 with u = x - mean_x, v = y - mean_y.

    Returns a dict of float32 arrays: mx, my, l11, l21, l22, T, vmax (the
    ellipse's half height), vL (v of its leftmost point; -vL is that of the
    rightmost), and boolean ``cull`` (False where the constants are not usable:
    such a splat keeps its whole rectangle) and ``dead`` (the float32 product
    255 o is below 1, so alpha <= o < 1/255 everywhere)."""
    f = np.float32
    m = np.asarray(means2d, dtype=f)
    q = np.asarray(conics, dtype=f)
    o = np.asarray(opacities, dtype=f)
    with np.errstate(all="ignore"):
        y = f(255.0) * o
        mant, ex = np.frexp(y)                       # y = mant * 2^ex, mant in [0.5, 1)
        m2 = mant * f(2.0)                           # in [1, 2)
        e2 = (ex - 1).astype(f)
        lnb = e2 * LN2_F32 + (m2 - f(1.0)) / np.sqrt(m2)
        T = f(2.0) * lnb
        T = (T + T * f(1.0 / 1024.0)) + f(1.0 / 1024.0)
        l11 = np.sqrt(q[:, 0])
        l21 = q[:, 1] / l11
        l22 = np.sqrt(np.maximum(q[:, 2] - l21 * l21, f(0.0)))
        sT = np.sqrt(T)
        vmax = sT / l22
        nrm = np.sqrt(l21 * l21 + l22 * l22)
        vL = (sT * l21) / (l22 * nrm)
        dead = ~(y >= f(1.0))           # 255 o < 1: alpha <= o < 1/255 everywhere
        usable = np.isfinite(T) & np.isfinite(l11) & np.isfinite(l21) & np.isfinite(l22) & \
            np.isfinite(vmax) & np.isfinite(vL) & (l11 > 0) & (l22 > 0) & np.isfinite(m).all(axis=1)
    return {"mx": m[:, 0], "my": m[:, 1], "l11": l11, "l21": l21, "l22": l22, "T": T, "vmax": vmax, "vL": vL,
            "cull": usable & ~dead, "dead": dead}


LN2_F32 = np.float32(0.6931471805599453)  # rounds up: float32(ln 2) > ln 2


def row_columns(ce, idx, ty, tx0, tx1):
    """For splat idx[k] and tile row ty[k]: the range [c_lo, c_hi] of tile
    columns of [tx0[k], tx1[k]) whose pixel-centre rectangle meets the
    culling ellipse (empty when c_lo > c_hi). Float32, every operation rounded
    once in the order written.

    Over the row's band of pixel centres y in [Y0, Y0 + 15], v = y - mean_y,
    the ellipse's points have u = (-l21 v +- sqrt(T - (l22 v)^2)) / l11; the
    left end is convex in v and least at the leftmost point's v (clamped to
    the band and to |v| <= vmax), the right end concave and largest at the
    rightmost's. A column c (pixel centres x in [16 c + 0.5, 16 c + 15.5])
    meets the ellipse's part in the band iff 16 c + 15.5 >= xl and
    16 c + 0.5 <= xr."""
    f = np.float32
    mx, my, l11, l21, l22 = (ce[k][idx] for k in ("mx", "my", "l11", "l21", "l22"))
    T, vmax, vL = ce["T"][idx], ce["vmax"][idx], ce["vL"][idx]
    with np.errstate(all="ignore"):
        Y0 = ty.astype(f) * f(16.0) + f(0.5)
        v0 = Y0 - my
        v1 = v0 + f(15.0)
        lo = np.maximum(v0, -vmax)
        hi = np.minimum(v1, vmax)
        row_ok = lo <= hi
        vl = np.minimum(np.maximum(vL, lo), hi)
        vr = np.minimum(np.maximum(-vL, lo), hi)
        tl = l22 * vl
        sl = np.sqrt(np.maximum(T - tl * tl, f(0.0)))
        xl = mx + (-(l21 * vl) - sl) / l11
        tr = l22 * vr
        sr = np.sqrt(np.maximum(T - tr * tr, f(0.0)))
        xr = mx + (-(l21 * vr) + sr) / l11
        txf0, txf1 = tx0.astype(f), tx1.astype(f)
        # smallest c with 16 c + 15.5 >= xl, largest with 16 c + 0.5 <= xr
        # (estimates clamped near the rectangle, then corrected by one)
        cl = np.minimum(np.maximum(np.ceil((xl - f(15.5)) * f(0.0625)), txf0 - f(1.0)), txf1 + f(1.0))
        cl = np.where((cl - f(1.0)) * f(16.0) + f(15.5) >= xl, cl - f(1.0), cl)
        cl = np.where(cl * f(16.0) + f(15.5) < xl, cl + f(1.0), cl)
        ch = np.minimum(np.maximum(np.floor((xr - f(0.5)) * f(0.0625)), txf0 - f(2.0)), txf1)
        ch = np.where((ch + f(1.0)) * f(16.0) + f(0.5) <= xr, ch + f(1.0), ch)
        ch = np.where(ch * f(16.0) + f(0.5) > xr, ch - f(1.0), ch)
    # (rows of splats whose constants are not usable compute NaN here; their
    # pairs take the whole rectangle or nothing, see kept_pairs)
    c_lo = np.maximum(np.nan_to_num(cl).astype(np.int64), tx0)
    c_hi = np.minimum(np.nan_to_num(ch).astype(np.int64), tx1 - 1)
    empty = ~row_ok
    c_lo = np.where(empty, tx1, c_lo)
    c_hi = np.where(empty, tx1 - 1, c_hi)
    return c_lo, c_hi


def kept_pairs(means2d, conics, opacities, radii, depths, width: int, height: int):
    """Every (splat, tile) pair of the splats' tile rectangles, splat by splat,
    each splat's tiles row-major (the pair numbering the backward's slots use),
    with whether the binning keeps it. Returns (ids, tx, ty, kept)."""
    tx0, tx1, ty0, ty1 = tile_rects(means2d, radii, depths, width, height)
    nx = tx1 - tx0
    cnt = nx * (ty1 - ty0)
    total = int(cnt.sum())
    ids = np.repeat(np.arange(len(cnt), dtype=np.int32), cnt)
    local = np.arange(total, dtype=np.int64) - np.repeat(np.cumsum(cnt) - cnt, cnt)
    nxr = np.maximum(np.repeat(nx, cnt), 1)
    tx = np.repeat(tx0, cnt) + local % nxr
    ty = np.repeat(ty0, cnt) + local // nxr
    del local, nxr
    ce = cull_ellipses(means2d, conics, opacities)
    # the column range of each (splat, row), taken once per row
    rows = (ty1 - ty0)
    r_ids = np.repeat(np.arange(len(cnt), dtype=np.int64), rows)
    r_ty = np.repeat(ty0, rows) + (np.arange(int(rows.sum()), dtype=np.int64) - np.repeat(np.cumsum(rows) - rows, rows))
    c_lo, c_hi = row_columns(ce, r_ids, r_ty, tx0[r_ids], tx1[r_ids])
    row_first = np.cumsum(rows) - rows                 # first row task of each splat
    rt = row_first[ids] + (ty - ty0[ids])              # row task of each pair
    kept = (tx >= c_lo[rt]) & (tx <= c_hi[rt])
    # splats whose constants are unusable keep their whole rectangle; dead ones none
    kept = np.where(ce["cull"][ids], kept, ~ce["dead"][ids])
    return ids, tx, ty, kept


def bin_tiles(means2d, conics, opacities, radii, depths, width: int, height: int):
    """Tile lists, as (sorted_ids int32 [I], tile_ranges int32 [GX*GY, 2]).

    Each tile's list holds the splats whose rectangle covers it and whose
    culling ellipse (:func:`cull_ellipses`) meets its pixel-centre rectangle,
    ordered by the float32 bit pattern of depth (positive floats order like
    their bit patterns), ties broken by ascending splat id. Tile ids are
    row-major, ``ty * GX + tx``; the lists are concatenated in tile-id order.

    Written as the definition: every kept (splat, tile) pair is listed, then
    one library sort orders the pairs by (tile id, depth bits, splat id)."""
    GX, GY = grid(width, height)
    ids, tx, ty, kept = kept_pairs(means2d, conics, opacities, radii, depths, width, height)
    ids, tx, ty = ids[kept], tx[kept], ty[kept]
    tile = ty * GX + tx
    del tx, ty
    dbits = np.asarray(depths, dtype=np.float32).view(np.uint32)
    # np.lexsort sorts by its last key first: tile, then depth bits, then id
    perm = np.lexsort((ids, dbits[ids], tile))
    sorted_ids = ids[perm]
    counts = np.bincount(tile, minlength=GX * GY)
    ends = np.cumsum(counts)
    ranges = np.stack([ends - counts, ends], axis=1).astype(np.int32)
    ranges[counts == 0] = 0
    return sorted_ids, ranges


# ----------------------------------------------------------------------------
# Forward / backward (C core)
# ----------------------------------------------------------------------------

def _arrs(means2d, conics, colors, opacities):
    # float64 copies of the (usually float32) inputs: the values are exact, and
    # finite-difference pins can perturb them below float32 resolution.
    return (np.ascontiguousarray(means2d, dtype=np.float64),
            np.ascontiguousarray(conics, dtype=np.float64),
            np.ascontiguousarray(colors, dtype=np.float64),
            np.ascontiguousarray(opacities, dtype=np.float64))


def rasterize_fwd(means2d, conics, colors, opacities, background, width: int, height: int,
                  tile_ranges, sorted_ids, tiles=None):
    """Forward composite. Returns dict with image [H,W,3] f64, final_T [H,W]
    f64, n_contrib [H,W] i32 and ambiguous [H,W] bool. With ``tiles`` (a list
    of tile ids) only those tiles' pixels are computed (others stay 0)."""
    lib = _load()
    m, q, c, o = _arrs(means2d, conics, colors, opacities)
    bg = np.ascontiguousarray(np.zeros(3) if background is None else background, dtype=np.float64)
    rng_ = np.ascontiguousarray(tile_ranges, dtype=np.int32)
    ids = np.ascontiguousarray(sorted_ids, dtype=np.int32)
    img = np.zeros((height, width, 3), dtype=np.float64)
    T = np.zeros((height, width), dtype=np.float64)
    nc = np.zeros((height, width), dtype=np.int32)
    amb = np.zeros((height, width), dtype=np.uint8)
    if tiles is None:
        tl, ntl = None, 0
    else:
        tarr = np.ascontiguousarray(tiles, dtype=np.int32)
        tl, ntl = _ptr(tarr), len(tarr)
    lib.gso_forward(width, height, _ptr(rng_), _ptr(ids), _ptr(m), _ptr(q), _ptr(c), _ptr(o),
                    _ptr(bg), tl, ntl, _ptr(img), _ptr(T), _ptr(nc), _ptr(amb))
    return {"image": img, "final_T": T, "n_contrib": nc, "ambiguous": amb.astype(bool)}


def rasterize_bwd(means2d, conics, colors, opacities, background, width: int, height: int,
                  tile_ranges, sorted_ids, dL_dimage, tiles=None):
    """Exact gradients of L = sum <dL_dimage, image>. Returns dict of float64
    arrays: dmeans2d [n,2], dconics [n,3], dcolors [n,3], dopacities [n],
    accum_weight [n]. With ``tiles`` only those tiles' pixels contribute."""
    lib = _load()
    m, q, c, o = _arrs(means2d, conics, colors, opacities)
    n = m.shape[0]
    bg = np.ascontiguousarray(np.zeros(3) if background is None else background, dtype=np.float64)
    rng_ = np.ascontiguousarray(tile_ranges, dtype=np.int32)
    ids = np.ascontiguousarray(sorted_ids, dtype=np.int32)
    g = np.ascontiguousarray(dL_dimage, dtype=np.float64)
    grads = np.zeros((n, 9), dtype=np.float64)
    aw = np.zeros(n, dtype=np.float64)
    if tiles is None:
        tl, ntl = None, 0
    else:
        tarr = np.ascontiguousarray(tiles, dtype=np.int32)
        tl, ntl = _ptr(tarr), len(tarr)
    lib.gso_backward(width, height, n, _ptr(rng_), _ptr(ids), _ptr(m), _ptr(q), _ptr(c), _ptr(o),
                     _ptr(bg), _ptr(g), tl, ntl, _ptr(grads), _ptr(aw))
    return {"dmeans2d": grads[:, 0:2].copy(), "dconics": grads[:, 2:5].copy(),
            "dcolors": grads[:, 5:8].copy(), "dopacities": grads[:, 8].copy(),
            "accum_weight": aw}


def max_weight(means2d, conics, colors, opacities, background, width: int, height: int,
               tile_ranges, sorted_ids, tiles=None, tol: float = 1e-5, bounds: bool = False):
    """Per-splat maximum compositing weight alpha T over composited pairs (0
    for a splat no pixel composites): the "max wt" statistic that the Spirula
    Studio page's raster_bench times (section 亲手验证) without defining it.
    Returns (max_weight float64 [n], uncertain bool [n]); ``uncertain`` marks
    the splats whose maximum a float32 walk may legitimately change by more
    than ``tol``: a pixel with an ambiguous decision may give them a weight
    that reaches their maximum less ``tol``. With ``bounds`` also (lo, hi)
    [n]: every admissible maximum lies in [lo, hi] (lo from the pairs
    composited before their pixel's first ambiguous decision, hi the larger
    of the maximum and the bound at ambiguous pixels)."""
    lib = _load()
    m, q, c, o = _arrs(means2d, conics, colors, opacities)
    n = m.shape[0]
    bg = np.ascontiguousarray(np.zeros(3) if background is None else background, dtype=np.float64)
    rng_ = np.ascontiguousarray(tile_ranges, dtype=np.int32)
    ids = np.ascontiguousarray(sorted_ids, dtype=np.int32)
    mw = np.zeros(n, dtype=np.float64)
    amb = np.zeros(n, dtype=np.float64)
    cert = np.zeros(n, dtype=np.float64)
    if tiles is None:
        tl, ntl = None, 0
    else:
        tarr = np.ascontiguousarray(tiles, dtype=np.int32)
        tl, ntl = _ptr(tarr), len(tarr)
    lib.gso_max_weight(width, height, n, _ptr(rng_), _ptr(ids), _ptr(m), _ptr(q), _ptr(c), _ptr(o),
                       _ptr(bg), tl, ntl, _ptr(mw), _ptr(amb), _ptr(cert))
    # a splat is certain when every weight an ambiguous pixel may give it is
    # within tol of zero, or stays below its maximum less tol
    unc = (amb > tol) & (amb >= mw - tol)
    if bounds:
        return mw, unc, cert, np.maximum(mw, amb)
    return mw, unc


def _tiles_arg(tiles):
    if tiles is None:
        return None, 0, None
    tarr = np.ascontiguousarray(tiles, dtype=np.int32)
    return _ptr(tarr), len(tarr), tarr


def rasterize_fwd_depth(means2d, conics, colors, opacities, background, width: int, height: int,
                        tile_ranges, sorted_ids, depths, tiles=None):
    """Depth terms of the forward: the distortion and median-depth options
    that the Spirula Studio page lists for rasterize_bwd_2d (section 机制拆解:
    a per-pixel float4 of distortion totals, and a median output) without a
    formula. Read as

      distortion  D = sum over composited pairs i < j of w_i w_j (z_i - z_j)^2
                  (w = alpha T, z = the splat's depth)
      median      the depth of the last composited splat whose transmittance
                  before it is still > 1/2 (0 when nothing composites), and
                  its list position + 1 (0: none)

    Returns dict: totals [H,W,4] = (A, B, C, D) with A = sum w,
    B = sum w (z - median), C = sum w (z - median)^2; distortion [H,W] (= D);
    median_depth [H,W]; median_pos [H,W] int32; median_ambiguous [H,W] bool
    (the T > 1/2 decision lies inside its float32 error band)."""
    lib = _load()
    m, q, c, o = _arrs(means2d, conics, colors, opacities)
    bg = np.ascontiguousarray(np.zeros(3) if background is None else background, dtype=np.float64)
    rng_ = np.ascontiguousarray(tile_ranges, dtype=np.int32)
    ids = np.ascontiguousarray(sorted_ids, dtype=np.int32)
    z = np.ascontiguousarray(depths, dtype=np.float64)
    tot = np.zeros((height, width, 4), dtype=np.float64)
    med = np.zeros((height, width), dtype=np.float64)
    pos = np.zeros((height, width), dtype=np.int32)
    amb = np.zeros((height, width), dtype=np.uint8)
    tl, ntl, _keep = _tiles_arg(tiles)
    lib.gso_forward_depth(width, height, _ptr(rng_), _ptr(ids), _ptr(m), _ptr(q), _ptr(c), _ptr(o), _ptr(bg),
                          _ptr(z), tl, ntl, _ptr(tot), _ptr(med), _ptr(pos), _ptr(amb))
    return {"totals": tot, "distortion": tot[..., 3].copy(), "median_depth": med, "median_pos": pos,
            "median_ambiguous": amb.astype(bool)}


def rasterize_bwd_depth(means2d, conics, colors, opacities, background, width: int, height: int,
                        tile_ranges, sorted_ids, depths, dL_ddist=None, dL_dmedian=None, tiles=None):
    """Exact gradients of L = sum_p dL_ddist_p D_p + dL_dmedian_p median_p
    (terms of :func:`rasterize_fwd_depth`; either upstream may be None), every
    discrete decision held fixed. Returns dict of float64 arrays: dmeans2d
    [n,2], dconics [n,3], dcolors [n,3] (zeros), dopacities [n], ddepths [n]."""
    lib = _load()
    m, q, c, o = _arrs(means2d, conics, colors, opacities)
    n = m.shape[0]
    bg = np.ascontiguousarray(np.zeros(3) if background is None else background, dtype=np.float64)
    rng_ = np.ascontiguousarray(tile_ranges, dtype=np.int32)
    ids = np.ascontiguousarray(sorted_ids, dtype=np.int32)
    z = np.ascontiguousarray(depths, dtype=np.float64)
    gd = None if dL_ddist is None else np.ascontiguousarray(dL_ddist, dtype=np.float64)
    gm = None if dL_dmedian is None else np.ascontiguousarray(dL_dmedian, dtype=np.float64)
    grads = np.zeros((n, 9), dtype=np.float64)
    dz = np.zeros(n, dtype=np.float64)
    tl, ntl, _keep = _tiles_arg(tiles)
    lib.gso_backward_depth(width, height, n, _ptr(rng_), _ptr(ids), _ptr(m), _ptr(q), _ptr(c), _ptr(o),
                           _ptr(bg), _ptr(z), None if gd is None else _ptr(gd), None if gm is None else _ptr(gm),
                           tl, ntl, _ptr(grads), _ptr(dz))
    return {"dmeans2d": grads[:, 0:2].copy(), "dconics": grads[:, 2:5].copy(),
            "dcolors": grads[:, 5:8].copy(), "dopacities": grads[:, 8].copy(), "ddepths": dz}


def pixel_outcomes(means2d, conics, colors, opacities, background, width: int, height: int,
                   tile_ranges, sorted_ids, xs, ys, cap: int = 64):
    """Every admissible (image, final_T, n_contrib) of the pixels (xs, ys):
    at each decision that lies inside its float32 error band both outcomes are
    followed. Returns image [P, cap, 3], final_T [P, cap], n_contrib [P, cap]
    and count [P] (the outcomes filled in; -1 when there were more than
    ``cap``). An unflagged pixel has exactly one outcome, the forward's."""
    lib = _load()
    m, q, c, o = _arrs(means2d, conics, colors, opacities)
    bg = np.ascontiguousarray(np.zeros(3) if background is None else background, dtype=np.float64)
    rng_ = np.ascontiguousarray(tile_ranges, dtype=np.int32)
    ids = np.ascontiguousarray(sorted_ids, dtype=np.int32)
    xs = np.ascontiguousarray(xs, dtype=np.int32)
    ys = np.ascontiguousarray(ys, dtype=np.int32)
    P = len(xs)
    img = np.zeros((P, cap, 3), dtype=np.float64)
    T = np.zeros((P, cap), dtype=np.float64)
    nc = np.zeros((P, cap), dtype=np.int32)
    cnt = np.zeros(P, dtype=np.int32)
    if P:
        lib.gso_pixel_outcomes(width, height, _ptr(rng_), _ptr(ids), _ptr(m), _ptr(q), _ptr(c), _ptr(o),
                               _ptr(bg), P, _ptr(xs), _ptr(ys), cap, _ptr(img), _ptr(T), _ptr(nc), _ptr(cnt))
    return img, T, nc, cnt


def matches_an_outcome(img, T, nc, outcomes, img_tol: float, T_tol: float):
    """Per pixel: whether (img [P, 3], T [P], nc [P]) equals one of the
    pixel's admissible outcomes (from :func:`pixel_outcomes`) within the
    tolerances (n_contrib exactly). Pixels with too many outcomes count as
    not matched."""
    oi, oT, onc, cnt = outcomes
    cap = oT.shape[1]
    valid = np.arange(cap)[None, :] < cnt[:, None]
    ok = (np.abs(oi - np.asarray(img, dtype=np.float64)[:, None, :]).max(axis=2) <= img_tol) & \
         (np.abs(oT - np.asarray(T, dtype=np.float64)[:, None]) <= T_tol) & \
         (onc == np.asarray(nc)[:, None]) & valid
    return ok.any(axis=1)


# ----------------------------------------------------------------------------
# Brute force (no tiles), numpy
# ----------------------------------------------------------------------------

def composite_bruteforce(means2d, conics, colors, opacities, depths, radii, background,
                         width: int, height: int, return_margin: bool = False,
                         return_max_weight: bool = False):
    """Every pixel walks every live splat in (float32 depth bits, id) order,
    with the same skip / clamp / stop rules; no tiles and no radius test
    beyond the per-splat cull (radius <= 0 or depth not > 0). Float64 numpy,
    vectorised over pixels. Returns (image, final_T, n_steps) where n_steps
    counts composited splats per pixel; with ``return_margin`` also the
    smallest relative distance of any decision taken (skip, clamp, stop) to
    its threshold, and with ``return_max_weight`` (last) each splat's largest
    alpha T over the pixels that composite it."""
    m = np.asarray(means2d, dtype=np.float64)
    q = np.asarray(conics, dtype=np.float64)
    col = np.asarray(colors, dtype=np.float64)
    op = np.asarray(opacities, dtype=np.float64)
    d32 = np.asarray(depths, dtype=np.float32)
    live = (np.asarray(radii) > 0) & (d32 > 0) & np.isfinite(m).all(axis=1)
    ids = np.nonzero(live)[0]
    order = ids[np.lexsort((ids, d32.view(np.uint32)[ids]))]
    ys, xs = np.mgrid[0:height, 0:width]
    px = xs.ravel() + 0.5
    py = ys.ravel() + 0.5
    T = np.ones(px.shape)
    C = np.zeros((px.size, 3))
    done = np.zeros(px.shape, dtype=bool)
    nstep = np.zeros(px.shape, dtype=np.int64)
    maxw = np.zeros(m.shape[0])
    margin = np.inf
    for i in order:
        dx = px - m[i, 0]
        dy = py - m[i, 1]
        power = -0.5 * (q[i, 0] * dx * dx + q[i, 2] * dy * dy) - q[i, 1] * dx * dy
        raw = op[i] * np.exp(power)
        alpha = np.minimum(ALPHA_MAX, raw)
        use = (~done) & (alpha >= ALPHA_MIN)
        nxt = T * (1.0 - alpha)
        if return_margin:
            live_px = ~done
            if live_px.any():
                margin = min(margin, float(np.min(np.abs(alpha[live_px] / ALPHA_MIN - 1.0))))
            if use.any():
                margin = min(margin, float(np.min(np.abs(raw[use] / ALPHA_MAX - 1.0))),
                             float(np.min(np.abs(nxt[use] / T_MIN - 1.0))))
        stop = use & (nxt < T_MIN)
        done |= stop
        use &= ~stop
        C[use] += col[i] * (alpha[use] * T[use])[:, None]
        if use.any():
            maxw[i] = float(np.max(alpha[use] * T[use]))
        T = np.where(use, nxt, T)
        nstep += use
    bg = np.zeros(3) if background is None else np.asarray(background, dtype=np.float64)
    img = C + T[:, None] * bg[None, :]
    res = (img.reshape(height, width, 3), T.reshape(height, width), nstep.reshape(height, width))
    if return_margin:
        res = res + (margin,)
    if return_max_weight:
        res = res + (maxw,)
    return res


def depth_terms_bruteforce(means2d, conics, opacities, depths, radii, width: int, height: int):
    """Distortion and median with no tiles and no running sums: every pixel
    walks every live splat in (float32 depth bits, id) order with the skip /
    clamp / stop rules, recording each splat's weight w = alpha T and the
    transmittance before it; then

      D_p      = 1/2 sum_i sum_j w_i w_j (z_i - z_j)^2   (the full double sum)
      median_p = z of the last splat with w > 0 and T before it > 1/2

    Float64 numpy, vectorised over pixels; O(pixels x splats^2) memory-light
    (one splat pair row at a time). Returns (D [H,W], median_depth [H,W],
    weights [H*W, K], T_before [H*W, K], order [K])."""
    m = np.asarray(means2d, dtype=np.float64)
    q = np.asarray(conics, dtype=np.float64)
    op = np.asarray(opacities, dtype=np.float64)
    d32 = np.asarray(depths, dtype=np.float32)
    z = np.asarray(depths, dtype=np.float64)
    live = (np.asarray(radii) > 0) & (d32 > 0) & np.isfinite(m).all(axis=1)
    ids = np.nonzero(live)[0]
    order = ids[np.lexsort((ids, d32.view(np.uint32)[ids]))]
    ys, xs = np.mgrid[0:height, 0:width]
    px = xs.ravel() + 0.5
    py = ys.ravel() + 0.5
    P, K = px.size, len(order)
    Wm = np.zeros((P, K))
    Tb = np.zeros((P, K))
    T = np.ones(P)
    done = np.zeros(P, dtype=bool)
    for k, i in enumerate(order):
        dx = px - m[i, 0]
        dy = py - m[i, 1]
        alpha = np.minimum(ALPHA_MAX, op[i] * np.exp(-0.5 * (q[i, 0] * dx * dx + q[i, 2] * dy * dy) - q[i, 1] * dx * dy))
        use = (~done) & (alpha >= ALPHA_MIN)
        nxt = T * (1.0 - alpha)
        stop = use & (nxt < T_MIN)
        done |= stop
        use &= ~stop
        Wm[use, k] = alpha[use] * T[use]
        Tb[:, k] = T
        T = np.where(use, nxt, T)
    zo = z[order]
    D = np.zeros(P)
    for a in range(K):
        D += 0.5 * Wm[:, a] * (Wm * (zo[a] - zo[None, :]) ** 2).sum(axis=1)
    med = np.zeros(P)
    for k in range(K):
        sel = (Wm[:, k] > 0) & (Tb[:, k] > 0.5)
        med[sel] = zo[k]
    return D.reshape(height, width), med.reshape(height, width), Wm, Tb, order


# ----------------------------------------------------------------------------
# Convenience over a scenes.Scene
# ----------------------------------------------------------------------------

def run_scene(sc, tiles=None, backward=True, dL_dimage=None):
    """Bin, forward and (optionally) backward a scene. Returns a dict."""
    ids, rng_ = bin_tiles(sc.means2d, sc.conics, sc.opacities, sc.radii, sc.depths, sc.width, sc.height)
    out = {"sorted_ids": ids, "tile_ranges": rng_}
    out.update(rasterize_fwd(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background,
                             sc.width, sc.height, rng_, ids, tiles=tiles))
    if backward:
        g = sc.dL_dimage if dL_dimage is None else dL_dimage
        out.update(rasterize_bwd(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background,
                                 sc.width, sc.height, rng_, ids, g, tiles=tiles))
    return out
