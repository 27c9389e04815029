"""Seeded synthetic splat scenes for the tile rasterizer.

This module only draws inputs. It holds none of the rasterizer's arithmetic
(no alpha, no compositing, no binning, no gradients), so both the HIP library's
tests/benchmarks and the CPU oracle may use it without sharing method code.

A scene is what the rasterization step receives from the (out-of-scope)
projection step: per-splat 2D means in pixels, an inverse 2D covariance
("conic"), colour, opacity, view depth and an integer screen radius, plus the
upstream gradient dL/dImage.

Workloads (sizes from the pages where they give them):
  * ``tiny``   64x64, 256 splats: a small case that spans several tiles.
  * ``early``  256x256, 5,207 splats: the splat count before densification in
    the run timed on page "Phase 5 step 30b — kernel-by-kernel timing"
    (section 本文, "splat 数").
  * ``mid``    1237x822, 76,363 splats: the splat count after densification on
    that same page; 1237x822 is the raster_bench scene size of the Spirula
    Studio page (section 亲手验证). The page's scene is not named, so means
    are drawn as 70% clustered / 30% uniform to give an uneven tile load.
  * ``bench``  1237x822, 2,000,000 splats: the fixed raster_bench load of the
    Spirula Studio page (section 亲手验证: 2M splats, 20 iterations).
  * ``stress`` 1920x1080, 1,000,000 large splats (hundreds per tile), with the
    per-splat accumulated blend weight switched on (the "accum weight"
    optional feature named in section 机制拆解 of the Spirula Studio page).

Neither page publishes its value distributions; the laws below are the
documented synthetic stand-ins.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

TILE = 16


@dataclasses.dataclass
class Scene:
    name: str
    seed: int
    width: int
    height: int
    means2d: np.ndarray      # [n, 2] float32, pixels, image spans [0, W) x [0, H)
    conics: np.ndarray       # [n, 3] float32, (a, b, c) = upper triangle of Sigma^-1
    colors: np.ndarray       # [n, 3] float32
    opacities: np.ndarray    # [n]    float32
    depths: np.ndarray       # [n]    float32, > 0
    radii: np.ndarray        # [n]    int32, <= 0 means culled
    dL_dimage: np.ndarray    # [H, W, 3] float32
    background: np.ndarray   # [3] float32
    accum_weight: bool       # whether the workload asks for sum(alpha*T) per splat

    @property
    def n(self) -> int:
        return int(self.means2d.shape[0])

    @property
    def grid(self) -> tuple[int, int]:
        return ((self.width + TILE - 1) // TILE, (self.height + TILE - 1) // TILE)


@dataclasses.dataclass(frozen=True)
class Recipe:
    width: int
    height: int
    n: int
    sigma_law: str           # "uniform" or "loguniform"
    sigma_lo: float
    sigma_hi: float
    opacity_law: str         # "uniform" or "beta22"
    opacity_lo: float
    opacity_hi: float
    depth_hi: float
    grad_std: float
    clustered: bool = False
    accum_weight: bool = False


RECIPES: dict[str, Recipe] = {
    "tiny":   Recipe(64, 64, 256, "uniform", 1.0, 6.0, "uniform", 0.05, 0.99, 10.0, 1.0),
    "early":  Recipe(256, 256, 5207, "loguniform", 0.5, 8.0, "uniform", 0.05, 0.99, 10.0, 1.0),
    "mid":    Recipe(1237, 822, 76363, "loguniform", 0.5, 12.0, "beta22", 0.0, 0.99, 20.0, 0.1,
                     clustered=True),
    "bench":  Recipe(1237, 822, 2_000_000, "loguniform", 0.3, 6.0, "uniform", 0.01, 0.99, 50.0, 0.1),
    "stress": Recipe(1920, 1080, 1_000_000, "loguniform", 4.0, 40.0, "uniform", 0.01, 0.5, 50.0, 0.1,
                     accum_weight=True),
}

CONFIG_ORDER = ["tiny", "early", "mid", "bench", "stress"]


def screen_radius(sigma_max: np.ndarray, opacity: np.ndarray) -> np.ndarray:
    """Integer screen radius handed over by the projection step.

    Conservative for a 1/255 alpha cut: a splat with opacity o is below 1/255
    wherever d^T Sigma^-1 d > 2 ln(255 o), which lies inside |d| <= s_max *
    sqrt(2 ln(255 o)). One pixel of margin is added. Splats that can never
    reach 1/255 (255 o <= 1) get radius 0 (culled). Computed in float64.
    """
    o = opacity.astype(np.float64)
    arg = 255.0 * o
    r = np.zeros(o.shape, dtype=np.int64)
    ok = arg > 1.0
    ext = sigma_max[ok] * np.sqrt(2.0 * np.log(arg[ok]))
    r[ok] = np.ceil(ext).astype(np.int64) + 1
    return r.astype(np.int32)


def _means(rng: np.random.Generator, rc: Recipe) -> np.ndarray:
    W, H, n = rc.width, rc.height, rc.n
    if not rc.clustered:
        return np.stack([rng.uniform(0.0, W, n), rng.uniform(0.0, H, n)], axis=1)
    n_cl = int(round(0.7 * n))
    centres = np.stack([rng.uniform(0.0, W, 32), rng.uniform(0.0, H, 32)], axis=1)
    which = rng.integers(0, 32, n_cl)
    pts = centres[which] + rng.normal(0.0, 60.0, (n_cl, 2))
    bad = (pts[:, 0] < 0) | (pts[:, 0] >= W) | (pts[:, 1] < 0) | (pts[:, 1] >= H)
    while bad.any():   # resample outliers until every clustered mean lies in the image
        k = int(bad.sum())
        pts[bad] = centres[which[bad]] + rng.normal(0.0, 60.0, (k, 2))
        bad = (pts[:, 0] < 0) | (pts[:, 0] >= W) | (pts[:, 1] < 0) | (pts[:, 1] >= H)
    uni = np.stack([rng.uniform(0.0, W, n - n_cl), rng.uniform(0.0, H, n - n_cl)], axis=1)
    out = np.concatenate([pts, uni], axis=0)
    return out[rng.permutation(n)]


def _sigmas(rng: np.random.Generator, rc: Recipe) -> np.ndarray:
    if rc.sigma_law == "uniform":
        return rng.uniform(rc.sigma_lo, rc.sigma_hi, (rc.n, 2))
    lo, hi = math.log(rc.sigma_lo), math.log(rc.sigma_hi)
    return np.exp(rng.uniform(lo, hi, (rc.n, 2)))


def conic_from_axes(sig: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """Sigma = R(theta) diag(s1^2, s2^2) R(theta)^T, returned as Sigma^-1 (a, b, c) in float64."""
    c, s = np.cos(theta), np.sin(theta)
    i1, i2 = 1.0 / sig[:, 0] ** 2, 1.0 / sig[:, 1] ** 2
    # Sigma^-1 = R diag(1/s1^2, 1/s2^2) R^T
    a = c * c * i1 + s * s * i2
    b = c * s * (i1 - i2)
    cc = s * s * i1 + c * c * i2
    return np.stack([a, b, cc], axis=1)


def make_scene(name: str, seed: int = 0, n: int | None = None) -> Scene:
    """Draw the named workload with ``numpy.random.default_rng(seed)``.

    ``n`` optionally overrides the splat count (used for reduced-size cases
    of the same distributions)."""
    rc = RECIPES[name]
    if n is not None:
        rc = dataclasses.replace(rc, n=int(n))
    rng = np.random.default_rng(seed)
    means = _means(rng, rc)
    sig = _sigmas(rng, rc)
    theta = rng.uniform(0.0, math.pi, rc.n)
    if rc.opacity_law == "uniform":
        opac = rng.uniform(rc.opacity_lo, rc.opacity_hi, rc.n)
    else:
        opac = rc.opacity_hi * rng.beta(2.0, 2.0, rc.n)
    colors = rng.uniform(0.0, 1.0, (rc.n, 3))
    depths = rng.uniform(0.1, rc.depth_hi, rc.n)
    dimg = rng.normal(0.0, rc.grad_std, (rc.height, rc.width, 3))
    conic = conic_from_axes(sig, theta)
    radii = screen_radius(sig.max(axis=1), opac.astype(np.float32))
    return Scene(
        name=name, seed=seed, width=rc.width, height=rc.height,
        means2d=np.ascontiguousarray(means, dtype=np.float32),
        conics=np.ascontiguousarray(conic, dtype=np.float32),
        colors=np.ascontiguousarray(colors, dtype=np.float32),
        opacities=np.ascontiguousarray(opac, dtype=np.float32),
        depths=np.ascontiguousarray(depths, dtype=np.float32),
        radii=np.ascontiguousarray(radii, dtype=np.int32),
        dL_dimage=np.ascontiguousarray(dimg, dtype=np.float32),
        background=np.zeros(3, dtype=np.float32),
        accum_weight=rc.accum_weight,
    )


def custom_scene(width: int, height: int, means2d, sigmas, thetas, opacities, colors, depths,
                 dL_dimage=None, background=None, radii=None, seed: int = 0,
                 accum_weight: bool = False) -> Scene:
    """Build a hand-specified scene (for the small closed-form and edge cases)."""
    means2d = np.asarray(means2d, dtype=np.float64).reshape(-1, 2)
    n = means2d.shape[0]
    sig = np.asarray(sigmas, dtype=np.float64).reshape(n, 2)
    th = np.asarray(thetas, dtype=np.float64).reshape(n)
    op = np.asarray(opacities, dtype=np.float64).reshape(n)
    if radii is None:
        radii = screen_radius(sig.max(axis=1), op.astype(np.float32))
    if dL_dimage is None:
        dL_dimage = np.random.default_rng(seed).normal(0.0, 1.0, (height, width, 3))
    if background is None:
        background = np.zeros(3)
    return Scene(
        name="custom", seed=seed, width=int(width), height=int(height),
        means2d=np.ascontiguousarray(means2d, dtype=np.float32),
        conics=np.ascontiguousarray(conic_from_axes(sig, th), dtype=np.float32),
        colors=np.ascontiguousarray(np.asarray(colors).reshape(n, 3), dtype=np.float32),
        opacities=np.ascontiguousarray(op, dtype=np.float32),
        depths=np.ascontiguousarray(np.asarray(depths).reshape(n), dtype=np.float32),
        radii=np.ascontiguousarray(np.asarray(radii).reshape(n), dtype=np.int32),
        dL_dimage=np.ascontiguousarray(dL_dimage, dtype=np.float32),
        background=np.ascontiguousarray(background, dtype=np.float32),
        accum_weight=accum_weight,
    )


def depth_upstream(sc: Scene, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Upstream gradients of the per-pixel depth outputs (distortion, median
    depth) for a scene: two [H, W] float32 fields of standard normals, drawn
    with ``numpy.random.default_rng(10000 + seed)``."""
    rng = np.random.default_rng(10000 + seed)
    g_dist = rng.standard_normal((sc.height, sc.width), dtype=np.float32)
    g_median = rng.standard_normal((sc.height, sc.width), dtype=np.float32)
    return g_dist, g_median
