"""Pins for the CPU oracle, against things other than itself.

* a brute-force composite with no tiles (numpy, separate code);
* hand-derived closed forms (tests/golden/closed_forms.json) and the
  Gaussian density of scipy.stats.multivariate_normal (pins the conic
  convention: conic = Sigma^-1 with b the off-diagonal entry);
* central finite differences of the forward (pins every gradient field);
* exact identities (colour-gradient sum, weight sum, linearity, tile
  translation) and the compositing invariants;
* a naive per-tile membership loop for binning and sort order.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.stats

import oracle
import scenes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _scene_from_case(case):
    sp = case["splats"]
    return scenes.custom_scene(
        case["width"], case["height"],
        means2d=[s["mean"] for s in sp], sigmas=[s["sigma"] for s in sp],
        thetas=[s.get("theta", 0.0) for s in sp], opacities=[s["opacity"] for s in sp],
        colors=[s["color"] for s in sp], depths=[s["depth"] for s in sp],
        background=case.get("background"))


def _tiled(sc, **kw):
    return oracle.run_scene(sc, **kw)


def _loss(sc, ids, rng_, means, conics, colors, opac, g):
    out = oracle.rasterize_fwd(means, conics, colors, opac, sc.background, sc.width, sc.height, rng_, ids)
    return float(np.sum(out["image"] * g))


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_closed_forms(case):
    sc = _scene_from_case(case)
    out = _tiled(sc, backward=False)
    x, y = case["at"]
    np.testing.assert_allclose(out["image"][y, x], case["image"], atol=case["tol"], rtol=0)
    assert abs(out["final_T"][y, x] - case["final_T"]) <= case["tol"]
    assert out["n_contrib"][y, x] == case["n_contrib"]


def test_density_matches_scipy_mvn():
    """One anisotropic splat: every pixel equals colour * min(0.99, o * G) with
    G the unnormalised Gaussian density of covariance inv([[a, b], [b, c]])."""
    sc = scenes.custom_scene(32, 32, means2d=[[13.3, 17.9]], sigmas=[[2.5, 5.0]], thetas=[0.6],
                             opacities=[0.8], colors=[[0.3, 0.6, 0.9]], depths=[1.0])
    out = _tiled(sc, backward=False)
    a, b, c = sc.conics[0].astype(np.float64)
    cov = np.linalg.inv(np.array([[a, b], [b, c]]))
    mvn = scipy.stats.multivariate_normal(mean=sc.means2d[0].astype(np.float64), cov=cov)
    ys, xs = np.mgrid[0:32, 0:32]
    pts = np.stack([xs.ravel() + 0.5, ys.ravel() + 0.5], axis=1)
    G = mvn.pdf(pts) * 2.0 * math.pi * math.sqrt(np.linalg.det(cov))
    alpha = np.minimum(0.99, float(sc.opacities[0]) * G)
    alpha = np.where(alpha >= 1.0 / 255.0, alpha, 0.0)
    exp_img = alpha[:, None] * sc.colors[0].astype(np.float64)[None, :]
    np.testing.assert_allclose(out["image"].reshape(-1, 3), exp_img, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(out["final_T"].ravel(), 1.0 - alpha, atol=1e-12)


# ----------------------------------------------------------- brute force pins

def _ragged_scene(seed, W=50, H=37, n=40):
    rng = np.random.default_rng(seed)
    return scenes.custom_scene(
        W, H, means2d=np.stack([rng.uniform(-5, W + 5, n), rng.uniform(-5, H + 5, n)], 1),
        sigmas=rng.uniform(0.7, 7.0, (n, 2)), thetas=rng.uniform(0, math.pi, n),
        opacities=rng.uniform(0.05, 1.0, n), colors=rng.uniform(0, 1, (n, 3)),
        depths=rng.uniform(0.1, 10, n), background=rng.uniform(0, 1, 3), seed=seed)


@pytest.mark.parametrize("maker", [
    lambda: scenes.make_scene("tiny", 0), lambda: scenes.make_scene("tiny", 1),
    lambda: scenes.make_scene("tiny", 2), lambda: _ragged_scene(3), lambda: _ragged_scene(4),
    lambda: scenes.make_scene("early", 0, n=800),
], ids=["tiny0", "tiny1", "tiny2", "ragged3", "ragged4", "early-800"])
def test_tiled_equals_bruteforce(maker):
    sc = maker()
    out = _tiled(sc, backward=False)
    img, T, _ = oracle.composite_bruteforce(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.depths,
                                            sc.radii, sc.background, sc.width, sc.height)
    np.testing.assert_allclose(out["image"], img, atol=1e-12, rtol=0)
    np.testing.assert_allclose(out["final_T"], T, atol=1e-12, rtol=0)


def test_compositing_invariants():
    sc = scenes.make_scene("tiny", 0)
    out = _tiled(sc, backward=False)
    T = out["final_T"]
    assert np.all(T <= 1.0) and np.all(T >= 1e-4)
    lens = out["tile_ranges"][:, 1] - out["tile_ranges"][:, 0]
    GX, _ = oracle.grid(sc.width, sc.height)
    ys, xs = np.mgrid[0:sc.height, 0:sc.width]
    tile_of_px = (ys // 16) * GX + xs // 16
    assert np.all(out["n_contrib"] <= lens[tile_of_px])
    assert np.all(out["n_contrib"] >= 0)
    # a pixel with no composited splat has T = 1
    assert np.all(T[out["n_contrib"] == 0] == 1.0)


# ---------------------------------------------------------------- binning

def _min_q_over_rect(a, b, c, mx, my, x0, x1, y0, y1):
    """Float64 minimum of Q(u, v) = a u^2 + 2 b u v + c v^2 (u = x - mx,
    v = y - my) over the rectangle [x0, x1] x [y0, y1]: 0 if the mean is
    inside, else the least of the four edges' minima (a 1D quadratic along an
    edge, its minimiser clamped to the edge)."""
    if x0 <= mx <= x1 and y0 <= my <= y1:
        return 0.0
    best = math.inf
    for x in (x0, x1):                  # vertical edges: u fixed, v in [y0 - my, y1 - my]
        u = x - mx
        v = min(max(-b * u / c, y0 - my), y1 - my)
        best = min(best, a * u * u + 2 * b * u * v + c * v * v)
    for y in (y0, y1):                  # horizontal edges
        v = y - my
        u = min(max(-b * v / a, x0 - mx), x1 - mx)
        best = min(best, a * u * u + 2 * b * u * v + c * v * v)
    return best


def _cull_threshold64(o):
    """The culling threshold's formula in float64: 2 (e2 ln 2 + (m2 - 1) /
    sqrt(m2)) (1 + 2^-10) + 2^-10 with 255 o = m2 2^e2, m2 in [1, 2)."""
    y = 255.0 * float(np.float32(255.0) * np.float32(o)) / 255.0
    mant, ex = math.frexp(y)
    m2, e2 = 2.0 * mant, ex - 1
    T = 2.0 * (e2 * math.log(2.0) + (m2 - 1.0) / math.sqrt(m2))
    return T * (1.0 + 2.0 ** -10) + 2.0 ** -10


def _naive_bins(sc):
    """Per tile, loop over every splat: the float32 rectangle test, then the
    culling test written independently (float64 minimum of the quadratic form
    over the tile's pixel-centre rectangle against the threshold). Returns the
    lists and the (tile, splat) pairs whose culling decision lies within 1e-4
    of its threshold (there a float32 evaluation may decide either way)."""
    GX, GY = oracle.grid(sc.width, sc.height)
    f = np.float32
    lists, ambiguous = [], set()
    for ty in range(GY):
        for tx in range(GX):
            mem = []
            for i in range(sc.n):
                if not (sc.radii[i] > 0 and sc.depths[i] > 0 and f(255.0) * sc.opacities[i] >= 1):
                    continue
                r = f(sc.radii[i])
                lo_x = math.floor(f(sc.means2d[i, 0] - r) * f(0.0625))
                hi_x = math.floor(f(sc.means2d[i, 0] + r) * f(0.0625))
                lo_y = math.floor(f(sc.means2d[i, 1] - r) * f(0.0625))
                hi_y = math.floor(f(sc.means2d[i, 1] + r) * f(0.0625))
                if not (lo_x <= tx <= hi_x and lo_y <= ty <= hi_y):
                    continue
                a, b, c = (float(v) for v in sc.conics[i])
                q = _min_q_over_rect(a, b, c, float(sc.means2d[i, 0]), float(sc.means2d[i, 1]),
                                     16 * tx + 0.5, 16 * tx + 15.5, 16 * ty + 0.5, 16 * ty + 15.5)
                T = _cull_threshold64(sc.opacities[i])
                if abs(q - T) <= 1e-4 * max(T, 1.0):
                    ambiguous.add((ty * GX + tx, i))
                if q <= T:
                    mem.append((int(sc.depths[i:i + 1].view(np.uint32)[0]), i))
            lists.append([i for _, i in sorted(mem)])
    return lists, ambiguous


def _bins(sc):
    return oracle.bin_tiles(sc.means2d, sc.conics, sc.opacities, sc.radii, sc.depths, sc.width, sc.height)


@pytest.mark.parametrize("seed", [0, 1])
def test_binning_matches_naive_membership(seed):
    sc = _ragged_scene(seed, n=60)
    # force some equal depths so the id tie-break is exercised
    sc.depths[::3] = sc.depths[0]
    ids, rng_ = _bins(sc)
    naive, amb = _naive_bins(sc)
    for t, lst in enumerate(naive):
        s, e = rng_[t]
        got = list(ids[s:e])
        if got != lst:  # only decisions within the ambiguity band may differ
            assert set(got) ^ set(lst) <= {i for (tt, i) in amb if tt == t}, t
            assert [i for i in got if i in lst] == [i for i in lst if i in got], t
    assert len(amb) <= 2
    assert sum(len(x) for x in naive) > 0.3 * len(oracle.kept_pairs(
        sc.means2d, sc.conics, sc.opacities, sc.radii, sc.depths, sc.width, sc.height)[3])


def test_binning_invariants_tiny():
    sc = scenes.make_scene("tiny", 0)
    ids, rng_ = _bins(sc)
    _, _, _, kept = oracle.kept_pairs(sc.means2d, sc.conics, sc.opacities, sc.radii, sc.depths, sc.width, sc.height)
    assert int(kept.sum()) == len(ids)
    nonempty = rng_[rng_[:, 1] > rng_[:, 0]]
    assert nonempty[0, 0] == 0 and nonempty[-1, 1] == len(ids)
    assert np.all(nonempty[1:, 0] == nonempty[:-1, 1])       # contiguous, in tile order
    db = sc.depths.view(np.uint32)
    for s, e in nonempty:
        key = db[ids[s:e]].astype(np.int64) * (1 << 32) + ids[s:e]
        assert np.all(np.diff(key) > 0)


def _member(ids, rng_, GX, i, tile):
    s, e = rng_[tile]
    return i in set(ids[s:e].tolist())


@pytest.mark.parametrize("maker", [lambda: scenes.make_scene("tiny", 1), lambda: _ragged_scene(7, n=80)],
                         ids=["tiny1", "ragged7"])
def test_binning_is_conservative(maker):
    """Every pixel where a splat reaches alpha >= 1/255 (float64) lies in a
    tile whose list holds the splat: the rectangle and the culling ellipse
    both keep every such pixel's tile."""
    sc = maker()
    ids, rng_ = _bins(sc)
    GX, _ = oracle.grid(sc.width, sc.height)
    lists = [set(ids[s:e].tolist()) for s, e in rng_]
    ys, xs = np.mgrid[0:sc.height, 0:sc.width]
    tested = 0
    for i in range(sc.n):
        if not (sc.radii[i] > 0 and sc.depths[i] > 0):
            continue
        dx = xs + 0.5 - float(sc.means2d[i, 0])
        dy = ys + 0.5 - float(sc.means2d[i, 1])
        a, b, c = sc.conics[i].astype(np.float64)
        al = float(sc.opacities[i]) * np.exp(-0.5 * (a * dx * dx + c * dy * dy) - b * dx * dy)
        yy, xx = np.nonzero(al >= 1.0 / 255.0)
        for t in set(((yy // 16) * GX + xx // 16).tolist()):
            assert i in lists[t], (i, t)
            tested += 1
    assert tested > 100


def test_binning_culls_tightly():
    """Every listed pair's tile rectangle comes within the threshold's slack of
    the splat's alpha = 1/255 ellipse (the logarithm bound adds at most 0.028,
    the margin 2^-10 (T + 1)), and the culling really removes pairs."""
    sc = scenes.make_scene("early", 0, n=1500)
    ids, tx, ty, kept = oracle.kept_pairs(sc.means2d, sc.conics, sc.opacities, sc.radii, sc.depths,
                                          sc.width, sc.height)
    assert 0.3 < kept.mean() < 0.8
    sel = np.nonzero(kept)[0][::7]
    for k in sel:
        i = ids[k]
        a, b, c = (float(v) for v in sc.conics[i])
        q = _min_q_over_rect(a, b, c, float(sc.means2d[i, 0]), float(sc.means2d[i, 1]),
                             16 * tx[k] + 0.5, 16 * tx[k] + 15.5, 16 * ty[k] + 0.5, 16 * ty[k] + 15.5)
        T = 2.0 * math.log(255.0 * float(sc.opacities[i]))
        assert q <= T + 0.028 + 2.0 ** -10 * (T + 1.0) + 1e-4 * (T + 1.0), (k, q, T)


def test_rect_is_conservative():
    """Every pixel where a splat reaches alpha >= 1/255 lies in a tile of its rectangle."""
    sc = scenes.make_scene("tiny", 1)
    tx0, tx1, ty0, ty1 = oracle.tile_rects(sc.means2d, sc.radii, sc.depths, sc.width, sc.height)
    ys, xs = np.mgrid[0:sc.height, 0:sc.width]
    for i in range(sc.n):
        dx = xs + 0.5 - float(sc.means2d[i, 0])
        dy = ys + 0.5 - float(sc.means2d[i, 1])
        a, b, c = sc.conics[i].astype(np.float64)
        al = float(sc.opacities[i]) * np.exp(-0.5 * (a * dx * dx + c * dy * dy) - b * dx * dy)
        yy, xx = np.nonzero(al >= 1.0 / 255.0)
        assert np.all((xx // 16 >= tx0[i]) & (xx // 16 < tx1[i]) & (yy // 16 >= ty0[i]) & (yy // 16 < ty1[i]))


def test_culled_splats_never_binned():
    sc = _ragged_scene(5, n=20)
    sc.radii[0] = 0
    sc.depths[1] = -1.0
    sc.depths[2] = 0.0
    sc.opacities[3] = np.float32(1.0 / 256.0)   # 255 o <= 1: alpha never reaches 1/255
    ids, _ = _bins(sc)
    assert not np.isin([0, 1, 2, 3], ids).any()


def degenerate_cull_scene():
    """Splats whose culling constants are degenerate, each with a non-empty
    rectangle: the binning keeps the whole rectangle where the factors are not
    finite and positive, and nothing where 255 o < 1 (float32) or o is NaN.
    Shared with the GPU binning test."""
    sc = _ragged_scene(21, n=40)
    f = np.float32
    sc.radii[:12] = np.maximum(sc.radii[:12], 20)
    sc.depths[:12] = np.abs(sc.depths[:12]) + f(1.0)
    q = sc.conics
    q[0] = (0.0, 0.0, 0.5)                 # a = 0: l11 = 0
    q[1] = (-0.2, 0.0, 0.5)                # a < 0: l11 NaN
    q[2] = (0.25, 0.5, 1.0)                # c = b^2 / a: l22 = 0
    q[3] = (np.inf, 0.0, 0.5)              # l11 infinite
    q[4] = (0.3, 0.0, np.nan)              # l22 NaN
    sc.opacities[5] = f(0.5 / 255.0)       # 255 o < 1: nowhere
    sc.opacities[6] = f(np.nan)            # nowhere
    sc.opacities[7] = f(np.inf)            # T infinite: whole rectangle
    sc.opacities[8] = f(1.0) / f(255.0)    # 255 o rounds to 1: T = 2^-10, a speck
    sc.opacities[9] = np.nextafter(f(1.0) / f(255.0), f(0.0))
    return sc


def test_culling_degenerate_inputs():
    sc = degenerate_cull_scene()
    ids, tx, ty, kept = oracle.kept_pairs(sc.means2d, sc.conics, sc.opacities, sc.radii, sc.depths, sc.width,
                                          sc.height)
    for i in range(5):
        assert (ids == i).sum() > 0 and kept[ids == i].all(), i      # whole rectangle
    for i in (5, 6):
        assert (ids == i).sum() > 0 and not kept[ids == i].any(), i  # nowhere
    assert kept[ids == 7].all()
    # 255 o rounded to 1: the threshold is 2^-10, the ellipse a speck around
    # the mean: at most the tiles holding pixel centres within ~0.1 px of it
    assert 0 < kept[ids == 8].sum() <= 4
    y9 = np.float32(255.0) * sc.opacities[9]
    assert kept[ids == 9].any() == bool(y9 >= 1.0)


# ---------------------------------------------------------------- gradients

def _fd_scene(seed, n=6, bg=None, clamp=False):
    rng = np.random.default_rng(100 + seed)
    op = rng.uniform(0.3, 0.95, n)
    means = rng.uniform(3, 13, (n, 2))
    sig = rng.uniform(1.5, 4.0, (n, 2))
    if clamp:
        # two near-opaque splats centred close to a pixel centre: o G > 0.99 there
        op[:2] = [1.0, 0.995]
        means[:2] = [[8.6, 8.4], [4.55, 11.45]]
        sig[:2] = [[4.0, 4.0], [3.5, 3.0]]
    return scenes.custom_scene(
        16, 16, means2d=means, sigmas=sig,
        thetas=rng.uniform(0, math.pi, n), opacities=op, colors=rng.uniform(0, 1, (n, 3)),
        depths=rng.uniform(0.1, 10, n), background=bg, seed=seed)


def _margin(sc):
    return oracle.composite_bruteforce(
        sc.means2d, sc.conics, sc.colors, sc.opacities, sc.depths, sc.radii, sc.background,
        sc.width, sc.height, return_margin=True)[3]


def _first_clear(make, seeds):
    """First scene whose decisions all sit > 1e-3 (relative) from a threshold,
    so that a finite-difference step cannot cross one."""
    for s in seeds:
        sc = make(s)
        if _margin(sc) > 1e-3:
            return sc
    raise AssertionError("no scene clear of the thresholds")


def _fd_check(sc):
    out = _tiled(sc)
    ids, rng_ = out["sorted_ids"], out["tile_ranges"]
    base = [sc.means2d.astype(np.float64), sc.conics.astype(np.float64),
            sc.colors.astype(np.float64), sc.opacities.astype(np.float64)]
    g = sc.dL_dimage.astype(np.float64)
    fields = [("dmeans2d", 0, 2), ("dconics", 1, 3), ("dcolors", 2, 3), ("dopacities", 3, 1)]
    for name, arg, width in fields:
        an = out[name].reshape(sc.n, width)
        fd = np.zeros_like(an)
        for i in range(sc.n):
            for k in range(width):
                vals = []
                for sgn in (+1, -1):
                    p = [b.copy() for b in base]
                    view = p[arg].reshape(sc.n, width)
                    h = 1e-6 * max(1.0, abs(view[i, k]))
                    view[i, k] += sgn * h
                    vals.append(_loss(sc, ids, rng_, *p, g))
                fd[i, k] = (vals[0] - vals[1]) / (2 * h)
        scale = max(np.abs(an).max(), 1e-3)
        np.testing.assert_allclose(an, fd, atol=1e-6 * scale, rtol=1e-6, err_msg=name)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_gradients_match_central_differences(seed):
    _fd_check(_first_clear(_fd_scene, range(10 * seed, 10 * seed + 10)))


def test_gradients_fd_with_background():
    _fd_check(_first_clear(lambda s: _fd_scene(s, bg=[0.3, 0.5, 0.9]), range(50, 60)))


def test_gradients_fd_with_clamped_splats():
    sc = _first_clear(lambda s: _fd_scene(s, clamp=True), range(60, 90))
    # the clamp is really hit: some pixel has opacity * G > 0.99
    ys, xs = np.mgrid[0:16, 0:16]
    a, b, c = sc.conics[0].astype(np.float64)
    dx, dy = xs + 0.5 - float(sc.means2d[0, 0]), ys + 0.5 - float(sc.means2d[0, 1])
    assert (float(sc.opacities[0]) * np.exp(-0.5 * (a * dx * dx + c * dy * dy) - b * dx * dy) > 0.99).any()
    _fd_check(sc)


def _stacked(seed, n=6):
    rng = np.random.default_rng(seed)
    return scenes.custom_scene(16, 16, means2d=8.0 + rng.uniform(-1.5, 1.5, (n, 2)),
                               sigmas=rng.uniform(6.0, 9.0, (n, 2)), thetas=rng.uniform(0, 3, n),
                               opacities=rng.uniform(0.93, 0.97, n), colors=rng.uniform(0, 1, (n, 3)),
                               depths=np.arange(1, n + 1, dtype=float), seed=seed)


def test_gradients_fd_with_early_stop():
    """Stacked dense splats so that most pixels stop early."""
    sc = _first_clear(_stacked, range(5, 40))
    out = _tiled(sc, backward=False)
    assert (out["n_contrib"] < sc.n).mean() > 0.2      # the stop is actually exercised
    _fd_check(sc)


def test_colour_gradient_and_weight_identities():
    sc = scenes.make_scene("tiny", 2)
    out = _tiled(sc)
    g = sc.dL_dimage.astype(np.float64)
    one_minus_T = 1.0 - out["final_T"]
    np.testing.assert_allclose(out["dcolors"].sum(axis=0), (g * one_minus_T[..., None]).sum(axis=(0, 1)),
                               rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(out["accum_weight"].sum(), one_minus_T.sum(), rtol=1e-12)


def test_gradients_linear_in_upstream():
    sc = scenes.make_scene("tiny", 0)
    rng = np.random.default_rng(9)
    g1 = rng.normal(size=sc.dL_dimage.shape)
    g2 = rng.normal(size=sc.dL_dimage.shape)
    r1 = _tiled(sc, dL_dimage=g1)
    r2 = _tiled(sc, dL_dimage=g2)
    r3 = _tiled(sc, dL_dimage=2 * g1 - 3 * g2)
    r0 = _tiled(sc, dL_dimage=np.zeros_like(g1))
    for k in ["dmeans2d", "dconics", "dcolors", "dopacities"]:
        np.testing.assert_allclose(r3[k], 2 * r1[k] - 3 * r2[k], atol=1e-10)
        assert np.all(r0[k] == 0)


def test_translation_by_one_tile():
    """Moving every mean and the upstream gradient by (16, 16) on a larger image changes nothing."""
    sc = _ragged_scene(8, W=40, H=40, n=30)
    # means on a 1/1024 grid so that adding 16 is exact in float32
    sc.means2d[:] = np.round(np.clip(sc.means2d, 2, 38) * 1024) / 1024
    big = scenes.custom_scene(56, 56, means2d=sc.means2d + 16, sigmas=np.ones((sc.n, 2)),
                              thetas=np.zeros(sc.n), opacities=sc.opacities, colors=sc.colors,
                              depths=sc.depths, radii=sc.radii, background=sc.background)
    big.conics[:] = sc.conics
    g = np.zeros((56, 56, 3), dtype=np.float32)
    g[16:, 16:] = sc.dL_dimage[:40, :40]
    big.dL_dimage = g
    a = _tiled(sc)
    b = _tiled(big)
    np.testing.assert_allclose(b["image"][16:, 16:], a["image"], atol=1e-13)
    for k in ["dmeans2d", "dconics", "dcolors", "dopacities", "accum_weight"]:
        if k == "accum_weight":
            continue   # weight also collects from the border pixels outside the old image
        np.testing.assert_allclose(b[k], a[k], atol=1e-11, rtol=1e-9, err_msg=k)


def test_ambiguity_flags_only_near_thresholds_early():
    sc = scenes.make_scene("early", 0)
    out = _tiled(sc, backward=False)
    frac = out["ambiguous"].mean()
    assert frac < 1e-3, frac


# ------------------------------------------------------------------ max weight
# The per-splat "max wt" statistic: the largest alpha T a splat receives over
# the pixels that composite it (the raster_bench line of the Spirula Studio
# page, section 亲手验证, named there without a formula).

def _max_weight(sc, out):
    return oracle.max_weight(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background,
                             sc.width, sc.height, out["tile_ranges"], out["sorted_ids"])


@pytest.mark.parametrize("maker", [
    lambda: scenes.make_scene("tiny", 0), lambda: scenes.make_scene("tiny", 1),
    lambda: _ragged_scene(3), lambda: scenes.make_scene("early", 0, n=800),
], ids=["tiny0", "tiny1", "ragged3", "early-800"])
def test_max_weight_equals_bruteforce(maker):
    sc = maker()
    out = _tiled(sc, backward=False)
    mw, _ = _max_weight(sc, out)
    *_, bmw = oracle.composite_bruteforce(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.depths,
                                          sc.radii, sc.background, sc.width, sc.height,
                                          return_max_weight=True)
    np.testing.assert_allclose(mw, bmw, atol=1e-12, rtol=0)


@pytest.mark.parametrize("o", [0.3, 0.7, 0.995])
def test_max_weight_single_splat(o):
    """Alone, a splat centred on a pixel centre takes its largest weight there,
    with T = 1 and G = 1: min(0.99, o)."""
    sc = scenes.custom_scene(16, 16, means2d=[[8.5, 7.5]], sigmas=[[1.5, 2.5]], thetas=[0.4],
                             opacities=[o], colors=[[0.5, 0.5, 0.5]], depths=[1.0])
    mw, unc = _max_weight(sc, _tiled(sc, backward=False))
    assert not unc.any()
    assert abs(mw[0] - min(0.99, o)) <= 1e-7   # float32 storage of the opacity


def test_max_weight_behind_a_weak_splat():
    """Two concentric isotropic splats, front opacity o1 <= 1/2: the back one's
    weight o2 G (1 - o1 G) grows with G up to G = 1, so its maximum is at the
    centre pixel: o2 (1 - o1); the front one's is o1."""
    o1, o2 = 0.375, 0.8125   # exact in float32
    sc = scenes.custom_scene(32, 32, means2d=[[16.5, 16.5]] * 2, sigmas=[[3.0, 3.0]] * 2,
                             thetas=[0.0, 0.0], opacities=[o1, o2], colors=[[1, 0, 0], [0, 1, 0]],
                             depths=[1.0, 2.0])
    mw, _ = _max_weight(sc, _tiled(sc, backward=False))
    np.testing.assert_allclose(mw, [o1, o2 * (1 - o1)], atol=1e-12, rtol=0)


def test_max_weight_off_centre():
    """Front opacity o1 > 1/2: the back splat's weight o2 G (1 - o1 G) peaks on
    the ring G = 1 / (2 o1) at o2 / (4 o1), not at the centre. Wide splats make
    the pixel grid sample G finely near the ring: the maximum over pixels lies
    just below the continuous one and never above it."""
    o1, o2 = 0.875, 0.75
    sc = scenes.custom_scene(96, 96, means2d=[[48.5, 48.5]] * 2, sigmas=[[20.0, 20.0]] * 2,
                             thetas=[0.0, 0.0], opacities=[o1, o2], colors=[[1, 0, 0], [0, 1, 0]],
                             depths=[1.0, 2.0])
    mw, _ = _max_weight(sc, _tiled(sc, backward=False))
    peak = o2 / (4 * o1)
    assert mw[1] <= peak + 1e-12
    assert mw[1] >= peak - 2e-4
    assert mw[1] > o2 * (1 - o1) + 0.05   # well above the value at the centre


def test_max_weight_invariants():
    for sc in [scenes.make_scene("tiny", 2), scenes.make_scene("early", 1, n=600)]:
        out = _tiled(sc)
        mw, _ = _max_weight(sc, out)
        aw = out["accum_weight"]
        assert np.all(mw >= 0) and np.all(mw <= 0.99)
        assert np.all(mw <= aw + 1e-12)                 # the largest term of a sum of positives
        np.testing.assert_array_equal(mw > 0, aw > 0)   # composited somewhere, or nowhere


# ------------------------------------------- ambiguity flags, max-weight marks
# The oracle flags a pixel when one of its decisions (skip at 1/255, clamp at
# 0.99, stop at 1e-4) lies within its bound on the error of a float32
# evaluation, and marks a splat's max weight uncertain when a flagged pixel
# could move it. Pinned here against an independent walk of the plain
# definition carried out twice, in float64 and in float32 (numpy): every pixel
# where the two walks decide differently must be flagged, every splat whose
# float32 maximum moves must be marked, and on scenes built to sit on the
# thresholds every constructed pixel must be flagged. The flagged fractions
# are bounded near their measured values, so that a band grown far wider than
# the float32 error fails too.

F32 = np.float32


def _dual_walk(sc, ids, rng_, tiles):
    """Each pixel of ``tiles`` walked twice, each walk to its end, by the
    plain definition: in float64 and in float32 (means, conic, opacity and
    colour as stored; sigma, exp, the clamp, the thresholds, T and the colour
    sums all in the walk's precision). ``differs`` marks the pixels whose two
    walks decide differently somewhere (skip, stop or clamp)."""
    GX, _ = oracle.grid(sc.width, sc.height)
    tiles = np.asarray(tiles)
    ly, lx = np.mgrid[0:16, 0:16]
    xs = ((tiles % GX)[:, None] * 16 + lx.ravel()[None, :]).ravel()
    ys = ((tiles // GX)[:, None] * 16 + ly.ravel()[None, :]).ravel()
    tl = np.repeat(tiles, 256)
    keep = (xs < sc.width) & (ys < sc.height)
    xs, ys, tl = xs[keep], ys[keep], tl[keep]
    start = rng_[tl, 0].astype(np.int64)
    L = (rng_[tl, 1] - rng_[tl, 0]).astype(np.int64)
    P = len(xs)
    bg = np.zeros(3) if sc.background is None else np.asarray(sc.background, dtype=np.float64)
    walks = {}
    for dt in (np.float64, F32):
        m, q, o = sc.means2d.astype(F32).astype(dt), sc.conics.astype(F32).astype(dt), \
            sc.opacities.astype(F32).astype(dt)
        col = sc.colors.astype(F32).astype(dt)
        px, py = (xs + 0.5).astype(dt), (ys + 0.5).astype(dt)
        w = {"T": np.ones(P, dt), "C": np.zeros((P, 3), dt), "nc": np.zeros(P, np.int64),
             "done": np.zeros(P, bool), "mw": np.zeros(sc.n, dt), "dec": {}}
        for j in range(int(L.max(initial=0))):
            act = np.nonzero((j < L) & ~w["done"])[0]
            if act.size == 0:
                break
            i = ids[start[act] + j]
            dx, dy = px[act] - m[i, 0], py[act] - m[i, 1]
            ah = o[i] * np.exp(dt(-0.5) * (q[i, 0] * dx * dx + q[i, 2] * dy * dy) - q[i, 1] * dx * dy)
            a = np.minimum(dt(0.99), ah)
            use = a >= dt(1.0 / 255.0)
            t = w["T"][act] * (dt(1.0) - a)
            stop = use & (t < dt(1e-4))
            comp = use & ~stop
            # decision code per (pixel, step): 0 skip, 1 stop, 2 composite, 3 composite clamped
            w["dec"][j] = (act, np.where(~use, 0, np.where(stop, 1, np.where(ah < dt(0.99), 2, 3))))
            ac = act[comp]
            wt = a[comp] * w["T"][ac]
            np.maximum.at(w["mw"], i[comp], wt)
            w["C"][ac] += col[i[comp]] * wt[:, None]
            w["T"][ac] = t[comp]
            w["nc"][ac] = j + 1
            w["done"][act[stop]] = True
        walks[dt] = w
    w64, w32 = walks[np.float64], walks[F32]
    differs = np.zeros(P, bool)
    for j, (act64, d64) in w64["dec"].items():
        act32, d32 = w32["dec"].get(j, (np.zeros(0, np.int64), np.zeros(0, np.int64)))
        a = np.full(P, -1)
        a[act64] = d64
        b = np.full(P, -1)
        b[act32] = d32
        differs |= a != b
    img = {k: w["C"].astype(np.float64) + w["T"].astype(np.float64)[:, None] * bg[None, :]
           for k, w in (("64", w64), ("32", w32))}
    return {"x": xs, "y": ys, "differs": differs, "T64": w64["T"], "T32": w32["T"].astype(np.float64),
            "nc64": w64["nc"], "nc32": w32["nc"], "img64": img["64"], "img32": img["32"],
            "mw64": w64["mw"], "mw32": w32["mw"].astype(np.float64)}


def _threshold_scene(seed, W=256, H=256):
    """Isolated splats (one 16x16 cell each, nothing else reaching the cell's
    centre pixel) built so that a pixel sits within float32 rounding of a
    threshold:
      skip   alpha = 1/255 on the ring at 2-4 px from an isotropic mean;
      clamp  opacity G = 0.99 a quarter pixel from the mean (sigma 2, so
             that a = 1/4 and sigma are exact);
      stop   three splats centred on the pixel (G = 1 there, alpha = o),
             then one whose alpha brings T (1 - alpha) within 1.5e-7
             (relative) of 1e-4;
      maxw   a small splat whose only candidate pixels sit on the skip
             threshold, so that its max weight is 1/255 or 0.
    Returns the scene, each splat's kind and its cell's centre pixel."""
    rng = np.random.default_rng(seed)
    cells = [(cx, cy) for cy in range(8, H - 8, 16) for cx in range(8, W - 8, 16)]
    rng.shuffle(cells)
    means, sig, op, kinds, at = [], [], [], [], []

    def put(m, s, o, kind, cell):
        means.append(m)
        sig.append([s, s])
        op.append(o)
        kinds.append(kind)
        at.append(cell)

    cell = iter(cells)
    for _ in range(50):
        cx, cy = next(cell)
        s, r = float(rng.uniform(1.0, 2.5)), float(rng.integers(2, 5))
        a = float(F32(1.0 / (s * s)))                  # the stored conic (b = 0)
        put([cx + 0.5 + r, cy + 0.5], s, F32(math.exp(0.5 * a * r * r) / 255.0), "skip", (cx, cy))
    for _ in range(30):
        cx, cy = next(cell)
        put([cx + 0.75, cy + 0.5], 2.0, F32(0.99 * math.exp(0.5 * 0.25 * 0.0625)), "clamp", (cx, cy))
    for _ in range(30):
        cx, cy = next(cell)
        v = int(rng.integers(51, 461)) / 1024.0   # on a 1/1024 grid: cy + 0.5 + v is exact in float32
        put([cx + 1.0, cy + 0.5 + v], 0.5, F32(math.exp(2.0 * (0.25 + v * v)) / 255.0), "maxw", (cx, cy))
    found = 0
    while found < 30:
        o3 = rng.uniform(0.85, 0.95, 3).astype(F32)
        T3 = float(np.prod(1.0 - o3.astype(np.float64)))
        o4 = F32(1.0 - 1e-4 / T3)
        if abs(T3 * (1.0 - float(o4)) / 1e-4 - 1.0) > 1.5e-7:
            continue
        cx, cy = next(cell)
        found += 1
        for o in [*o3, o4]:
            put([cx + 0.5, cy + 0.5], 0.8, o, "stop", (cx, cy))
    n = len(means)
    sc = scenes.custom_scene(W, H, means2d=means, sigmas=sig, thetas=np.zeros(n), opacities=op,
                             colors=rng.uniform(0, 1, (n, 3)), depths=np.arange(1, n + 1, dtype=float),
                             seed=seed)
    return sc, np.array(kinds), at


@pytest.mark.parametrize("seed", [0, 1])
def test_threshold_pixels_are_flagged(seed):
    sc, kinds, at = _threshold_scene(seed)
    out = _tiled(sc, backward=False)
    amb = out["ambiguous"]
    for kind in ("skip", "clamp", "stop"):
        cells = sorted({c for k, c in zip(kinds, at) if k == kind})
        missed = [c for c in cells if not amb[c[1], c[0]]]
        assert not missed, (kind, missed)
    _, unc = _max_weight(sc, out)
    assert unc[kinds == "maxw"].all()
    # the flags stay where the thresholds are: cells of other kinds' centre
    # pixels aside, nearly every pixel is clear
    assert amb.mean() < 0.01


def _rewalk_check(sc, tiles=None, need_flips=False):
    out = _tiled(sc, backward=False)
    GX, GY = oracle.grid(sc.width, sc.height)
    tiles = np.arange(GX * GY) if tiles is None else tiles
    r = _dual_walk(sc, out["sorted_ids"], out["tile_ranges"], tiles)
    at = (r["y"], r["x"])
    amb = out["ambiguous"][at]
    # the float64 re-walk is the oracle's walk
    np.testing.assert_array_equal(r["nc64"], out["n_contrib"][at])
    np.testing.assert_allclose(r["T64"], out["final_T"][at], atol=1e-12, rtol=0)
    np.testing.assert_allclose(r["img64"], out["image"][at], atol=1e-12, rtol=0)
    # float32 decides differently only on flagged pixels, and agrees with the
    # float64 walk to the forward's tolerance where it decides the same
    assert not (r["differs"] & ~amb).any(), "a float32 decision flip on an unflagged pixel"
    ok = ~r["differs"]
    np.testing.assert_array_equal(r["nc32"][ok], r["nc64"][ok])
    assert np.abs(r["T32"] - r["T64"])[ok].max(initial=0.0) <= 1e-5
    assert np.abs(r["img32"] - r["img64"])[ok].max(initial=0.0) <= 1e-5
    # everywhere, the float32 result is one of the pixel's admissible outcomes
    # (an unflagged pixel has one: the forward's)
    outc = oracle.pixel_outcomes(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background, sc.width,
                                 sc.height, out["tile_ranges"], out["sorted_ids"], r["x"], r["y"])
    assert np.all(outc[3][~amb] == 1)
    np.testing.assert_allclose(outc[0][~amb, 0], out["image"][at][~amb], atol=1e-12, rtol=0)
    assert np.all(outc[3][amb] >= 1)
    match = oracle.matches_an_outcome(r["img32"], r["T32"], r["nc32"], outc, 1e-5, 1e-5)
    assert match.all(), np.nonzero(~match)[0][:10]
    # max weight: every splat's float32 maximum lies in the oracle's bounds,
    # and moves by more than 1e-5 only for splats the oracle marks uncertain
    mw, unc, lo, hi = oracle.max_weight(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background,
                                        sc.width, sc.height, out["tile_ranges"], out["sorted_ids"], tiles=tiles,
                                        bounds=True)
    np.testing.assert_allclose(r["mw64"], mw, atol=1e-12, rtol=0)
    moved = np.abs(r["mw32"] - mw) > 1e-5
    assert not (moved & ~unc).any(), np.nonzero(moved & ~unc)[0][:10]
    assert np.all(r["mw32"] >= lo - 1e-5) and np.all(r["mw32"] <= hi + 1e-5)
    assert np.all(lo <= mw) and np.all(mw <= hi)
    if need_flips:  # the constructed scenes really make float32 decide differently
        assert r["differs"].sum() >= 10 and moved.sum() >= 1, (int(r["differs"].sum()), int(moved.sum()))
        assert (outc[3][amb] >= 2).mean() > 0.5
    return r, amb


@pytest.mark.parametrize("seed", [0, 1])
def test_float32_rewalk_flips_are_flagged_on_threshold_scenes(seed):
    _rewalk_check(_threshold_scene(seed)[0], need_flips=True)


@pytest.mark.parametrize("name", ["tiny", "early"])
def test_float32_rewalk_flips_are_flagged(name):
    _rewalk_check(scenes.make_scene(name, 0))


def test_decisions_clear_of_thresholds_are_not_flagged():
    """A scene whose every decision sits more than 1e-3 (relative) from its
    threshold has no flagged pixel and no uncertain max weight."""
    sc = _first_clear(_fd_scene, range(0, 10))
    out = _tiled(sc, backward=False)
    assert not out["ambiguous"].any()
    assert not _max_weight(sc, out)[1].any()


# measured flagged fractions: early 1.37e-4, mid 1.97e-4 (seed 0); bounds 2x
@pytest.mark.parametrize("name,bound", [("early", 2.8e-4), ("mid", 4e-4)])
def test_flagged_fraction_near_measured(name, bound):
    sc = scenes.make_scene(name, 0)
    frac = _tiled(sc, backward=False)["ambiguous"].mean()
    assert 0 < frac <= bound, frac
