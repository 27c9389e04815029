"""Pins for the oracle's depth terms (distortion and median depth), against
things other than the oracle's own running sums.

* hand-derived cases (tests/golden/depth_closed_forms.json);
* a brute force with no tiles that forms the distortion as the full double
  sum over splat pairs and the median from the recorded transmittances;
* the identity D = A C - B^2 of the totals, and A = 1 - final_T;
* central finite differences of L = sum gD D + gM median in every input the
  terms depend on (mean, conic, opacity through alpha; depth directly);
* invariances: a common depth shift leaves D and its gradients unchanged,
  scaling depths by s scales D by s^2; the depth gradients of the
  distortion sum to zero.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import scenes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "depth_closed_forms.json")


def _scene_from_case(case):
    sp = case["splats"]
    return scenes.custom_scene(
        case["width"], case["height"],
        means2d=[s["mean"] for s in sp], sigmas=[s["sigma"] for s in sp],
        thetas=[s.get("theta", 0.0) for s in sp], opacities=[s["opacity"] for s in sp],
        colors=[s["color"] for s in sp], depths=[s["depth"] for s in sp],
        background=case.get("background"))


def _fwd(sc, ids, rng_, depths=None, means=None, conics=None, opac=None):
    return oracle.rasterize_fwd_depth(sc.means2d if means is None else means,
                                      sc.conics if conics is None else conics, sc.colors,
                                      sc.opacities if opac is None else opac, sc.background,
                                      sc.width, sc.height, rng_, ids, sc.depths if depths is None else depths)


def _bwd(sc, ids, rng_, gd, gm, depths=None):
    return oracle.rasterize_bwd_depth(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background,
                                      sc.width, sc.height, rng_, ids, sc.depths if depths is None else depths,
                                      gd, gm)


def _bins(sc):
    return oracle.bin_tiles(sc.means2d, sc.conics, sc.opacities, sc.radii, sc.depths, sc.width, sc.height)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_depth_closed_forms(case):
    sc = _scene_from_case(case)
    ids, rng_ = _bins(sc)
    f = _fwd(sc, ids, rng_)
    x, y = case["at"]
    tol = case["tol"]
    assert abs(f["distortion"][y, x] - case["distortion"]) <= tol
    assert abs(f["median_depth"][y, x] - case["median_depth"]) <= tol
    assert f["median_pos"][y, x] == case["median_pos"]
    assert not f["median_ambiguous"][y, x]
    one = np.zeros((sc.height, sc.width))
    one[y, x] = 1.0
    bd = _bwd(sc, ids, rng_, one, None)
    np.testing.assert_allclose(bd["ddepths"], case["ddepths_dist"], atol=tol, rtol=0)
    if "dopacities_dist" in case:
        np.testing.assert_allclose(bd["dopacities"], case["dopacities_dist"], atol=tol, rtol=0)
    assert not bd["dcolors"].any()
    bm = _bwd(sc, ids, rng_, None, one)
    np.testing.assert_allclose(bm["ddepths"], case["ddepths_median"], atol=0, rtol=0)
    for k in ("dmeans2d", "dconics", "dopacities"):  # the median passes no gradient through alpha
        assert not bm[k].any()


# ---------------------------------------------------------------- brute force

def _ragged(seed, W=50, H=37, n=40):
    rng = np.random.default_rng(seed)
    return scenes.custom_scene(W, H, means2d=rng.uniform(-4, [W + 4, H + 4], (n, 2)),
                               sigmas=rng.uniform(1.0, 6.0, (n, 2)), thetas=rng.uniform(0, math.pi, n),
                               opacities=rng.uniform(0.2, 0.99, n), colors=rng.uniform(0, 1, (n, 3)),
                               depths=rng.uniform(0.5, 30.0, n), seed=seed)


def _dense(seed, W=48, H=40, n=160):
    """Many near-opaque splats: most pixels stop early, and the median falls
    at varying list positions."""
    rng = np.random.default_rng(seed)
    return scenes.custom_scene(W, H, means2d=rng.uniform(0, [W, H], (n, 2)),
                               sigmas=rng.uniform(2.0, 9.0, (n, 2)), thetas=rng.uniform(0, math.pi, n),
                               opacities=rng.uniform(0.5, 0.99, n), colors=rng.uniform(0, 1, (n, 3)),
                               depths=rng.uniform(1.0, 60.0, n), seed=seed)


@pytest.mark.parametrize("maker", [
    lambda: scenes.make_scene("tiny", 0), lambda: scenes.make_scene("tiny", 1),
    lambda: _ragged(3), lambda: _ragged(4), lambda: _dense(5),
], ids=["tiny0", "tiny1", "ragged3", "ragged4", "dense"])
def test_depth_terms_equal_bruteforce(maker):
    sc = maker()
    ids, rng_ = _bins(sc)
    f = _fwd(sc, ids, rng_)
    amb = oracle.rasterize_fwd(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background,
                               sc.width, sc.height, rng_, ids)["ambiguous"]
    D, med, Wm, Tb, order = oracle.depth_terms_bruteforce(sc.means2d, sc.conics, sc.opacities, sc.depths,
                                                          sc.radii, sc.width, sc.height)
    scale = max(1.0, np.abs(D).max())
    np.testing.assert_allclose(f["distortion"], D, atol=1e-10 * scale, rtol=1e-9)
    ok = ~f["median_ambiguous"] & ~amb
    assert ok.mean() > 0.99
    np.testing.assert_array_equal(f["median_depth"][ok], med[ok])
    # the totals: A is the total weight, B and C the first two moments about the median
    z = np.asarray(sc.depths, dtype=np.float64)[order]
    u = z[None, :] - f["median_depth"].reshape(-1, 1)
    tot = f["totals"].reshape(-1, 4)
    np.testing.assert_allclose(tot[:, 0], Wm.sum(axis=1), atol=1e-12)
    np.testing.assert_allclose(tot[:, 1], (Wm * u).sum(axis=1), atol=1e-10 * scale)
    np.testing.assert_allclose(tot[:, 2], (Wm * u * u).sum(axis=1), atol=1e-10 * scale, rtol=1e-10)
    # the median is the last composited splat with T before it > 1/2
    pos = f["median_pos"]
    assert ((pos > 0) == (f["totals"][..., 0] > 0)).all()


def test_totals_identities():
    """D = A C - B^2 (half the double sum of w_i w_j (u_i - u_j)^2 over all
    pairs) and A = 1 - final_T, on every pixel."""
    for sc in [scenes.make_scene("tiny", 2), _ragged(7), _dense(8)]:
        ids, rng_ = _bins(sc)
        f = _fwd(sc, ids, rng_)
        A, B, C, D = np.moveaxis(f["totals"], -1, 0)
        scale = max(1.0, np.abs(A * C).max())
        np.testing.assert_allclose(D, A * C - B * B, atol=1e-11 * scale)
        fc = oracle.rasterize_fwd(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background,
                                  sc.width, sc.height, rng_, ids)
        np.testing.assert_allclose(A, 1.0 - fc["final_T"], atol=1e-12)
        assert (D >= -1e-12 * scale).all()


# ---------------------------------------------------------------- gradients

def _fd_scene(seed, n=6):
    rng = np.random.default_rng(700 + seed)
    return scenes.custom_scene(
        16, 16, means2d=rng.uniform(3, 13, (n, 2)), sigmas=rng.uniform(1.5, 4.0, (n, 2)),
        thetas=rng.uniform(0, math.pi, n), opacities=rng.uniform(0.3, 0.95, n),
        colors=rng.uniform(0, 1, (n, 3)), depths=rng.uniform(1.0, 10.0, n), seed=seed)


def _median_margin(sc, ids, rng_):
    """Smallest |T - 1/2| over composited entries (the median decision)."""
    _, _, Wm, Tb, _ = oracle.depth_terms_bruteforce(sc.means2d, sc.conics, sc.opacities, sc.depths,
                                                    sc.radii, sc.width, sc.height)
    sel = Wm > 0
    return np.abs(Tb[sel] - 0.5).min() if sel.any() else np.inf


def _clear_scene(seeds):
    for s in seeds:
        sc = _fd_scene(s)
        ids, rng_ = _bins(sc)
        margin = oracle.composite_bruteforce(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.depths,
                                             sc.radii, sc.background, sc.width, sc.height,
                                             return_margin=True)[3]
        if margin > 1e-3 and _median_margin(sc, ids, rng_) > 1e-3:
            return sc, ids, rng_
    raise AssertionError("no scene clear of the thresholds")


def _loss(sc, ids, rng_, gd, gm, **kw):
    f = _fwd(sc, ids, rng_, **kw)
    return float(np.sum(gd * f["distortion"]) + np.sum(gm * f["median_depth"]))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_depth_gradients_match_central_differences(seed):
    sc, ids, rng_ = _clear_scene(range(10 * seed, 10 * seed + 10))
    rng = np.random.default_rng(seed)
    gd = rng.normal(size=(sc.height, sc.width))
    gm = rng.normal(size=(sc.height, sc.width))
    an = _bwd(sc, ids, rng_, gd, gm)
    base = {"means": sc.means2d.astype(np.float64), "conics": sc.conics.astype(np.float64),
            "opac": sc.opacities.astype(np.float64), "depths": sc.depths.astype(np.float64)}
    for key, name, width in [("means", "dmeans2d", 2), ("conics", "dconics", 3), ("opac", "dopacities", 1),
                             ("depths", "ddepths", 1)]:
        a = an[name].reshape(sc.n, width)
        fd = np.zeros_like(a)
        for i in range(sc.n):
            for k in range(width):
                vals = []
                for sgn in (+1, -1):
                    p = {kk: v.copy() for kk, v in base.items()}
                    view = p[key].reshape(sc.n, width)
                    h = 1e-6 * max(1.0, abs(view[i, k]))
                    view[i, k] += sgn * h
                    vals.append(_loss(sc, ids, rng_, gd, gm, **p))
                fd[i, k] = (vals[0] - vals[1]) / (2 * h)
        scale = max(np.abs(a).max(), 1e-3)
        np.testing.assert_allclose(a, fd, atol=2e-6 * scale, rtol=1e-5, err_msg=name)


def test_depth_shift_and_scale():
    sc = scenes.make_scene("tiny", 1)
    ids, rng_ = _bins(sc)
    rng = np.random.default_rng(3)
    gd = rng.normal(size=(sc.height, sc.width))
    z = sc.depths.astype(np.float64)
    f0 = _fwd(sc, ids, rng_, depths=z)
    b0 = _bwd(sc, ids, rng_, gd, None, depths=z)
    f1 = _fwd(sc, ids, rng_, depths=z + 7.25)
    b1 = _bwd(sc, ids, rng_, gd, None, depths=z + 7.25)
    f2 = _fwd(sc, ids, rng_, depths=3.0 * z)
    b2 = _bwd(sc, ids, rng_, gd, None, depths=3.0 * z)
    s = max(1.0, np.abs(f0["distortion"]).max())
    np.testing.assert_allclose(f1["distortion"], f0["distortion"], atol=1e-9 * s)
    np.testing.assert_allclose(f2["distortion"], 9.0 * f0["distortion"], atol=1e-9 * s)
    np.testing.assert_allclose(f1["median_depth"][f0["median_pos"] > 0],
                               f0["median_depth"][f0["median_pos"] > 0] + 7.25, atol=1e-12)
    for k in ("dmeans2d", "dconics", "dopacities", "ddepths"):
        g = max(1e-12, np.abs(b0[k]).max())
        np.testing.assert_allclose(b1[k], b0[k], atol=1e-9 * g, err_msg=k)
        mult = 3.0 if k == "ddepths" else 9.0
        np.testing.assert_allclose(b2[k], mult * b0[k], atol=1e-9 * g * mult, err_msg=k)


def test_distortion_depth_gradients_sum_to_zero():
    """D depends on depth differences only, so its depth gradients sum to zero
    pixel by pixel, hence over all splats."""
    for sc in [scenes.make_scene("tiny", 0), _ragged(5)]:
        ids, rng_ = _bins(sc)
        gd = np.random.default_rng(1).normal(size=(sc.height, sc.width))
        dz = _bwd(sc, ids, rng_, gd, None)["ddepths"]
        assert abs(dz.sum()) <= 1e-10 * np.abs(dz).sum()
        assert np.abs(dz).max() > 0


def test_median_gradient_counts_pixels():
    """With dL/dmedian = 1 everywhere, each splat's depth gradient is the
    number of pixels whose median it is."""
    sc = scenes.make_scene("tiny", 2)
    ids, rng_ = _bins(sc)
    f = _fwd(sc, ids, rng_)
    dz = _bwd(sc, ids, rng_, None, np.ones((sc.height, sc.width)))["ddepths"]
    cnt = np.zeros(sc.n)
    H, W = sc.height, sc.width
    GX = (W + 15) // 16
    for y in range(H):
        for x in range(W):
            p = f["median_pos"][y, x]
            if p:
                t = (y // 16) * GX + x // 16
                cnt[ids[rng_[t, 0] + p - 1]] += 1
    np.testing.assert_array_equal(dz, cnt)
    assert cnt.sum() == (f["median_pos"] > 0).sum() > 0


def test_depth_gradients_linear_in_upstream():
    sc = scenes.make_scene("tiny", 0)
    ids, rng_ = _bins(sc)
    rng = np.random.default_rng(4)
    g1, g2, m1 = (rng.normal(size=(sc.height, sc.width)) for _ in range(3))
    a = _bwd(sc, ids, rng_, g1, m1)
    b = _bwd(sc, ids, rng_, g2, None)
    c = _bwd(sc, ids, rng_, 2 * g1 - 3 * g2, 2 * m1)
    for k in ("dmeans2d", "dconics", "dopacities", "ddepths"):
        np.testing.assert_allclose(c[k], 2 * a[k] - 3 * b[k], atol=1e-9 * max(1.0, np.abs(c[k]).max()))


def test_median_ambiguity_flag():
    """A pixel whose T before a composited splat is within the float32 band
    of 1/2 is flagged; nudging it clear of 1/2 clears the flag."""
    def sc_with(o):
        return scenes.custom_scene(16, 16, means2d=[[8.5, 8.5], [8.5, 8.5]], sigmas=[[3, 3], [3, 3]],
                                   thetas=[0, 0], opacities=[o, 0.3], colors=[[1, 1, 1]] * 2,
                                   depths=[1.0, 2.0])
    sc = sc_with(0.5)  # T before the second splat is exactly 1/2 at the centre
    ids, rng_ = _bins(sc)
    f = _fwd(sc, ids, rng_)
    assert f["median_ambiguous"][8, 8]
    sc = sc_with(0.45)
    ids, rng_ = _bins(sc)
    f = _fwd(sc, ids, rng_)
    assert not f["median_ambiguous"][8, 8]
    assert f["median_pos"][8, 8] == 2 and f["median_depth"][8, 8] == 2.0


def test_dense_scene_exercises_early_stop_and_median():
    sc = _dense(5)
    ids, rng_ = _bins(sc)
    fc = oracle.rasterize_fwd(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background,
                              sc.width, sc.height, rng_, ids)
    f = _fwd(sc, ids, rng_)
    lens = np.zeros((sc.height, sc.width), dtype=np.int64)
    GX = (sc.width + 15) // 16
    for y in range(sc.height):
        for x in range(sc.width):
            t = (y // 16) * GX + x // 16
            lens[y, x] = rng_[t, 1] - rng_[t, 0]
    assert (fc["n_contrib"] < lens).mean() > 0.5       # most pixels stop before their list ends
    assert len(np.unique(f["median_pos"])) > 10        # medians at many list positions
