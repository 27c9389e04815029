"""The benchmark's pair count (bench.py's value: the sum over pixels of
n_contrib under the tile-rectangle lists) against the oracle's forward run on
the rectangle lists themselves. CPU only: torch on the host and the oracle."""
import numpy as np
import pytest
import torch

import bench
import oracle
import scenes


def _rect_lists(sc):
    """Every (splat, tile) pair of the splats' tile rectangles, listed in
    (tile, depth bits, splat id) order: the lists before the culling."""
    GX, GY = oracle.grid(sc.width, sc.height)
    ids, tx, ty, _ = oracle.kept_pairs(sc.means2d, sc.conics, sc.opacities, sc.radii, sc.depths, sc.width,
                                       sc.height)
    tile = ty * GX + tx
    dbits = sc.depths.view(np.uint32)
    perm = np.lexsort((ids, dbits[ids], tile))
    counts = np.bincount(tile, minlength=GX * GY)
    ends = np.cumsum(counts)
    rng = np.stack([ends - counts, ends], 1).astype(np.int32)
    rng[counts == 0] = 0
    return ids[perm].astype(np.int32), rng


@pytest.mark.parametrize("name,seed", [("tiny", 0), ("tiny", 2), ("early", 1)])
def test_rect_pair_count_matches_rectangle_lists(name, seed):
    sc = scenes.make_scene(name, seed)
    ids_c, rng_c = oracle.bin_tiles(sc.means2d, sc.conics, sc.opacities, sc.radii, sc.depths, sc.width, sc.height)
    ids_r, rng_r = _rect_lists(sc)
    assert len(ids_r) > len(ids_c)   # the culling drops pairs
    fc = oracle.rasterize_fwd(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background, sc.width, sc.height,
                              rng_c, ids_c)
    fr = oracle.rasterize_fwd(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background, sc.width, sc.height,
                              rng_r, ids_r)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    nrect = bench.rect_walk_pairs(torch, t(sc.means2d), t(sc.radii), t(sc.depths), sc.width, sc.height,
                                  t(fc["n_contrib"]), t(ids_c), t(rng_c)).numpy()
    np.testing.assert_array_equal(nrect, fr["n_contrib"])
    assert nrect.sum() > fc["n_contrib"].astype(np.int64).sum()
