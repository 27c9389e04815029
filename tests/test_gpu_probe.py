"""GPU checks of the measurement library: the wave fold reduction maps each
field to the row-leader lane the backward's flush expects, and the walk
counters agree with the oracle's own counts."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import scenes
import differentiable_tile_rasterization_amd as gsr

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(gsr.__file__), "libgsprobe.so")


def _probe():
    lib = ctypes.CDLL(PROBE)
    lib.gsp_fold_selftest.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.gsp_walk_stats.argtypes = [ctypes.c_int32] + [ctypes.c_void_p] * 3 + [ctypes.c_int32] * 2 + \
        [ctypes.c_void_p] * 6
    return lib


def test_fold_lane_mapping():
    lib = _probe()
    rng = np.random.default_rng(0)
    vals = rng.integers(-1000, 1000, (10, 64)).astype(np.float32)   # exact sums in float32
    inp = torch.from_numpy(vals.ravel()).cuda()
    out = torch.zeros(12, dtype=torch.float32, device="cuda")
    assert lib.gsp_fold_selftest(ctypes.c_void_p(inp.data_ptr()), ctypes.c_void_p(out.data_ptr()), None) == 0
    got = out.cpu().numpy().reshape(4, 3)
    s = vals.sum(axis=1)
    # slot (row, reg) -> field, as read by the backward's flush
    expect = np.array([[s[0], s[4], s[8]], [s[2], s[6], s[8]], [s[1], s[5], s[9]], [s[3], s[7], s[9]]])
    np.testing.assert_array_equal(got, expect)


def test_walk_counts_match_oracle():
    sc = scenes.make_scene("tiny", 0)
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    m, q, c, o = t(sc.means2d), t(sc.conics), t(sc.colors), t(sc.opacities)
    bins = gsr.gs_bin_tiles(m, q, o, t(sc.radii), t(sc.depths), sc.width, sc.height)
    _, _, nc = gsr.gs_rasterize_fwd(m, q, c, o, t(sc.background), sc.width, sc.height, bins.tile_ranges,
                                    bins.sorted_ids)
    cnt = torch.zeros(12, dtype=torch.int64, device=dev)
    lib = _probe()
    P = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731
    assert lib.gsp_walk_stats(sc.n, P(m), P(q), P(o), sc.width, sc.height, P(bins.tile_ranges),
                              P(bins.sorted_ids), P(nc), P(cnt), None, None) == 0
    cnt = cnt.cpu().numpy()
    assert cnt[0] == int(nc.sum().item())
    # composited pairs = sum of alpha*T weights' support: count them with the oracle
    ids_o, rng_o = oracle.bin_tiles(sc.means2d, sc.conics, sc.opacities, sc.radii, sc.depths, sc.width, sc.height)
    ys, xs = np.mgrid[0:sc.height, 0:sc.width]
    img, T, nstep = oracle.composite_bruteforce(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.depths,
                                                sc.radii, sc.background, sc.width, sc.height)
    assert abs(int(cnt[1]) - int(nstep.sum())) <= 2
    assert cnt[6] <= cnt[5]          # culling never keeps more than it walks
