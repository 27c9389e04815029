"""Benchmark of gs_rasterize_bwd on one MI355X (first cut: timing only)."""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="bench")
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import differentiable_tile_rasterization_amd as gsr
    import scenes

    sc = scenes.make_scene(args.config, args.seed)
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    m, q, c, o, bg = t(sc.means2d), t(sc.conics), t(sc.colors), t(sc.opacities), t(sc.background)
    r, d, g = t(sc.radii), t(sc.depths), t(sc.dL_dimage)
    bins = gsr.gs_bin_tiles(m, r, d, sc.width, sc.height)
    img, T, nc = gsr.gs_rasterize_fwd(m, q, c, o, bg, sc.width, sc.height, bins.tile_ranges, bins.sorted_ids)
    out = gsr.gs_rasterize_bwd(m, q, c, o, bg, sc.width, sc.height, bins.tile_ranges, bins.sorted_ids, T, nc, g,
                               accum_weight=sc.accum_weight)
    torch.cuda.synchronize()

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    bwd = lambda: gsr.gs_rasterize_bwd(m, q, c, o, bg, sc.width, sc.height, bins.tile_ranges,  # noqa: E731
                                       bins.sorted_ids, T, nc, g, accum_weight=sc.accum_weight, out=out)
    fwd = lambda: gsr.gs_rasterize_fwd(m, q, c, o, bg, sc.width, sc.height, bins.tile_ranges,  # noqa: E731
                                       bins.sorted_ids)
    t_bwd = timed(bwd, args.steps, args.warmup)
    t_fwd = timed(fwd, 5, 1)
    t0 = time.perf_counter()
    for _ in range(3):
        gsr.gs_bin_tiles(m, r, d, sc.width, sc.height, capacity=bins.n_isect)
    torch.cuda.synchronize()
    t_bin = (time.perf_counter() - t0) / 3 * 1e3
    p_walk = int(nc.to(torch.int64).sum().item())
    ms = float(np.median(t_bwd))
    rec = {"metric": "rasterize_bwd ms/call + (splat,pixel) pairs/s", "value": p_walk / (ms * 1e-3),
           "unit": "pairs/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": f"{args.config}: {sc.width}x{sc.height}, {sc.n} splats", "seed": args.seed},
           "stages_ms": {"tile_isect": t_bin, "raster_fwd": float(np.median(t_fwd)), "raster_bwd": ms,
                         "raster_bwd_min": float(np.min(t_bwd))},
           "p_walk": p_walk, "n_isect": bins.n_isect}
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
