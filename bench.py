"""Benchmark of gs_rasterize_bwd on one MI355X.

One step = one gs_rasterize_bwd call over the whole scene (binning and the
forward that produce its inputs run once, before the timed region; their
times are reported alongside as raster_bench-style stage lines). Default
workload: the fixed raster_bench load of the Spirula Studio page (section
亲手验证): 2,000,000 splats at 1237x822, 20 timed iterations.

Prints one JSON line with the metric (pairs/s; pairs = sum over pixels of
n_contrib, the list entries the backward must revisit), ms/call, a roofline
object for the call's dominant kernel, the reverse walk (algorithmic work /
its mean launch time, from HIP events the library records around it on the
call's stream, against the bound that dominates, with every term listed) and
a CPU baseline (the float64 oracle on a bounded sample of the same scene, on
the host's cores).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Algorithmic floating-point work per pair, counted from the formulas as
# written (an FMA counts 2, a division, exp or compare-free min counts 1):
#   per walked (pixel, entry) pair:    alpha evaluation                 13
#   per composited pair, in addition:  T recovery, dL/dalpha, colour
#                                      behind, 9 gradient terms + sums  45
#   accumulated weight (optional):     +1 per composited pair
FLOP_WALK = 13
FLOP_CONTRIB = 45
# fp32 VALU peak without packed FP32 forms (the library is compiled without them):
# 256 CUs x 4 SIMD x 16 lanes x 2 flops (FMA) x 2.4 GHz.
PEAK_ALU_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0

PROFILE_PMC = os.path.join(ROOT, "profiles", "bwd_bench_pmc.json")
KERNEL_SOURCES = ["differentiable_tile_rasterization_amd/csrc/gs_raster.hip",
                  "differentiable_tile_rasterization_amd/csrc/gs_common.hpp"]


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and whitespace are dropped,
    so that editing a comment does not retire the traffic counters."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_probe():
    path = os.path.join(ROOT, "differentiable_tile_rasterization_amd", "libgsprobe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build with python -m differentiable_tile_rasterization_amd.build")
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_longlong
    lib.gsp_walk_stats.argtypes = [i32, P, P, P, i32, i32, P, P, P, P, P, P]
    lib.gsp_copy.argtypes = [P, P, i64, ctypes.c_int, P]
    lib.gsp_atomic_replay.argtypes = [P, P, i64, P, P, P, P, P, P]
    lib.gsp_valu_peak.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
    lib.gsp_exp_peak.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
    for f in ["gsp_walk_stats", "gsp_copy", "gsp_atomic_replay", "gsp_valu_peak", "gsp_exp_peak"]:
        getattr(lib, f).restype = ctypes.c_int
    return lib


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="bench")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=float, default=1.0, help="fraction of tiles the oracle baseline runs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU "
              "path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import differentiable_tile_rasterization_amd as gsr
    import scenes

    def log(*a):
        print("[bench]", *a, file=sys.stderr, flush=True)

    sc = scenes.make_scene(args.config, args.seed)
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    m, q, c, o, bg = t(sc.means2d), t(sc.conics), t(sc.colors), t(sc.opacities), t(sc.background)
    r, d, g = t(sc.radii), t(sc.depths), t(sc.dL_dimage)
    aw = sc.accum_weight
    log(f"workload {args.config}: {sc.width}x{sc.height}, {sc.n} splats, accum_weight={aw}")
    bins = gsr.gs_bin_tiles(m, r, d, sc.width, sc.height)
    img, T, nc = gsr.gs_rasterize_fwd(m, q, c, o, bg, sc.width, sc.height, bins.tile_ranges, bins.sorted_ids)
    ws = torch.empty(gsr.gs_rasterize_bwd_workspace_size(sc.n, bins.n_isect, sc.width, sc.height) + 256, dtype=torch.uint8,
                     device=dev)
    out = gsr.gs_rasterize_bwd(m, q, c, o, r, bg, sc.width, sc.height, bins, T, nc, g, accum_weight=aw,
                               workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)

    def bwd():
        gsr.gs_rasterize_bwd(m, q, c, o, r, bg, sc.width, sc.height, bins, T, nc, g, accum_weight=aw, out=out,
                             workspace=ws)

    def fwd():
        gsr.gs_rasterize_fwd(m, q, c, o, bg, sc.width, sc.height, bins.tile_ranges, bins.sorted_ids)

    def fwd_max_weight():
        gsr.gs_rasterize_fwd(m, q, c, o, bg, sc.width, sc.height, bins.tile_ranges, bins.sorted_ids,
                             max_weight=True)

    def per_call(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    # The counts and the measured ceilings run before the timed region: their
    # kernels also bring the GPU's clocks up to their sustained level (after
    # only a few calls of a cold GPU the walk runs about 8% slower).
    # ---- exact algorithmic counts
    probe = load_probe()
    cnt = torch.zeros(12, dtype=torch.int64, device=dev)
    flags = torch.zeros(max(bins.n_isect, 1), dtype=torch.uint8, device=dev)
    rc = probe.gsp_walk_stats(sc.n, m.data_ptr(), q.data_ptr(), o.data_ptr(), sc.width, sc.height,
                              bins.tile_ranges.data_ptr(), bins.sorted_ids.data_ptr(), nc.data_ptr(),
                              cnt.data_ptr(), flags.data_ptr(), st)
    assert rc == 0
    torch.cuda.synchronize()
    cnt = [int(v) for v in cnt.cpu().tolist()]
    p_walk, p_contrib, entries, groups_tile, groups_wave, ew_walk, ew_kept = cnt[:7]
    groups_half, groups_blk, iters_half, iters_blk = cnt[7:11]
    p_walk_check = int(nc.to(torch.int64).sum().item())
    assert p_walk == p_walk_check, (p_walk, p_walk_check)

    # ---- measured ceilings
    def gpu_time(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    n4 = 64 * 1024 * 1024  # 1 GiB per buffer
    src = torch.empty(n4 * 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    t_copy = gpu_time(lambda: probe.gsp_copy(src.data_ptr(), dst.data_ptr(), n4, 256 * 8 * 4, st))
    hbm_gbs = 2 * n4 * 16 / t_copy / 1e9
    del src, dst
    scratch = {k: torch.zeros_like(v) for k, v in out.items()}
    t_atomic = gpu_time(lambda: probe.gsp_atomic_replay(
        flags.data_ptr(), bins.sorted_ids.data_ptr(), bins.n_isect, scratch["dL_dmeans2d"].data_ptr(),
        scratch["dL_dconics"].data_ptr(), scratch["dL_dcolors"].data_ptr(), scratch["dL_dopacities"].data_ptr(),
        scratch["accum_weight"].data_ptr() if aw else None, st))
    nfields = 10 if aw else 9
    n_atomics = groups_tile * nfields
    atomic_rate = n_atomics / t_atomic
    pk = torch.zeros(4096, dtype=torch.float32, device=dev)
    iters = 512
    t_valu = gpu_time(lambda: probe.gsp_valu_peak(pk.data_ptr(), 256 * 32, iters, st))
    valu_tflops = 256 * 32 * 256 * iters * 8 * 2 / t_valu / 1e12
    t_exp = gpu_time(lambda: probe.gsp_exp_peak(pk.data_ptr(), 256 * 32, iters, st))
    exp_rate = 256 * 32 * 256 * iters * 4 / t_exp

    # ---- timed region: exactly K backward calls, synchronised on both sides
    for _ in range(args.warmup):
        bwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        bwd()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_region = e0.elapsed_time(e1) / args.steps
    log(f"timed region: {args.steps} calls, {ms_region:.4f} ms/call (events), wall {wall * 1e3 / args.steps:.4f}")
    t_calls = per_call(bwd, args.steps, 1)
    # per-stage times of the same calls, from HIP events the library records
    # on this stream at its stage boundaries (gs_rasterize_bwd_timed)
    stage_ms = {"setup": [], "walk": [], "gather": []}
    for _ in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in evs:
            e.record(stream)
        gsr.gs_rasterize_bwd(m, q, c, o, r, bg, sc.width, sc.height, bins, T, nc, g, accum_weight=aw, out=out,
                             workspace=ws, events=evs)
        torch.cuda.synchronize()
        for k, (a, b) in zip(stage_ms, [(0, 1), (1, 2), (2, 3)]):
            stage_ms[k].append(evs[a].elapsed_time(evs[b]))
    stage_mean = {k: float(np.mean(v)) for k, v in stage_ms.items()}
    log("stages (ms, mean of %d calls): " % args.steps + ", ".join(f"{k} {v:.4f}" for k, v in stage_mean.items()))
    t_fwd = per_call(fwd, 10, 2)
    t_mw = per_call(fwd_max_weight, 10, 2)
    t0 = time.perf_counter()
    for _ in range(3):
        gsr.gs_bin_tiles(m, r, d, sc.width, sc.height, capacity=bins.n_isect)
    torch.cuda.synchronize()
    t_bin = (time.perf_counter() - t0) / 3 * 1e3

    # ---- roofline of the reverse-walk kernel (the call's dominant kernel)
    ms = float(ms_region)
    t_s = ms * 1e-3
    t_walk = stage_mean["walk"] * 1e-3
    flops = FLOP_WALK * p_walk + (FLOP_CONTRIB + (1 if aw else 0)) * p_contrib
    hbm_bytes = sc.n * 36 + entries * 4 + len(bins.tile_ranges) * 8 + sc.width * sc.height * 20 \
        + sc.n * 4 * nfields
    terms = {
        "alu_ms": flops / (PEAK_ALU_TFLOPS * 1e12) * 1e3,
        "hbm_ms": hbm_bytes / (PEAK_HBM_GBS * 1e9) * 1e3,
    }
    bound = max(terms, key=terms.get).split("_")[0]
    traffic = None
    if os.path.exists(PROFILE_PMC):
        with open(PROFILE_PMC) as f:
            pmc = json.load(f)
        if pmc.get("source_hash") == kernel_source_hash() and pmc.get("config") == args.config:
            traffic = pmc.get("hbm_bytes_per_launch")
    if bound == "alu":
        roof = {"bound": "alu", "achieved": flops / t_walk / 1e12, "peak": PEAK_ALU_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": hbm_bytes / t_walk / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    # the library's choice of reverse walk (more than 16 tiles per splat: stored partials)
    roof["kernel"] = ("bwd_store_kernel (reverse walk, stored partials)" if bins.n_isect > 16 * sc.n
                      else "bwd_kernel (reverse walk, LDS adds)")
    roof["kernel_ms"] = stage_mean["walk"]
    roof["terms_ms"] = terms
    roof["call_frac"] = terms[bound + "_ms"] / ms  # the same work against the whole call's time
    roof["stages_ms"] = stage_mean
    roof["algorithmic"] = {"flops": flops, "hbm_bytes": hbm_bytes, "atomics": n_atomics,
                           "flop_per_walked_pair": FLOP_WALK, "flop_per_composited_pair": FLOP_CONTRIB}
    # the flush as 9-10 scattered float atomics per (splat, tile) group, timed
    # alone: what an atomic-accumulating design would pay (this one stores)
    roof["atomic_flush_replay_ms"] = t_atomic * 1e3
    roof["ceilings_measured"] = {"hbm_copy_GBs": hbm_gbs, "atomic_replay_per_s": atomic_rate,
                                 "valu_fma_TFLOPs": valu_tflops, "exp_per_s": exp_rate}

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        GX, GY = gsr.tile_grid(sc.width, sc.height)
        ntiles = GX * GY
        k = max(1, int(round(args.cpu_sample * ntiles)))
        tiles = np.sort(np.random.default_rng(0).choice(ntiles, k, replace=False)).astype(np.int32)
        ids_h = bins.sorted_ids.cpu().numpy()
        rng_h = bins.tile_ranges.cpu().numpy()
        nc_h = nc.cpu().numpy()
        ys, xs = np.mgrid[0:sc.height, 0:sc.width]
        sel = np.isin((ys // 16) * GX + xs // 16, tiles)
        pw_sample = int(nc_h[sel].astype(np.int64).sum())
        oracle.threads()
        c0 = time.perf_counter()
        oracle.rasterize_bwd(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background, sc.width, sc.height,
                             rng_h, ids_h, sc.dL_dimage, tiles=tiles)
        c_s = time.perf_counter() - c0
        cpu = {"value": pw_sample / c_s, "unit": "pairs/s", "cores": oracle.threads(), "kind": "oracle",
               "seconds": c_s,
               "sample": f"float64 oracle rasterize_bwd over {k} of {ntiles} tiles (random, seed 0) of the same "
                         f"scene, {pw_sample} walked pairs; binning excluded"}
        log(f"cpu oracle: {c_s:.2f} s on {cpu['cores']} threads, {cpu['value']:.3e} pairs/s")

    value = p_walk / t_s
    rec = {
        "metric": "rasterize_bwd ms/call + (splat,pixel) pairs/s", "value": value, "unit": "pairs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.config}: {sc.width}x{sc.height} RGB, {sc.n} splats"
                               + (", accum weight" if aw else ""), "seed": args.seed,
                   "width": sc.width, "height": sc.height, "splats": sc.n},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stages_ms": {"tile_isect": t_bin, "raster_fwd": float(np.median(t_fwd)),
                      "raster_fwd_max_wt": float(np.median(t_mw)), "raster_bwd": ms,
                      "raster_bwd_median": float(np.median(t_calls)), "raster_bwd_min": float(np.min(t_calls))},
        "counts": {"p_walk": p_walk, "p_composited": p_contrib, "walked_entries": entries,
                   "splat_tile_groups": groups_tile, "splat_quadrant_groups": groups_wave,
                   "entry_quadrant_walk": ew_walk, "entry_quadrant_kept": ew_kept, "n_isect": bins.n_isect,
                   "splat_half_groups": groups_half, "splat_block4_groups": groups_blk,
                   "lockstep_half_iters": iters_half, "lockstep_block4_iters": iters_blk},
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
