"""Benchmark of gs_rasterize_bwd on one MI355X.

One step = one gs_rasterize_bwd call over the whole scene (binning and the
forward that produce its inputs run once, before the timed region; their
times are reported alongside as raster_bench-style stage lines). Default
workload: the fixed raster_bench load of the Spirula Studio page (section
亲手验证): 2,000,000 splats at 1237x822, 20 timed iterations.

Prints one JSON line with the metric (pairs/s; pairs = sum over pixels of
n_contrib under the tile-rectangle lists, i.e. the list entries a backward
must revisit when each splat is listed in every tile of its rectangle: the
scene's count, which does not depend on how tightly the binning culls; the
library's own lists skip the tiles a splat's alpha >= 1/255 ellipse cannot
reach, and their smaller sum is reported beside it), ms/call, a roofline
object for the call's dominant kernel, the reverse walk, and a CPU baseline
(the float64 oracle on the same scene, on the host's threads, plus one-thread
times of the three small workloads).

Roofline: T_roof = max(T_VALU,min, T_LDS, T_HBM), each an algorithmic count
over a ceiling measured in the same run (FMA and exp issue, LDS broadcast
reads and writes, streaming HBM copy); there is no atomic term, the path
issues no global atomics. T_LDS counts one record write per walked entry and
one wave-broadcast read per (splat, half-wave) group with a composited pixel. ``frac`` is the walk's min-model VALU rate against
the part's VALU issue rate from its unit counts; ``frac_measured_roof`` is
T_roof over the walk's time (its mean launch time from HIP events the library
records around it on the call's stream); ``call_frac`` the same over the
whole call.
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

# Algorithmic work of the reverse walk, per composited (pixel, splat) pair, in
# VALU lane-operations: the minimum model (every evaluated lane composites):
# alpha recomputation and the skip test (14), T recovery, dL/dalpha, the colour
# behind and the nine gradient terms with their sums (46); plus 2
# transcendentals (exp, reciprocal). The walk model, a diagnostic of a kernel
# that evaluates every walked pair in lockstep, adds 14 lane-ops and one
# transcendental per walked pair on top of the 46 + 1 per composited pair.
VALU_MIN_PER_PAIR = 60
TRANS_PER_PAIR = 2
VALU_WALK_PER_WALKED = 14
VALU_WALK_PER_PAIR = 46
# LDS traffic of a walk that stages its records in LDS: a 40-byte record
# written once per walked list entry, and read (wave-broadcast) once per
# (splat, 8x4 half-wave) group with a composited pixel -- the reads no
# culling can avoid. The unculled model (every entry read by each of the four
# waves) is reported beside it as a diagnostic.
LDS_RECORD_BYTES = 40
LDS_READS_PER_ENTRY = 4
# VALU issue of the part, from its unit counts: 256 CUs x 4 SIMDs, one wave64
# instruction per SIMD every 4 cycles (16 lanes per cycle), 2.4 GHz. The
# published 157.3 TFLOP/s counts packed FP32 FMAs (two lanes' worth per
# instruction slot and 2 flops each); the library is compiled without packed
# forms, so one lane-operation per lane-slot is the ceiling.
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
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


def rect_walk_pairs(torch, m, r, d, width, height, n_contrib, sorted_ids, tile_ranges):
    """Per pixel, n_contrib under the tile-rectangle lists: the number of
    splats of the pixel's tile rectangle list (every splat whose rectangle
    covers the tile, in (depth bits, id) order) up to and including the last
    one the pixel composites. The last composited splat comes from the
    culled lists the forward walked (a culled list keeps the rectangle
    list's order and drops only splats that cannot composite there). All on
    the device; int64 [height, width]."""
    dev = m.device
    f32 = torch.float32
    GX, GY = (width + 15) // 16, (height + 15) // 16
    rf = r.to(f32)
    # the binning's float32 tile rectangle
    tx0 = torch.floor((m[:, 0] - rf) * 0.0625).clamp(0, GX)
    tx1 = (torch.floor((m[:, 0] + rf) * 0.0625) + 1.0).clamp(0, GX)
    ty0 = torch.floor((m[:, 1] - rf) * 0.0625).clamp(0, GY)
    ty1 = (torch.floor((m[:, 1] + rf) * 0.0625) + 1.0).clamp(0, GY)
    live = (r > 0) & (d > 0) & torch.isfinite(m[:, 0]) & torch.isfinite(m[:, 1])
    tx0, tx1, ty0, ty1 = (v.nan_to_num(0.0).to(torch.int64) for v in (tx0, tx1, ty0, ty1))
    nx, ny = (tx1 - tx0).clamp(min=0), (ty1 - ty0).clamp(min=0)
    cnt = torch.where(live, nx * ny, torch.zeros_like(nx))
    n = m.shape[0]
    # each splat's rank in (depth bits, id) order
    order = torch.sort(d.view(torch.int32).to(torch.int64) * (1 << 32) + torch.arange(n, device=dev)).indices
    drank = torch.empty(n, dtype=torch.int64, device=dev)
    drank[order] = torch.arange(n, device=dev)
    sid = torch.repeat_interleave(torch.arange(n, device=dev), cnt)
    local = torch.arange(sid.numel(), device=dev) - torch.repeat_interleave(torch.cumsum(cnt, 0) - cnt, cnt)
    nxs = nx[sid]
    tile = (ty0[sid] + local // nxs) * GX + tx0[sid] + local % nxs
    sh = 1 << max(1, (n - 1).bit_length())  # above every depth rank
    keys = torch.sort(tile * sh + drank[sid]).values
    del sid, local, nxs, tile
    ys, xs = torch.meshgrid(torch.arange(height, device=dev), torch.arange(width, device=dev), indexing="ij")
    tp = (ys // 16) * GX + xs // 16
    nc = n_contrib.to(torch.int64)
    start = tile_ranges[:, 0].to(torch.int64)[tp]
    last = sorted_ids.to(torch.int64)[(start + nc - 1).clamp(min=0)]
    kp = tp * sh + drank[last]
    upto = torch.searchsorted(keys, kp, right=True) - torch.searchsorted(keys, tp * sh)
    return torch.where(nc > 0, upto, torch.zeros_like(upto))


def load_probe():
    path = os.path.join(ROOT, "differentiable_tile_rasterization_amd", "libgsprobe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build with python -m differentiable_tile_rasterization_amd.build")
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_longlong
    lib.gsp_walk_stats.argtypes = [i32, P, P, P, i32, i32, P, P, P, P, P, P]
    lib.gsp_copy.argtypes = [P, P, i64, ctypes.c_int, P]
    lib.gsp_copy_stream.argtypes = [P, P, i64, ctypes.c_int, P]
    lib.gsp_lds_peak.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
    lib.gsp_atomic_replay.argtypes = [P, P, i64, P, P, P, P, P, P]
    lib.gsp_valu_peak.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
    lib.gsp_exp_peak.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
    for f in ["gsp_walk_stats", "gsp_copy", "gsp_copy_stream", "gsp_lds_peak", "gsp_atomic_replay",
              "gsp_valu_peak", "gsp_exp_peak"]:
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
    ap.add_argument("--walk", default=None, choices=["add", "store", "defer"],
                    help="force one reverse walk (default: the library's choice)")
    ap.add_argument("--cpu-sample", type=float, default=1.0, help="fraction of tiles the oracle baseline runs")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the backward on the other workloads (profiler runs: their launches of the same "
                         "kernels would mix into the per-kernel figures)")
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
    bins = gsr.gs_bin_tiles(m, q, o, r, d, sc.width, sc.height)
    img, T, nc = gsr.gs_rasterize_fwd(m, q, c, o, bg, sc.width, sc.height, bins.tile_ranges, bins.sorted_ids)
    ws = torch.empty(gsr.gs_rasterize_bwd_workspace_size(sc.n, bins.n_slots, sc.width, sc.height) + 256, dtype=torch.uint8,
                     device=dev)
    out = gsr.gs_rasterize_bwd(m, q, c, o, r, bg, sc.width, sc.height, bins, T, nc, g, accum_weight=aw,
                               workspace=ws, walk=args.walk)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)

    def bwd():
        gsr.gs_rasterize_bwd(m, q, c, o, r, bg, sc.width, sc.height, bins, T, nc, g, accum_weight=aw, out=out,
                             workspace=ws, walk=args.walk)

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
    nrect = rect_walk_pairs(torch, m, r, d, sc.width, sc.height, nc, bins.sorted_ids, bins.tile_ranges)
    p_rect = int(nrect.sum().item())
    assert p_rect >= p_walk, (p_rect, p_walk)

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
    hbm_sweep = {}
    for blocks in (2048, 4096, 8192, 16384):
        t_c = gpu_time(lambda: probe.gsp_copy_stream(src.data_ptr(), dst.data_ptr(), n4, blocks, st))
        hbm_sweep[blocks] = 2 * n4 * 16 / t_c / 1e9
    t_copy_plain = gpu_time(lambda: probe.gsp_copy(src.data_ptr(), dst.data_ptr(), n4, 256 * 8 * 4, st))
    hbm_gbs = max(hbm_sweep.values())
    del src, dst
    scratch = {k: torch.zeros_like(v) for k, v in out.items()}
    t_atomic = gpu_time(lambda: probe.gsp_atomic_replay(
        flags.data_ptr(), bins.sorted_ids.data_ptr(), bins.n_isect, scratch["dL_dmeans2d"].data_ptr(),
        scratch["dL_dconics"].data_ptr(), scratch["dL_dcolors"].data_ptr(), scratch["dL_dopacities"].data_ptr(),
        scratch["accum_weight"].data_ptr() if aw else None, st))
    nfields = 10 if aw else 9
    n_atomics = groups_tile * nfields
    pk = torch.zeros(4096, dtype=torch.float32, device=dev)
    iters = 512
    t_valu = gpu_time(lambda: probe.gsp_valu_peak(pk.data_ptr(), 256 * 32, iters, st))
    fma_lane_ops = 256 * 32 * 256 * iters * 8 / t_valu      # FMA lane-operations per second
    t_exp = gpu_time(lambda: probe.gsp_exp_peak(pk.data_ptr(), 256 * 32, iters, st))
    exp_rate = 256 * 32 * 256 * iters * 4 / t_exp
    lds_blocks, lds_iters = 256 * 4, 2048
    t_lds_rd = gpu_time(lambda: probe.gsp_lds_peak(pk.data_ptr(), lds_blocks, lds_iters, 0, st))
    lds_bcast_Bps = lds_blocks * 4 * lds_iters * 8 * 16 / t_lds_rd      # 16 B per wave instruction
    t_lds_wr = gpu_time(lambda: probe.gsp_lds_peak(pk.data_ptr(), lds_blocks, lds_iters, 1, st))
    lds_write_Bps = lds_blocks * 256 * lds_iters * 8 * 16 / t_lds_wr   # 16 B per lane
    log(f"ceilings: HBM copy {hbm_gbs:.0f} GB/s (blocks sweep {({k: round(v) for k, v in hbm_sweep.items()})}), "
        f"FMA {fma_lane_ops / 1e12:.1f} T lane-op/s, exp {exp_rate / 1e12:.2f} T/s, LDS broadcast read "
        f"{lds_bcast_Bps / 1e12:.2f} TB/s, LDS write {lds_write_Bps / 1e12:.1f} TB/s")

    # ---- per-stage times, from HIP events the library records on this stream
    # at its stage boundaries (gs_rasterize_bwd_timed); measured once before
    # the timed region (the clocks then settle under sustained load) and once
    # after it, whose means the roofline uses
    def stage_times():
        stage_ms = {"setup": [], "walk": [], "gather": []}
        for _ in range(args.steps):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            for e in evs:
                e.record(stream)
            gsr.gs_rasterize_bwd(m, q, c, o, r, bg, sc.width, sc.height, bins, T, nc, g, accum_weight=aw, out=out,
                                 workspace=ws, events=evs, walk=args.walk)
            torch.cuda.synchronize()
            for k, (a, b) in zip(stage_ms, [(0, 1), (1, 2), (2, 3)]):
                stage_ms[k].append(evs[a].elapsed_time(evs[b]))
        return {k: float(np.mean(v)) for k, v in stage_ms.items()}

    stage_pre = stage_times()
    log("stages before the timed region (ms, mean of %d calls): " % args.steps
        + ", ".join(f"{k} {v:.4f}" for k, v in stage_pre.items()))

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
    stage_mean = stage_times()
    log("stages (ms, mean of %d calls): " % args.steps + ", ".join(f"{k} {v:.4f}" for k, v in stage_mean.items()))
    t_fwd = per_call(fwd, 10, 2)
    t_mw = per_call(fwd_max_weight, 10, 2)
    # the depth variants (distortion and median together), outside the timed region
    fwd_d = gsr.gs_rasterize_fwd_depth(m, q, c, o, d, bg, sc.width, sc.height, bins.tile_ranges, bins.sorted_ids)
    gD, gM = (t(a) for a in scenes.depth_upstream(sc, args.seed))
    out_d = dict(out, dL_ddepths=torch.empty((sc.n,), dtype=torch.float32, device=dev))
    t_fwd_depth = per_call(lambda: gsr.gs_rasterize_fwd_depth(m, q, c, o, d, bg, sc.width, sc.height,
                                                              bins.tile_ranges, bins.sorted_ids), 10, 2)
    t_bwd_depth = per_call(lambda: gsr.gs_rasterize_bwd_depth(
        m, q, c, o, d, r, bg, sc.width, sc.height, bins, T, nc, fwd_d["median_pos"], g,
        dist_totals=fwd_d["dist_totals"], dL_ddist=gD, dL_dmedian=gM, accum_weight=aw, out=out_d, workspace=ws),
        10, 2)
    # the binning: events around each call (it waits once on the host for its
    # pair counts, so a call's span includes that wait), median of 10
    t_bin = float(np.median(per_call(lambda: gsr.gs_bin_tiles(m, q, o, r, d, sc.width, sc.height,
                                                              capacity=bins.n_isect), 10, 3)))

    # ---- roofline of the reverse walk (the call's dominant kernel)
    ms = float(ms_region)
    t_s = ms * 1e-3
    t_walk = stage_mean["walk"] * 1e-3
    valu_min = VALU_MIN_PER_PAIR * p_contrib
    trans_min = TRANS_PER_PAIR * p_contrib
    valu_walk = VALU_WALK_PER_WALKED * p_walk + VALU_WALK_PER_PAIR * p_contrib
    trans_walk = p_walk + p_contrib
    lds_write_bytes = entries * LDS_RECORD_BYTES
    lds_read_bytes = groups_half * LDS_RECORD_BYTES
    lds_read_bytes_unculled = entries * LDS_RECORD_BYTES * LDS_READS_PER_ENTRY
    hbm_bytes = sc.n * 36 + entries * 4 + len(bins.tile_ranges) * 8 + sc.width * sc.height * 20 \
        + sc.n * 4 * nfields
    # each term: an algorithmic count over a ceiling measured above
    terms = {
        "valu_min_ms": (valu_min / fma_lane_ops + trans_min / exp_rate) * 1e3,
        "lds_ms": (lds_write_bytes / lds_write_Bps + lds_read_bytes / lds_bcast_Bps) * 1e3,
        "hbm_ms": hbm_bytes / (hbm_gbs * 1e9) * 1e3,
        "atomic_ms": None,  # not applicable: the path issues no global atomics (each pair's sums are stored)
    }
    bound_term = max((k for k in terms if terms[k] is not None), key=lambda k: terms[k])
    t_roof = terms[bound_term] * 1e-3
    traffic, traffic_src = None, None
    if os.path.exists(PROFILE_PMC):
        with open(PROFILE_PMC) as f:
            pmc = json.load(f)
        if pmc.get("source_hash") == kernel_source_hash() and pmc.get("config") == args.config:
            traffic = pmc.get("hbm_bytes_per_launch")
            traffic_src = ("stored: rocprofv3 FETCH_SIZE / WRITE_SIZE of this kernel source (hash "
                           f"{pmc.get('source_hash')}), profiles/bwd_bench_pmc.json; not measured in this run")
    roof = {
        "bound": "alu",
        # min-model VALU lane-operations (transcendentals counted as one) per
        # second of the walk, against the part's VALU issue rate
        "achieved": (valu_min + trans_min) / t_walk / 1e12,
        "peak": PEAK_VALU_TOPS,
        "unit": "T VALU lane-op/s",
    }
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    roof["traffic_source"] = traffic_src
    # the reverse walk that ran (the library's default: the deferred walk)
    walk_used = args.walk or "defer"
    roof["kernel"] = {"add": "bwd_kernel (reverse walk, LDS adds)",
                      "store": "bwd_store_kernel (reverse walk, stored partials)",
                      "defer": "bwd_defer_kernel (reverse walk, deferred reduction)"}[walk_used]
    roof["kernel_ms"] = stage_mean["walk"]
    roof["terms_ms"] = terms
    roof["binding_term"] = bound_term
    roof["t_roof_ms"] = t_roof * 1e3
    roof["frac_measured_roof"] = t_roof / t_walk     # T_roof / walk time, every term on a measured ceiling
    roof["call_frac"] = t_roof / t_s                 # the same against the whole call
    roof["stages_ms"] = stage_mean
    roof["stages_ms_before_timed_region"] = stage_pre
    roof["walk_model_ms"] = (valu_walk / fma_lane_ops + trans_walk / exp_rate) * 1e3   # diagnostic
    roof["lds_unculled_model_ms"] = (lds_write_bytes / lds_write_Bps + lds_read_bytes_unculled / lds_bcast_Bps) * 1e3
    roof["algorithmic"] = {
        "composited_pairs": p_contrib, "walked_pairs": p_walk, "walked_entries": entries,
        "valu_min_lane_ops": valu_min, "transcendentals_min": trans_min,
        "valu_walk_lane_ops": valu_walk, "lds_bytes": lds_write_bytes + lds_read_bytes, "hbm_bytes": hbm_bytes,
        "per_composited_pair": {"valu": VALU_MIN_PER_PAIR, "transcendental": TRANS_PER_PAIR}}
    # the flush as 9-10 scattered float atomics per (splat, tile) group, timed
    # alone: what an atomic-accumulating design would pay (this one stores)
    roof["atomic_flush_replay_ms"] = t_atomic * 1e3
    roof["ceilings_measured"] = {"hbm_copy_GBs": hbm_gbs, "hbm_copy_plain_GBs": 2 * n4 * 16 / t_copy_plain / 1e9,
                                 "fma_lane_ops_per_s": fma_lane_ops, "exp_per_s": exp_rate,
                                 "lds_broadcast_read_Bps": lds_bcast_Bps, "lds_write_Bps": lds_write_Bps,
                                 "atomic_replay_per_s": n_atomics / t_atomic}

    # ---- CPU baseline: the oracle beside the GPU, on the host's cores
    others = None
    if not args.no_other_workloads:
        others = other_workloads(torch, np, gsr, scenes, args, log)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cpu = cpu_baseline(oracle, sc, bins, nc, nrect, args, log)

    value = p_rect / t_s
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
                      "raster_fwd_max_wt": float(np.median(t_mw)),
                      "raster_fwd_depth": float(np.median(t_fwd_depth)),
                      "raster_bwd_depth": float(np.median(t_bwd_depth)), "raster_bwd": ms,
                      "raster_bwd_median": float(np.median(t_calls)), "raster_bwd_min": float(np.min(t_calls))},
        "pairs": {"value_counts": "p_walk_rect (sum of n_contrib under the tile-rectangle lists)",
                  "p_walk_rect": p_rect, "pairs_per_s_own_lists": p_walk / t_s},
        "counts": {"p_walk": p_walk, "p_walk_rect": p_rect, "p_composited": p_contrib, "walked_entries": entries,
                   "splat_tile_groups": groups_tile, "splat_quadrant_groups": groups_wave,
                   "entry_quadrant_walk": ew_walk, "entry_quadrant_kept": ew_kept, "n_isect": bins.n_isect,
                   "n_slots": bins.n_slots,
                   "splat_half_groups": groups_half, "splat_block4_groups": groups_blk,
                   "lockstep_half_iters": iters_half, "lockstep_block4_iters": iters_blk},
        "other_workloads": others,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(rec))


def other_workloads(torch, np, gsr, scenes, args, log):
    """The backward on the other four workloads, in the same run (not the
    headline: no roofline or CPU baseline here): per workload 20 calls back to
    back between two HIP events on the call's stream, after 10 warm-up calls
    (ms/call, as the headline), then the mean walk span over 10 calls from the
    library's stage events, and pairs/s counted as for the headline value
    (tile-rectangle lists)."""
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    stream = torch.cuda.current_stream()
    out = {}
    for name in ("tiny", "early", "mid", "bench", "stress"):
        if name == args.config:
            continue
        sc = scenes.make_scene(name, args.seed)
        m, q, c, o, bg = t(sc.means2d), t(sc.conics), t(sc.colors), t(sc.opacities), t(sc.background)
        r, d, g = t(sc.radii), t(sc.depths), t(sc.dL_dimage)
        aw = sc.accum_weight
        bins = gsr.gs_bin_tiles(m, q, o, r, d, sc.width, sc.height)
        _, T, nc = gsr.gs_rasterize_fwd(m, q, c, o, bg, sc.width, sc.height, bins.tile_ranges, bins.sorted_ids)
        ws = torch.empty(gsr.gs_rasterize_bwd_workspace_size(sc.n, bins.n_slots, sc.width, sc.height) + 256,
                         dtype=torch.uint8, device=dev)
        res = gsr.gs_rasterize_bwd(m, q, c, o, r, bg, sc.width, sc.height, bins, T, nc, g, accum_weight=aw,
                                   workspace=ws)
        def bwd(events=None):
            gsr.gs_rasterize_bwd(m, q, c, o, r, bg, sc.width, sc.height, bins, T, nc, g, accum_weight=aw,
                                 out=res, workspace=ws, events=events)
        for _ in range(10):
            bwd()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            bwd()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        walks = []
        for _ in range(10):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            for e in evs:
                e.record(stream)   # creates the HIP events the library records again
            bwd(evs)
            torch.cuda.synchronize()
            walks.append(evs[1].elapsed_time(evs[2]))
        nrect = rect_walk_pairs(torch, m, r, d, sc.width, sc.height, nc, bins.sorted_ids, bins.tile_ranges)
        p_rect = int(nrect.sum().item())
        out[name] = {"workload": f"{name}: {sc.width}x{sc.height} RGB, {sc.n} splats"
                                 + (", accum weight" if aw else ""),
                     "ms_per_call": ms, "walk_ms": float(np.mean(walks)), "p_walk_rect": p_rect,
                     "pairs_per_s": p_rect / (ms * 1e-3)}
        log(f"other workload {name}: {ms:.4f} ms/call, walk {np.mean(walks):.4f} ms, "
            f"{p_rect / (ms * 1e-3):.3e} pairs/s")
        del m, q, c, o, bg, r, d, g, bins, T, nc, ws, res, nrect
        torch.cuda.empty_cache()
    return out


def cpu_baseline(oracle, sc, bins, nc, nrect, args, log):
    """The float64 oracle on the host: forward and backward of the timed
    scene over a sample of its tiles (all tiles by default) on every host
    thread, and both on one thread for the three small workloads (tiny, early,
    mid; their own binning, by the oracle). Binning is excluded from the
    times."""
    import numpy as np
    import scenes

    GX, GY = oracle.grid(sc.width, sc.height)
    ntiles = GX * GY
    k = max(1, int(round(args.cpu_sample * ntiles)))
    tiles = np.sort(np.random.default_rng(0).choice(ntiles, k, replace=False)).astype(np.int32)
    ids_h = bins.sorted_ids.cpu().numpy()
    rng_h = bins.tile_ranges.cpu().numpy()
    nc_h = nc.cpu().numpy()
    ys, xs = np.mgrid[0:sc.height, 0:sc.width]
    sel = np.isin((ys // 16) * GX + xs // 16, tiles)
    # the sample's pairs counted like the GPU's value (tile-rectangle lists)
    pw_sample = int(nrect.cpu().numpy()[sel].sum())
    # the host threads OpenMP is given (OMP_NUM_THREADS: the CPU share of this
    # job, which may be fewer than the host's cores)
    threads = oracle.threads()
    used = threads
    c0 = time.perf_counter()
    oracle.rasterize_fwd(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background, sc.width, sc.height,
                         rng_h, ids_h, tiles=tiles)
    f_s = time.perf_counter() - c0
    c0 = time.perf_counter()
    oracle.rasterize_bwd(sc.means2d, sc.conics, sc.colors, sc.opacities, sc.background, sc.width, sc.height,
                         rng_h, ids_h, sc.dL_dimage, tiles=tiles)
    b_s = time.perf_counter() - c0
    log(f"cpu oracle ({used} threads): forward {f_s:.2f} s, backward {b_s:.2f} s, "
        f"{pw_sample / b_s:.3e} pairs/s")
    single = {}
    oracle.set_threads(1)
    for name in ("tiny", "early", "mid"):
        s2 = scenes.make_scene(name, 0)
        ids2, rng2 = oracle.bin_tiles(s2.means2d, s2.conics, s2.opacities, s2.radii, s2.depths, s2.width,
                                      s2.height)
        c0 = time.perf_counter()
        fo = oracle.rasterize_fwd(s2.means2d, s2.conics, s2.colors, s2.opacities, s2.background, s2.width,
                                  s2.height, rng2, ids2)
        f2 = time.perf_counter() - c0
        c0 = time.perf_counter()
        oracle.rasterize_bwd(s2.means2d, s2.conics, s2.colors, s2.opacities, s2.background, s2.width, s2.height,
                             rng2, ids2, s2.dL_dimage)
        b2 = time.perf_counter() - c0
        pw = int(fo["n_contrib"].astype(np.int64).sum())
        single[name] = {"forward_s": f2, "backward_s": b2, "walked_pairs": pw, "backward_pairs_per_s": pw / b2}
        log(f"cpu oracle, 1 thread, {name}: forward {f2:.3f} s, backward {b2:.3f} s")
    oracle.set_threads(threads)
    return {"value": pw_sample / b_s, "unit": "pairs/s", "cores": used, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "forward_s": f_s, "backward_s": b_s,
            "forward_pairs_per_s": pw_sample / f_s,
            "sample": f"float64 oracle rasterize_fwd and rasterize_bwd over {k} of {ntiles} tiles (random, "
                      f"seed 0) of the same scene, {pw_sample} walked pairs (tile-rectangle lists, as the GPU "
                      f"value), on {used} threads; binning excluded; value = those pairs / backward seconds",
            "single_thread": single}


if __name__ == "__main__":
    main()
