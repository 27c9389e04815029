"""Summarise rocprofv3 CSV output into the short text kept under profiles/.

    python -m differentiable_tile_rasterization_amd.profsum stats <kernel_stats.csv> <out.md> "<command>"
    python -m differentiable_tile_rasterization_amd.profsum pmc <fetch_dir> <write_dir> <out.json> <out.md> \\
        "<fetch command>" "<write command>" <config> "<call kernels, ';'-separated, the walk first>"
    python -m differentiable_tile_rasterization_amd.profsum counters <out.md> <kernel instance> \\
        <dir> "<command>" [<dir> "<command>" ...]

`counters` lists, for the last dispatch of the named kernel instance (its full
name up to the argument list) in each --pmc run directory, every counter summed over the device, with the LDS and VALU
utilisations they give. `stats` lists every kernel of a --kernel-trace --stats run (calls, average and
total time). `pmc` turns two --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
dispatch) into bytes per launch, scaled by what the same counters read for the
measurement library's 1 GiB float4 copy kernel (1 GiB read, 1 GiB written per
launch), and writes the JSON the benchmark reads for its `traffic` field: the
bytes of the reverse-walk kernel per launch (it records the hash of the
kernel sources it was taken on; the benchmark ignores it once the sources
change).
"""
from __future__ import annotations

import collections
import csv
import json
import os
import sys

COPY_BYTES = 1 << 30          # the copy kernel moves 1 GiB in and 1 GiB out per launch
COPY_NAME = "copy_kernel"
DOMINANT = ("bwd_defer_kernel<", "bwd_kernel<", "bwd_store_kernel<")  # the reverse walk (any form): the roofline's kernel


def _short(name: str) -> str:
    n = name.replace("gs::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0]


LDS_PER_CU = 160 * 1024   # gfx950
WAVES_PER_CU = 32         # 8 per SIMD


def _launch_shapes(csv_path: str) -> dict[str, tuple[int, int]]:
    """(LDS bytes per workgroup, workgroup size) of each kernel, from the
    kernel-trace CSV written beside the stats CSV (first dispatch)."""
    trace = os.path.join(os.path.dirname(csv_path), os.path.basename(csv_path).replace("kernel_stats", "kernel_trace"))
    shapes: dict[str, tuple[int, int]] = {}
    if os.path.exists(trace):
        for r in csv.DictReader(open(trace)):
            k = _short(r["Kernel_Name"])
            if k not in shapes:
                shapes[k] = (int(r["LDS_Block_Size"]), int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"])
                             * int(r["Workgroup_Size_Z"]))
    return shapes


def stats(csv_path: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    shapes = _launch_shapes(csv_path)
    lines = ["# Kernel time: " + os.path.basename(out_md).rsplit(".", 1)[0], "",
             "Command (repo root, on the MI355X host):", "", "    " + command, "",
             "LDS B/WG and WG size are the kernel trace's; \"waves/CU by LDS\" is the resident-wave",
             "limit that LDS alone sets (160 KB per CU, at most 32 waves per CU).", "",
             "| kernel | calls | avg us | min us | max us | total ms | % | LDS B/WG | WG size | waves/CU by LDS |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        k = _short(r["Name"])
        lds, wg = shapes.get(k, (0, 0))
        if wg:
            waves = -(-wg // 64)
            lim = WAVES_PER_CU if lds == 0 else min(WAVES_PER_CU, (LDS_PER_CU // lds) * waves)
            extra = f"{lds} | {wg} | {lim}"
        else:
            extra = "| |"
        lines.append(f"| {k} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} | {extra} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _per_kernel(dir_path: str) -> dict[str, list[float]]:
    path = [os.path.join(dir_path, f) for f in os.listdir(dir_path) if f.endswith("counter_collection.csv")][0]
    agg: dict[str, list[float]] = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        agg[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return agg


def pmc(fetch_dir: str, write_dir: str, out_json: str, out_md: str, cmd_fetch: str, cmd_write: str,
        config: str, call_kernels: str) -> None:
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from bench import kernel_source_hash  # the hash the benchmark compares against
    fe, wr = _per_kernel(fetch_dir), _per_kernel(write_dir)
    avg = lambda v: sum(v) / len(v)  # noqa: E731
    f_scale = COPY_BYTES / (avg(fe[COPY_NAME]) * 1024.0)
    w_scale = COPY_BYTES / (avg(wr[COPY_NAME]) * 1024.0)
    per = {}
    for k in sorted(set(fe) | set(wr)):
        fb = avg(fe[k]) * 1024.0 * f_scale if k in fe else 0.0
        wb = avg(wr[k]) * 1024.0 * w_scale if k in wr else 0.0
        per[k] = {"fetch_bytes": fb, "write_bytes": wb}
    # the call's kernel instances, named exactly (the benchmark also runs other
    # instances of the same kernels: the optional variants)
    call = [k.strip() for k in call_kernels.split(";") if k.strip()]
    missing = [k for k in call if k not in per]
    if missing:
        raise SystemExit(f"not in the counter output: {missing}")
    total = sum(per[k]["fetch_bytes"] + per[k]["write_bytes"] for k in call)
    dom = [k for k in call if k.startswith(DOMINANT)][:1]
    dom_bytes = sum(per[k]["fetch_bytes"] + per[k]["write_bytes"] for k in dom)
    rec = {"config": config, "source_hash": kernel_source_hash(), "fetch_scale": f_scale, "write_scale": w_scale,
           "dominant_kernel": dom, "hbm_bytes_per_launch": dom_bytes, "call_kernels": call,
           "call_bytes_per_launch": total, "per_kernel": per, "commands": [cmd_fetch, cmd_write]}
    json.dump(rec, open(out_json, "w"), indent=1)
    lines = ["# HBM traffic (FETCH_SIZE / WRITE_SIZE), " + config, "",
             "Commands (repo root, on the MI355X host):", "", "    " + cmd_fetch, "    " + cmd_write, "",
             f"Scale: the 1 GiB copy kernel reads {avg(fe[COPY_NAME]):.0f} KiB FETCH_SIZE and "
             f"{avg(wr[COPY_NAME]):.0f} KiB WRITE_SIZE per launch, so FETCH_SIZE is multiplied by "
             f"{f_scale:.3f} and WRITE_SIZE by {w_scale:.3f} to give bytes.", "",
             "| kernel | fetched MB / launch | written MB / launch |", "|---|---:|---:|"]
    for k, v in sorted(per.items(), key=lambda kv: -(kv[1]["fetch_bytes"] + kv[1]["write_bytes"])):
        lines.append(f"| {k} | {v['fetch_bytes'] / 1e6:.1f} | {v['write_bytes'] / 1e6:.1f} |")
    lines += ["", f"The reverse walk ({', '.join(dom)}): {dom_bytes / 1e6:.1f} MB per launch. "
                  f"One gs_rasterize_bwd call ({', '.join(call)}): {total / 1e6:.1f} MB "
                  f"(source hash {rec['source_hash']})."]
    open(out_md, "w").write("\n".join(lines) + "\n")


def counters(out_md: str, kernel: str, *runs: str) -> None:
    vals: dict[str, float] = {}
    cmds = []
    for d, cmd in zip(runs[0::2], runs[1::2]):
        path = [os.path.join(d, f) for f in os.listdir(d) if f.endswith("counter_collection.csv")][0]
        per: dict[int, dict[str, float]] = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in csv.DictReader(open(path)):
            if _short(r["Kernel_Name"]) == kernel:
                per[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        if not per:
            raise SystemExit(f"{kernel} not in {path}")
        last = per[max(per)]
        for k, v in last.items():
            vals[k if k != "GRBM_GUI_ACTIVE" else f"GRBM_GUI_ACTIVE ({os.path.basename(d)})"] = v
        cmds.append(cmd)
    lines = [f"# Counters of {kernel} (its last dispatch in each run, summed over the device)", "",
             "Commands (repo root, on the MI355X host):", ""] + ["    " + c for c in cmds] + [
             "", "| counter | value |", "|---|---:|"]
    lines += [f"| {k} | {v:.4g} |" for k, v in sorted(vals.items())]
    grbm = [v for k, v in vals.items() if k.startswith("GRBM_GUI_ACTIVE")]
    if grbm:
        cyc = max(grbm) / 8.0  # GRBM_GUI_ACTIVE counts per XCD; 8 XCDs
        lines += ["", f"Kernel cycles (GRBM_GUI_ACTIVE / 8 XCDs): {cyc:.4g} = {cyc / 2.4e3:.1f} us at 2.4 GHz."]
        if "SQ_LDS_IDX_ACTIVE" in vals:
            lines.append(f"LDS index unit busy: SQ_LDS_IDX_ACTIVE / (256 CUs x cycles) = "
                         f"{vals['SQ_LDS_IDX_ACTIVE'] / (256 * cyc):.2f}.")
        if "SQ_ACTIVE_INST_VALU" in vals:
            lines.append(f"VALU busy: SQ_ACTIVE_INST_VALU x 4 / (1024 SIMDs x cycles) = "
                         f"{vals['SQ_ACTIVE_INST_VALU'] * 4 / (1024 * cyc):.2f}.")
        if "SQ_WAVE_CYCLES" in vals:  # counted in units of 4 cycles
            lines.append(f"Mean resident waves per CU: SQ_WAVE_CYCLES x 4 / (256 CUs x cycles) = "
                         f"{vals['SQ_WAVE_CYCLES'] * 4 / (256 * cyc):.1f}.")
        if "SQ_INSTS_VALU" in vals:
            lines.append(f"VALU issue: SQ_INSTS_VALU x 4 / (1024 SIMDs x cycles) = "
                         f"{vals['SQ_INSTS_VALU'] * 4 / (1024 * cyc):.2f} of one wave instruction per 4 cycles.")
    open(out_md, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "pmc":
        pmc(*sys.argv[2:])
    elif sys.argv[1] == "counters":
        counters(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
