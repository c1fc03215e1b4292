"""Summaries of rocprofv3 runs of bench.py (host-side text processing only).

    python -m fp8_block_scaled_x128_amd.profiling stats STATS_CSV --command CMD --out FILE.md
        per-kernel duration table from a `rocprofv3 --kernel-trace --stats` run

    python -m fp8_block_scaled_x128_amd.profiling pmc CSV [CSV ...] --command CMD [--command CMD ...]
            --out FILE.md [--copy-mib N]
        per-kernel counter table from `rocprofv3 --pmc` runs (one CSV per
        pass), kernels told apart by name and grid size, with the derived
        figures: matrix-pipe utilization SQ_VALU_MFMA_BUSY_CYCLES / (cycles x
        1024 SIMDs), the shader clock GRBM_GUI_ACTIVE / duration, FP8 matrix
        TFLOP/s from SQ_INSTS_VALU_MFMA_MOPS_F8 (512 flop per MOP), and HBM
        bytes and GB/s from FETCH_SIZE and WRITE_SIZE scaled by what they read
        for the plain device copy of N MiB that bench.py --copy-probe-mib N
        runs (known bytes).  GRBM_GUI_ACTIVE is summed over the 8 XCDs.

    python -m fp8_block_scaled_x128_amd.profiling traffic --fetch CSV --write CSV
            --copy-mib N --grids G1,G2 --command-fetch CMD --command-write CMD --out FILE.json
        HBM bytes per launch of the MLP up and down GEMMs (dense BLOCK128,
        bf16 out, told apart by their grid sizes G1 and G2) from two
        `rocprofv3 --pmc` runs (FETCH_SIZE, then WRITE_SIZE, in KiB per
        dispatch).  Each counter is scaled by what it reads for the plain device copy of N MiB
        that bench.py --copy-probe-mib N runs after its timed region (known
        bytes read and written).  The record carries a hash of the GEMM
        sources, so bench.py reports it only while the kernel is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("gemm.hip", "device_common.h", "internal.h")]
DENSE_GEMM_KERNEL = "k_gemm<0, false, false, "       # BLOCK128 mode, dense, bf16 out, every tiling
COPY_KERNEL = "copyBuffer"


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed, so that a
    comment edit does not invalidate a counter record of unchanged code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def gemm_sources_hash() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def _short(name: str) -> str:
    name = name.replace("fp8bs::(anonymous namespace)::", "")
    for cut in ("(fp8bs", "(unsigned", "(float const"):
        i = name.find(cut)
        if i > 0:
            name = name[:i]
    name = name.replace("void ", "")
    return name if len(name) <= 80 else name[:77] + "..."


def stats_markdown(stats_csv: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", command, "```", "",
           "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| `%s` | %s | %.1f | %.1f | %.1f | %.2f |" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out) + "\n"


def _per_kernel(counter_csv: str, counter: str):
    """{kernel name: [(grid size, value KiB), ...]} in dispatch order."""
    res = {}
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] != counter:
            continue
        res.setdefault(r["Kernel_Name"], []).append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    return res


def _probe_mean(values):
    """Mean counter value of the copy probe's dispatches: the largest device
    copies of the run (other, smaller copies are the program's own uploads)."""
    top = max(values)
    return statistics.mean(v for v in values if v >= 0.5 * top)


def traffic_record(fetch_csv: str, write_csv: str, copy_mib: int, grids, cmd_fetch: str, cmd_write: str) -> dict:
    """HBM bytes per launch of the headline step's two GEMMs (dense BLOCK128,
    bf16 out), told apart by grid size: the mean per dispatch of each, then
    the mean of the two."""
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * (1 << 20)

    def pick(d, sub):
        keys = [k for k in d if sub in k]
        if not keys:
            raise SystemExit("no dispatches of %s in the counter file" % sub)
        return [v for k in keys for v in d[k]]

    f_copy = _probe_mean([v for _, v in pick(fetch, COPY_KERNEL)]) * 1024
    w_copy = _probe_mean([v for _, v in pick(write, COPY_KERNEL)]) * 1024
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    g_f = pick(fetch, DENSE_GEMM_KERNEL)
    g_w = pick(write, DENSE_GEMM_KERNEL)
    by_grid = {}
    for grid, v in g_f:
        by_grid.setdefault(grid, {"fetch": [], "write": []})["fetch"].append(v * 1024 * f_scale)
    for grid, v in g_w:
        by_grid.setdefault(grid, {"fetch": [], "write": []})["write"].append(v * 1024 * w_scale)
    missing = [g for g in grids if g not in by_grid]
    if missing:
        raise SystemExit("no GEMM dispatches with grid size %s" % missing)
    fetch_pl = statistics.mean(statistics.mean(by_grid[g]["fetch"]) for g in grids)
    write_pl = statistics.mean(statistics.mean(by_grid[g]["write"]) for g in grids)
    # the two GEMMs of the MLP step: up (M 4096, N 9728, K 2560) and down (M 4096, N 2560, K 9728);
    # minimum bytes = both FP8 operands, their FP32 scales and the bf16 output, once each
    mins = []
    for M, N, K in ((4096, 9728, 2560), (4096, 2560, 9728)):
        mins.append(M * K + N * K + 4 * (M * K // 128 + (N // 128) * (K // 128)) + 2 * M * N)
    return {
        "kernel": DENSE_GEMM_KERNEL,
        "gemm_sources_sha256": gemm_sources_hash(),
        "grids": list(grids),
        "hbm_bytes_per_launch": fetch_pl + write_pl,
        "fetch_bytes_per_launch": fetch_pl,
        "write_bytes_per_launch": write_pl,
        "algorithmic_min_bytes_per_launch": statistics.mean(mins),
        "per_grid_size": {str(g): {"dispatches": len(v["fetch"]), "fetch_bytes": statistics.mean(v["fetch"]),
                                   "write_bytes": statistics.mean(v["write"])}
                          for g, v in by_grid.items() if g in grids},
        "copy_calibration": {"bytes": copy_bytes, "fetch_counter_bytes": f_copy, "write_counter_bytes": w_copy,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "source": {"fetch": cmd_fetch, "write": cmd_write},
    }


XCDS, SIMDS = 8, 1024


def _pmc_rows(csvs):
    """{(kernel, grid): {"dur": [ns], counter: [values]}} over all passes."""
    res = {}
    for f in csvs:
        seen = set()
        for r in csv.DictReader(open(f)):
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
            d = res.setdefault(key, {"dur": []})
            d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            did = (f, r["Dispatch_Id"])
            if did not in seen:
                seen.add(did)
                d["dur"].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return res


def pmc_markdown(csvs, commands, copy_mib=0) -> str:
    res = _pmc_rows(csvs)
    mean = statistics.mean
    fs = ws = None
    if copy_mib:
        cf = [v for (name, _), d in res.items() if COPY_KERNEL in name for v in d.get("FETCH_SIZE", [])]
        cw = [v for (name, _), d in res.items() if COPY_KERNEL in name for v in d.get("WRITE_SIZE", [])]
        fs = copy_mib * (1 << 20) / (_probe_mean(cf) * 1024) if cf else None
        ws = copy_mib * (1 << 20) / (_probe_mean(cw) * 1024) if cw else None
    counters = sorted({c for d in res.values() for c in d if c != "dur"})
    out = ["# rocprofv3 counters per kernel", "", "Commands (one pass each):", "", "```"] + list(commands) + ["```", ""]
    if fs or ws:
        out += ["Copy calibration (%d MiB device copy): FETCH_SIZE x %s, WRITE_SIZE x %s." % (
            copy_mib, "%.4f" % fs if fs else "-", "%.4f" % ws if ws else "-"), ""]
    out += ["Derived (per dispatch, mean; durations are those of the counter runs, which serialize dispatches):", "",
            "| kernel | grid | dispatches | us | clock GHz | MFMA busy % | FP8 TFLOP/s | HBM read MB | HBM write MB | HBM GB/s |",
            "|---|---|---|---|---|---|---|---|---|---|"]
    for (name, grid), d in sorted(res.items(), key=lambda kv: -mean(kv[1]["dur"]) * len(kv[1]["dur"])):
        us = mean(d["dur"]) / 1e3
        cyc = mean(d["GRBM_GUI_ACTIVE"]) / XCDS if "GRBM_GUI_ACTIVE" in d else None
        clk = "%.2f" % (cyc / (us * 1e3)) if cyc else "-"
        busy = "%.1f" % (100 * mean(d["SQ_VALU_MFMA_BUSY_CYCLES"]) / (cyc * SIMDS)) \
            if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in d else "-"
        tf = "%.0f" % (mean(d["SQ_INSTS_VALU_MFMA_MOPS_F8"]) * 512 / (us * 1e-6) / 1e12) \
            if "SQ_INSTS_VALU_MFMA_MOPS_F8" in d and mean(d["SQ_INSTS_VALU_MFMA_MOPS_F8"]) > 0 else "-"
        rd = mean(d["FETCH_SIZE"]) * 1024 * fs if fs and "FETCH_SIZE" in d else None
        wr = mean(d["WRITE_SIZE"]) * 1024 * ws if ws and "WRITE_SIZE" in d else None
        gbs = "%.0f" % ((rd + wr) / (us * 1e-6) / 1e9) if rd is not None and wr is not None else "-"
        out.append("| `%s` | %d | %d | %.1f | %s | %s | %s | %s | %s | %s |" % (
            name, grid, len(d["dur"]), us, clk, busy, tf, "%.1f" % (rd / 1e6) if rd is not None else "-",
            "%.1f" % (wr / 1e6) if wr is not None else "-", gbs))
    out += ["", "Raw counters (mean per dispatch):", "",
            "| kernel | grid | " + " | ".join(counters) + " |", "|---|---|" + "---|" * len(counters)]
    for (name, grid), d in sorted(res.items()):
        out.append("| `%s` | %d | " % (name, grid) + " | ".join(
            "%.4g" % mean(d[c]) if c in d else "-" for c in counters) + " |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    m = sub.add_parser("pmc")
    m.add_argument("csvs", nargs="+")
    m.add_argument("--command", action="append", required=True)
    m.add_argument("--copy-mib", type=int, default=0)
    m.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--grids", required=True, help="grid sizes of the up and down GEMM launches, comma list")
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        with open(a.out, "w") as fh:
            fh.write(stats_markdown(a.stats_csv, a.command))
    elif a.cmd == "pmc":
        with open(a.out, "w") as fh:
            fh.write(pmc_markdown(a.csvs, a.command, a.copy_mib))
    else:
        rec = traffic_record(a.fetch, a.write, a.copy_mib, [int(g) for g in a.grids.split(",")], a.command_fetch,
                             a.command_write)
        with open(a.out, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
