"""Summaries of rocprofv3 runs of bench.py (host-side text processing only).

    python -m fp8_block_scaled_x128_amd.profiling stats STATS_CSV --command CMD --out FILE.md
        per-kernel duration table from a `rocprofv3 --kernel-trace --stats` run

    python -m fp8_block_scaled_x128_amd.profiling traffic --fetch CSV --write CSV
            --copy-mib N --gemm-calls C --command-fetch CMD --command-write CMD --out FILE.json
        HBM bytes per dense GEMM call from two `rocprofv3 --pmc` runs
        (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch) of a program that
        makes C dense BLOCK128 GEMM calls, half of them the MLP up projection
        and half the down projection (a call may launch two tilings).  Each
        counter is scaled by what it reads for the plain device copy of N MiB
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


def traffic_record(fetch_csv: str, write_csv: str, copy_mib: int, calls: int, cmd_fetch: str, cmd_write: str) -> dict:
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * (1 << 20)

    def pick(d, sub):
        keys = [k for k in d if sub in k]
        if not keys:
            raise SystemExit("no dispatches of %s in the counter file" % sub)
        return [v for k in keys for v in d[k]]

    f_copy = statistics.mean(v for _, v in pick(fetch, COPY_KERNEL)) * 1024
    w_copy = statistics.mean(v for _, v in pick(write, COPY_KERNEL)) * 1024
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    g_f = pick(fetch, DENSE_GEMM_KERNEL)
    g_w = pick(write, DENSE_GEMM_KERNEL)
    by_grid = {}
    for grid, v in g_f:
        by_grid.setdefault(grid, {"fetch": [], "write": []})["fetch"].append(v * 1024 * f_scale)
    for grid, v in g_w:
        by_grid.setdefault(grid, {"fetch": [], "write": []})["write"].append(v * 1024 * w_scale)
    fetch_pl = sum(v * 1024 * f_scale for _, v in g_f) / calls
    write_pl = sum(v * 1024 * w_scale for _, v in g_w) / calls
    # the two GEMMs of the MLP step: up (M 4096, N 9728, K 2560) and down (M 4096, N 2560, K 9728);
    # minimum bytes = both FP8 operands, their FP32 scales and the bf16 output, once each
    mins = []
    for M, N, K in ((4096, 9728, 2560), (4096, 2560, 9728)):
        mins.append(M * K + N * K + 4 * (M * K // 128 + (N // 128) * (K // 128)) + 2 * M * N)
    return {
        "kernel": DENSE_GEMM_KERNEL,
        "gemm_sources_sha256": gemm_sources_hash(),
        "gemm_calls": calls,
        "hbm_bytes_per_launch": fetch_pl + write_pl,
        "fetch_bytes_per_launch": fetch_pl,
        "write_bytes_per_launch": write_pl,
        "algorithmic_min_bytes_per_launch": statistics.mean(mins),
        "per_grid_size": {str(g): {"dispatches": len(v["fetch"]), "fetch_bytes": statistics.mean(v["fetch"]),
                                   "write_bytes": statistics.mean(v["write"])}
                          for g, v in by_grid.items()},
        "copy_calibration": {"bytes": copy_bytes, "fetch_counter_bytes": f_copy, "write_counter_bytes": w_copy,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "source": {"fetch": cmd_fetch, "write": cmd_write},
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--gemm-calls", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        with open(a.out, "w") as fh:
            fh.write(stats_markdown(a.stats_csv, a.command))
    else:
        rec = traffic_record(a.fetch, a.write, a.copy_mib, a.gemm_calls, a.command_fetch, a.command_write)
        with open(a.out, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
