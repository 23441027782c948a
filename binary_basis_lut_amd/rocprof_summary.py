"""Summaries of rocprofv3 CSV output (host only: reads files, runs nothing on the GPU).

The figures kept in profiles/ come from these commands, applied to the output
folders of the rocprofv3 runs each summary names:

  python3 -m binary_basis_lut_amd.rocprof_summary trace DIR
      the kernel statistics of a `--kernel-trace --stats --output-format csv`
      run: calls and average / min / max duration per kernel, as a markdown
      table;

  python3 -m binary_basis_lut_amd.rocprof_summary trace DIR --by-grid
      the same from the dispatch trace, one row per kernel and grid (so
      that launches of one instance on different layer shapes stay apart),
      with the median, 10th and 90th percentiles besides the average;

  python3 -m binary_basis_lut_amd.rocprof_summary pmc DIR --kernel REGEX
      the counters of a `--pmc ... --output-format csv` run for the dispatches
      of the kernels matching REGEX: each dispatch's value summed over the
      counter's hardware instances, then the median over the dispatches, with
      per-wave ratios when SQ_WAVES is among them, and the LDS bank-conflict
      share when SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE are;

  python3 -m binary_basis_lut_amd.rocprof_summary traffic --fetch DIR --write DIR \\
          --copy-fetch DIR --copy-write DIR --copy-bytes B --kernel REGEX \\
          --algorithmic-bytes A --workload TEXT --out FILE
      HBM bytes per launch of the kernel: the medians of FETCH_SIZE and
      WRITE_SIZE (KiB per dispatch), each scaled by known bytes / measured
      for a plain device copy of B bytes (the copy kernel the HIP runtime
      runs for torch's copy_), written as the JSON the benchmark reads,
      stamped with the hash of the GEMV kernel's sources.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the sources of the per-row g = 4 GEMV kernel the counters describe
KERNEL_SOURCES = ["binary_basis_lut_amd/csrc/common.hpp", "binary_basis_lut_amd/csrc/gemv_kernel.hpp",
                  "binary_basis_lut_amd/csrc/fluxbin.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(d: str, suffix: str) -> str:
    files = sorted(glob.glob(os.path.join(d, f"*{suffix}")))
    if not files:
        raise SystemExit(f"no *{suffix} in {d}")
    return files[0]


def trace_rows(d: str):
    with open(_one(d, "kernel_stats.csv")) as f:
        rows = list(csv.DictReader(f))
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])) for r in rows]


def pmc_medians(d: str, kernel: str) -> tuple[dict, int, str]:
    """Median over the matching dispatches of each counter (summed over its instances per dispatch)."""
    rx = re.compile(kernel)
    per = defaultdict(lambda: defaultdict(float))
    name = ""
    with open(_one(d, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if not rx.search(r["Kernel_Name"]):
                continue
            name = r["Kernel_Name"]
            per[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of a kernel matching {kernel!r} in {d}")
    counters = sorted({c for v in per.values() for c in v})
    med = {c: statistics.median(v[c] for v in per.values() if c in v) for c in counters}
    return med, len(per), name


def trace_by_grid(d: str):
    """Dispatch durations of the kernel trace grouped by (kernel, grid, workgroup size)."""
    groups = defaultdict(list)
    with open(_one(d, "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Workgroup_Size_X"]))
            groups[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return [(k, len(v), statistics.mean(v), statistics.median(v), percentile(v, 10), percentile(v, 90), min(v), max(v))
            for k, v in groups.items()]


def percentile(v, q: float) -> float:
    """The q-th percentile of v, linear between the closest ranks (numpy's default)."""
    s = sorted(v)
    pos = (len(s) - 1) * q / 100.0
    lo = int(pos)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (pos - lo)


def cmd_trace(a) -> None:
    if a.by_grid:
        print("| kernel | grid (workgroups) | calls | average ns | median ns | p10 ns | p90 ns | min ns | max ns |")
        print("|---|---|---|---|---|---|---|---|---|")
        for (name, gx, gy, wg), calls, avg, med, p10, p90, mn, mx in sorted(trace_by_grid(a.dir)):
            if a.kernel and not re.search(a.kernel, name):
                continue
            print(f"| {name} | {gx // wg} x {gy} | {calls} | {avg:.0f} | {med:.0f} | {p10:.0f} | {p90:.0f} | {mn} | {mx} |")
        return
    print("| kernel | calls | average ns | min ns | max ns |")
    print("|---|---|---|---|---|")
    for name, calls, avg, mn, mx in trace_rows(a.dir):
        if a.kernel and not re.search(a.kernel, name):
            continue
        print(f"| {name} | {calls} | {avg:.0f} | {mn:.0f} | {mx:.0f} |")


def cmd_pmc(a) -> None:
    med, n, name = pmc_medians(a.dir, a.kernel)
    print(f"kernel {name}: medians over {n} dispatches")
    print("| counter | median per dispatch |")
    print("|---|---|")
    for c, v in med.items():
        print(f"| {c} | {v:,.0f} |")
    w = med.get("SQ_WAVES")
    if w:
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD"):
            if c in med:
                print(f"{c} per wave: {med[c] / w:.1f}")
    if "SQ_LDS_BANK_CONFLICT" in med and "SQ_LDS_IDX_ACTIVE" in med:
        bc, ia = med["SQ_LDS_BANK_CONFLICT"], med["SQ_LDS_IDX_ACTIVE"]
        print(f"LDS bank-conflict cycles: {bc / ia:.3f} of LDS-active cycles ({bc / max(ia - bc, 1):.3f} per "
              f"conflict-free cycle)")


def cmd_traffic(a) -> None:
    fetch, nf, name = pmc_medians(a.fetch, a.kernel)
    write, nw, _ = pmc_medians(a.write, a.kernel)
    cfetch, _, cname = pmc_medians(a.copy_fetch, a.copy_kernel)
    cwrite, _, _ = pmc_medians(a.copy_write, a.copy_kernel)
    kib = 1024.0
    fs = a.copy_bytes / (cfetch["FETCH_SIZE"] * kib)
    ws = a.copy_bytes / (cwrite["WRITE_SIZE"] * kib)
    hbm = fetch["FETCH_SIZE"] * kib * fs + write["WRITE_SIZE"] * kib * ws
    out = {
        "kernel": name,
        "workload": a.workload,
        "kernel_source_hash": kernel_source_hash(),
        "fetch_size_kib_per_dispatch": fetch["FETCH_SIZE"],
        "write_size_kib_per_dispatch": write["WRITE_SIZE"],
        "fetch_scale_from_copy": round(fs, 4),
        "write_scale_from_copy": round(ws, 4),
        "copy_kernel": cname,
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_bytes_per_launch": a.algorithmic_bytes,
        "traffic_over_algorithmic": round(hbm / a.algorithmic_bytes, 4),
        "note": f"FETCH_SIZE and WRITE_SIZE medians over {nf} / {nw} dispatches, scaled by known / measured for a "
                f"{a.copy_bytes}-byte device copy",
    }
    text = json.dumps(out, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")
    print(text)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--kernel", default="")
    t.add_argument("--by-grid", action="store_true", help="one row per (kernel, grid) from the dispatch trace")
    p = sub.add_parser("pmc")
    p.add_argument("dir")
    p.add_argument("--kernel", required=True)
    tr = sub.add_parser("traffic")
    tr.add_argument("--fetch", required=True)
    tr.add_argument("--write", required=True)
    tr.add_argument("--copy-fetch", required=True)
    tr.add_argument("--copy-write", required=True)
    tr.add_argument("--copy-bytes", type=int, required=True)
    tr.add_argument("--copy-kernel", default="copyBuffer|elementwise|copy")
    tr.add_argument("--kernel", required=True)
    tr.add_argument("--algorithmic-bytes", type=int, required=True)
    tr.add_argument("--workload", required=True)
    tr.add_argument("--out", default="")
    a = ap.parse_args()
    {"trace": cmd_trace, "pmc": cmd_pmc, "traffic": cmd_traffic}[a.mode](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
