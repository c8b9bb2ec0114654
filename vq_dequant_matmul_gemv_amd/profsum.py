"""Condense rocprofv3 CSV output into the short text summaries kept under
profiles/.

  python -m vq_dequant_matmul_gemv_amd.profsum trace DIR --cmd "..." > out.txt
      per (kernel, grid) launch count and average / min / max duration from
      DIR/**/*kernel_trace.csv (rocprofv3 --kernel-trace --output-format csv),
      plus the --stats table (DIR/**/*kernel_stats.csv) for the library's kernels.

  python -m vq_dequant_matmul_gemv_amd.profsum pmc DIR --cmd "..." > out.txt
      per (kernel, grid) average value per dispatch of every counter in
      DIR/**/*counter_collection.csv (rocprofv3 --pmc ... --output-format csv).

Only the library's kernels (and, for the copy calibration, the copy kernel)
are listed.  The kernel source digest printed with each summary lets a reader
see whether the kernels have changed since the counters were taken (the
matmul kernels and the encoder have digests of their own).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))


ENCODER_SOURCES = ("vq_encode.hip",)


def source_digest(part: str = "matmul") -> str:
    """sha256 over kernel sources, 12 hex chars: "matmul" = every csrc/*.hip
    and csrc/*.h except the encoder's, "encoder" = the encoder's source and
    the shared headers.  The C-ABI wrapper and the public header are left
    out: they launch the kernels but do not change what a launch does on the
    GPU."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) +
                   glob.glob(os.path.join(HERE, "csrc", "*.h")))
    if part == "matmul":
        files = [f for f in files if os.path.basename(f) not in ENCODER_SOURCES]
    else:
        files = [f for f in files if os.path.basename(f) in ENCODER_SOURCES or f.endswith(".h")]
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:12]


def short_name(name: str) -> str:
    if "vqmi::" not in name:
        if "copy" in name.lower():
            return "torch copy"
        if "Fill" in name:
            return "torch fill"
        return "torch kernel"
    name = re.sub(r"^void ", "", name)
    if ">(" in name:  # template kernel: drop the parameter list
        name = name[:name.index(">(") + 1]
    name = re.sub(r"\(vqmi::\w+\)$", "", name)
    return name.replace("vqmi::", "")


def keep(name: str, with_copy: bool) -> bool:
    return "vqmi::" in name or (with_copy and "copy" in name.lower())


def _one(dirpath: str, pattern: str) -> list[str]:
    return sorted(glob.glob(os.path.join(dirpath, "**", pattern), recursive=True))


def trace(dirpath: str, with_copy: bool) -> list[str]:
    out = []
    groups = defaultdict(list)
    for f in _one(dirpath, "*kernel_trace.csv"):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                name = row["Kernel_Name"]
                if not keep(name, with_copy):
                    continue
                dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0
                grid = (row.get("Grid_Size_X") or row.get("Grid_Size"), row.get("Grid_Size_Y", "1"))
                groups[(short_name(name), grid, row.get("Workgroup_Size_X", row.get("Workgroup_Size")))].append(dur)
    out.append("per (kernel, grid) durations from the kernel trace, microseconds:")
    out.append(f"{'kernel':70s} {'grid(x,y)':>16s} {'wg':>5s} {'n':>5s} {'avg':>9s} {'min':>9s} {'max':>9s}")
    for (name, grid, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{name[:70]:70s} {grid[0] + ',' + grid[1]:>16s} {str(wg):>5s} {len(d):5d} "
                   f"{sum(d) / len(d):9.2f} {min(d):9.2f} {max(d):9.2f}")
    stats = _one(dirpath, "*kernel_stats.csv")
    if stats:
        out.append("")
        out.append("rocprofv3 --stats (library kernels; averages over every grid of one instantiation):")
        with open(stats[0], newline="") as fh:
            rows = list(csv.DictReader(fh))
        cols = [c for c in ("Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs") if c in rows[0]] \
            if rows else []
        out.append(f"{'kernel':70s} " + " ".join(f"{c:>16s}" for c in cols))
        for r in rows:
            if keep(r["Name"], with_copy):
                out.append(f"{short_name(r['Name'])[:70]:70s} " + " ".join(f"{r[c]:>16s}" for c in cols))
    return out


def pmc(dirpath: str, with_copy: bool) -> list[str]:
    vals = defaultdict(lambda: defaultdict(list))
    for f in _one(dirpath, "*counter_collection.csv"):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                name = row["Kernel_Name"]
                if not keep(name, with_copy):
                    continue
                key = (short_name(name), row["Grid_Size"], row["Workgroup_Size"])
                vals[key][row["Counter_Name"]].append(float(row["Counter_Value"]))
    out = ["average counter value per dispatch, per (kernel, grid):"]
    for (name, grid, wg), cs in sorted(vals.items()):
        n = max(len(v) for v in cs.values())
        parts = " ".join(f"{c}={sum(v) / len(v):.6g}" for c, v in sorted(cs.items()))
        out.append(f"{name[:70]:70s} grid={grid} wg={wg} dispatches={n} {parts}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["trace", "pmc"])
    ap.add_argument("dir")
    ap.add_argument("--cmd", required=True, help="the full command that produced DIR")
    ap.add_argument("--copy", action="store_true", help="also list torch's copy kernel")
    a = ap.parse_args()
    lines = [f"command: {a.cmd}", f"kernel source digest: {source_digest()}",
             f"encoder source digest: {source_digest('encoder')}", ""]
    lines += trace(a.dir, a.copy) if a.mode == "trace" else pmc(a.dir, a.copy)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
