"""Markdown summaries of rocprofv3 output for the profiles/ folder.

    python -m exact_attention_102_amd.profsum stats <prof_dir> --command "<cmd>" --title "<t>" --out F
    python -m exact_attention_102_amd.profsum sq <pmc_dir> --workload b4_h16_n2048_d128 --command "<cmd>" --out F

`stats` turns the `*_kernel_stats.csv` of a `rocprofv3 --kernel-trace --stats` run into a
table of calls and durations per kernel.  `sq` turns the `*_counter_collection.csv` of a
`rocprofv3 --pmc SQ_... GRBM_GUI_ACTIVE` run over `traffic.py --run` (one launch of each
kernel per mask) into per-kernel MFMA busy fraction, MFMA flops, VALU and transcendental
instructions per score element and the LDS bank-conflict ratio.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SIMDS = 1024  # 256 CUs x 4 SIMDs
XCDS = 8      # GRBM_GUI_ACTIVE is summed over the XCDs


def _one(dirname: str, suffix: str) -> str:
    files = glob.glob(os.path.join(dirname, "**", "*" + suffix), recursive=True)
    if not files:
        raise FileNotFoundError("no *%s under %s" % (suffix, dirname))
    return sorted(files)[0]


def _col(row: dict, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(names)


def stats_table(prof_dir: str) -> str:
    rows = []
    with open(_one(prof_dir, "kernel_stats.csv")) as fh:
        for r in csv.DictReader(fh):
            rows.append((_col(r, "Name", "KernelName", "Kernel_Name"), int(_col(r, "Calls")),
                         float(_col(r, "AverageNs", "Average_Ns")) / 1e3, float(_col(r, "MinNs", "Min_Ns")) / 1e3,
                         float(_col(r, "MaxNs", "Max_Ns")) / 1e3,
                         float(_col(r, "TotalDurationNs", "Total_Duration_Ns")) / 1e6,
                         float(_col(r, "Percentage"))))
    rows.sort(key=lambda t: -t[5])
    out = ["| kernel | calls | avg us | min us | max us | total ms | % |", "|---|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, tot, pct in rows:
        out.append("| `%s` | %d | %.1f | %.1f | %.1f | %.2f | %.1f |" % (name, calls, avg, mn, mx, tot, pct))
    return "\n".join(out)


def sq_table(pmc_dir: str, workload: str) -> str:
    from exact_attention_102_amd.traffic import classify
    from workloads import WORKLOADS
    w = WORKLOADS[workload]
    per = {}
    order = []
    with open(_one(pmc_dir, "counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            d = int(r.get("Dispatch_Id", 0))
            if d not in per:
                per[d] = {"name": r["Kernel_Name"]}
                order.append(d)
            per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = ["| kernel | MFMA busy % | MFMA GFLOP | VALU lane-ops / score elem | TRANS / elem | "
           "LDS conflict cycles / LDS active |", "|---|---|---|---|---|---|"]
    for d in sorted(order):
        c = per[d]
        cl = classify(c["name"])
        if cl is None:
            continue
        kind, mask = cl
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        busy = 100.0 * c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * SIMDS) if cyc else 0.0
        gflop = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / 1e9
        lds = c.get("SQ_LDS_IDX_ACTIVE", 0.0)
        conf = c.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds if lds else 0.0
        if kind == "preprocess":
            out.append("| `%s` | %.1f | %.1f | - | - | %.3f |" % (c["name"], busy, gflop, conf))
            continue
        pairs = w.B * w.H * (w.N * (w.N + 1) // 2 if mask == "causal" else w.N * w.N)
        valu = c.get("SQ_INSTS_VALU", 0.0) * 64 / pairs
        trans = c.get("SQ_INSTS_VALU_TRANS_F32", 0.0) * 64 / pairs
        out.append("| `%s` | %.1f | %.1f | %.2f | %.2f | %.3f |" % (c["name"], busy, gflop, valu, trans, conf))
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("kind", choices=["stats", "sq"])
    ap.add_argument("dir")
    ap.add_argument("--workload", default="b4_h16_n2048_d128")
    ap.add_argument("--command", required=True, help="the profiler command that produced dir")
    ap.add_argument("--title", default=None)
    ap.add_argument("--note", default="")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.kind == "stats":
        title = a.title or "rocprofv3 kernel stats: " + a.workload
        body = stats_table(a.dir)
    else:
        title = a.title or "rocprofv3 SQ counters: %s (one launch of each kernel per mask)" % a.workload
        body = sq_table(a.dir, a.workload)
    text = "# %s\n\nCommand (from the repository root, R = its path):\n\n```\n%s\n```\n\n" % (title, a.command)
    if a.note:
        text += a.note + "\n\n"
    text += body + "\n"
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
