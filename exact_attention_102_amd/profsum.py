"""Markdown summaries of rocprofv3 output for the profiles/ folder.

    python -m exact_attention_102_amd.profsum stats <prof_dir> --command "<cmd>" --title "<t>" --out F
    python -m exact_attention_102_amd.profsum trace <prof_dir> --bench <bench.json> --steps K --warmup W \
        --command "<cmd>" --out F
    python -m exact_attention_102_amd.profsum sq <pmc_dir> --workload b4_h16_n2048_d128 --command "<cmd>" --out F

`stats` turns the `*_kernel_stats.csv` of a `rocprofv3 --kernel-trace --stats` run into a
table of calls and durations per kernel.  `trace` reads the same run's `*_kernel_trace.csv`
together with the JSON line bench.py printed in that run: it assigns every dispatch to
its (workload, mask, kernel) by its position in the step, averages the K timed steps
(the W warm-up steps excluded, as bench.py's event means are) and sets the result beside
bench.py's event-timed mean, then recomputes the roofline of bench.py's dominant kernel
from the trace.  `sq` turns the `*_counter_collection.csv` of a
`rocprofv3 --pmc SQ_... GRBM_GUI_ACTIVE` run over `traffic.py --run` (one launch of each
kernel per mask) into per-kernel MFMA busy fraction, MFMA flops, VALU and transcendental
instructions per score element and the LDS bank-conflict ratio.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SIMDS = 1024  # 256 CUs x 4 SIMDs
XCDS = 8      # GRBM_GUI_ACTIVE is summed over the XCDs
# issue cost of one wave64 instruction on a SIMD, from the measured lane rates of
# csrc/probe_rates.hip (v_fma_f32 70.7, v_exp_f32 29.8 lanes per clock per CU)
VALU_CYCLES = 64 / (70.7 / 4)
TRANS_CYCLES = 64 / (29.8 / 4)
MFMA_FLOP = 32 * 32 * 16 * 2  # one v_mfma_f32_32x32x16_bf16


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


KERNEL_ORDER = ["fwd", "preprocess5", "dkdv_atomic", "dq", "dkdv"]   # bench.py's step order


def trace_table(prof_dir: str, bench_json: str, steps: int, warmup: int) -> str:
    with open(bench_json) as fh:
        bench = json.loads([l for l in fh if l.startswith("{")][-1])
    cases = list(bench["passes"])
    per_step = len(KERNEL_ORDER) * len(cases)
    rows = []
    with open(_one(prof_dir, "kernel_trace.csv")) as fh:
        for r in csv.DictReader(fh):
            name = _col(r, "Kernel_Name", "KernelName")
            if "fa::" not in name:
                continue
            rows.append((int(_col(r, "Start_Timestamp")), int(_col(r, "End_Timestamp")), name))
    rows.sort()
    if len(rows) != (steps + warmup) * per_step:
        raise ValueError("%d attention dispatches in the trace, expected (%d + %d) x %d"
                         % (len(rows), warmup, steps, per_step))
    timed = rows[warmup * per_step:]
    acc = {}
    for i, (t0, t1, name) in enumerate(timed):
        pos = i % per_step
        key = (cases[pos // len(KERNEL_ORDER)], KERNEL_ORDER[pos % len(KERNEL_ORDER)])
        acc.setdefault(key, [name, []])[1].append((t1 - t0) / 1e3)
    out = ["| workload / mask | kernel | trace mean us (K timed steps) | trace min us | bench.py event mean us | "
           "trace / event |", "|---|---|---|---|---|---|"]
    for (case, kn), (name, ds) in acc.items():
        mean = sum(ds) / len(ds)
        ev = bench["passes"][case]["kernel_ms"][kn] * 1e3
        out.append("| %s | `%s` (%s) | %.1f | %.1f | %.1f | %.3f |" % (case, name, kn, mean, min(ds), ev, mean / ev))
    rf = bench["roofline"]
    dom = rf["kernel"]  # "kernel (workload, mask mask)"
    kn = dom.split(" (")[0]
    wl, mask = dom.split(" (")[1].rstrip(")").split(", ")
    case = "%s/%s" % (wl, mask.split()[0])
    ds = acc[(case, kn)][1]
    mean_us = sum(ds) / len(ds)
    achieved = rf["flops_per_launch"] / (mean_us * 1e-6) / 1e12
    out += ["", "Roofline of bench.py's dominant kernel, %s: %.4g flop per launch / %.1f us (trace mean) = "
            "%.1f TFLOP/s = %.4f of %.0f; bench.py reported %.1f TFLOP/s = %.4f from its event mean of %.1f us "
            "(trace / event %.3f)." % (dom, rf["flops_per_launch"], mean_us, achieved, achieved / rf["peak"],
                                       rf["peak"], rf["achieved"], rf["frac"], rf["launch_ms"] * 1e3,
                                       mean_us / (rf["launch_ms"] * 1e3))]
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
    out = ["| kernel | MFMA busy % | VALU busy % (est.) | TRANS busy % (est.) | MFMA GFLOP | "
           "VALU lane-ops / score elem | TRANS / elem | LDS conflict cycles / LDS active |",
           "|---|---|---|---|---|---|---|---|"]
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
        # busy estimates: wave instructions x their measured issue cycles over the SIMD cycles
        # (the MFMA instructions, counted among the VALU ones, are left out of the VALU figure)
        n_valu, n_trans = c.get("SQ_INSTS_VALU", 0.0), c.get("SQ_INSTS_VALU_TRANS_F32", 0.0)
        n_mfma = gflop * 1e9 / MFMA_FLOP
        simd_cyc = cyc * SIMDS
        trans_busy = 100.0 * n_trans * TRANS_CYCLES / simd_cyc if cyc else 0.0
        valu_busy = 100.0 * (max(n_valu - n_mfma - n_trans, 0.0) * VALU_CYCLES + n_trans * TRANS_CYCLES) / simd_cyc \
            if cyc else 0.0
        if kind == "preprocess":
            out.append("| `%s` | %.1f | %.1f | %.1f | %.1f | - | - | %.3f |" % (c["name"], busy, valu_busy, trans_busy,
                                                                             gflop, conf))
            continue
        pairs = w.B * w.H * (w.N * (w.N + 1) // 2 if mask == "causal" else w.N * w.N)
        valu = n_valu * 64 / pairs
        trans = n_trans * 64 / pairs
        out.append("| `%s` | %.1f | %.1f | %.1f | %.1f | %.2f | %.2f | %.3f |" % (c["name"], busy, valu_busy, trans_busy,
                                                                               gflop, valu, trans, conf))
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("kind", choices=["stats", "trace", "sq"])
    ap.add_argument("dir")
    ap.add_argument("--workload", default="b4_h16_n2048_d128")
    ap.add_argument("--command", required=True, help="the profiler command that produced dir")
    ap.add_argument("--title", default=None)
    ap.add_argument("--note", default="")
    ap.add_argument("--out", required=True)
    ap.add_argument("--bench", default=None, help="trace: the JSON line bench.py printed in the profiled run")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    a = ap.parse_args()
    if a.kind == "stats":
        title = a.title or "rocprofv3 kernel stats: " + a.workload
        body = stats_table(a.dir)
    elif a.kind == "trace":
        title = a.title or "rocprofv3 kernel trace of bench.py, per workload, mask and kernel"
        body = trace_table(a.dir, a.bench, a.steps, a.warmup)
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
