"""Block-shape sweep: times every tile configuration of every kernel on one workload.

    python -m exact_attention_102_amd.sweep --workload b4_h16_n2048_d128 [--causal 0|1] [--d 96] [--passes 0,1,2,3]
    python -m exact_attention_102_amd.sweep --all --jsonl OUT.jsonl --md OUT.md

"Potential algorithmic improvements for backward pass" (flash-attention issue 1172)
treats the block shape -- rows owned per workgroup x rows walked per tile, and
what stays in registers -- as a search under register pressure, with non-square
shapes such as 32-64 x 160-320.  This tool measures each compiled configuration
(fa_num_configs / fa_config_name) with the same protocol as that page's benchmark
(5 trials of 5 back-to-back dispatches; best and median reported) and prints one
JSON record per (pass, configuration); the library's default table is set from
these results.  --all sweeps every head dim the library builds (64, 96, 128, 192,
256) with both masks on B4 H16 N2048, plus the benchmark workloads at their own
shapes, in one process, and writes the JSON records and a markdown table per
(workload, mask, pass) with the default marked.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def time_calls(fn, torch, trials=5, dispatches=5, warmup=2):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    per = []
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(dispatches):
            fn()
        e1.record(stream)
        e1.synchronize()
        per.append(e0.elapsed_time(e1) / dispatches)
    per.sort()
    return per[0], per[len(per) // 2]


def sweep(workload: str, causal_override=None, passes=(0, 1, 2, 3), d_override: int = 0):
    import torch

    import workloads
    from exact_attention_102_amd import (fa_bwd_dkdv, fa_bwd_dq_delta, fa_bwd_preprocess, fa_config_name,
                                         fa_default_config, fa_fwd, fa_num_configs)
    from exact_attention_102_amd.flops import attention_flops

    w = workloads.WORKLOADS[workload]
    if d_override:  # same batch, heads, length and seed at another head dim
        w = dataclasses.replace(w, name="%s_hd%d" % (w.name, d_override), d=d_override)
    causal = w.causal if causal_override is None else bool(causal_override)
    B, H, N, d = w.B, w.H, w.N, w.d
    q, k, v, do = (workloads.to_bf16(x).cuda() for x in workloads.draw_workload(w))
    f32 = dict(dtype=torch.float32, device="cuda")
    o = torch.empty((B, H, N, d), **f32)
    lse = torch.empty((B, H, N), **f32)
    delta = torch.empty((B, H, N), **f32)
    dq, dk, dv = (torch.empty((B, H, N, d), **f32) for _ in range(3))
    fa_fwd(q, k, v, causal, w.scale, o=o, lse=lse)
    fa_bwd_preprocess(o, do, delta=delta)
    fl = attention_flops(B, H, N, d, causal)
    p = fl["pairs"]
    gemms = {0: 2, 1: 4, 2: 5, 3: 3}
    out = []
    for pass_id in passes:
        for cfg in range(fa_num_configs(pass_id, d)):
            if pass_id == 0:
                fn = lambda: fa_fwd(q, k, v, causal, w.scale, o=o, lse=lse, cfg=cfg)
            elif pass_id in (1, 2):
                atomic = pass_id == 2
                fn = lambda: fa_bwd_dkdv(q, k, v, do, lse, delta, causal, w.scale, atomic, dk, dv, dq=dq, cfg=cfg)
            else:
                fn = lambda: fa_bwd_dq_delta(q, k, v, o, do, lse, causal, w.scale, delta, dq, cfg=cfg)
            best, med = time_calls(fn, torch)
            flops = 2 * gemms[pass_id] * d * p
            rec = {"workload": w.name, "causal": causal, "pass": ["fwd", "dkdv", "dkdv_atomic", "dq"][pass_id],
                   "cfg": cfg, "name": fa_config_name(pass_id, d, causal, cfg),
                   "default": cfg == fa_default_config(pass_id, d, causal),
                   "best_ms": round(best, 4), "median_ms": round(med, 4),
                   "tflops_best": round(flops / best / 1e9, 1), "tflops_median": round(flops / med / 1e9, 1)}
            print(json.dumps(rec), flush=True)
            out.append(rec)
    return out


# (workload, head dim override or 0, causal): every default of the library is chosen on one of these
ALL_SWEEPS = [("b4_h16_n2048_d128", d, c) for d in (64, 96, 128, 192, 256) for c in (False, True)] + [
    ("b2_h16_n8192_d128_causal", 0, True), ("b2_h16_n8192_d128_full", 0, False), ("b4_h8_n4096_d256", 0, False),
    ("b1_h32_n16384_d64_causal_sharp", 0, True)]


def markdown(records: list) -> str:
    out = []
    groups = {}
    for r in records:
        groups.setdefault((r["workload"], r["causal"], r["pass"]), []).append(r)
    for (wl, causal, pas), rs in groups.items():
        best = min(x["best_ms"] for x in rs)
        out += ["", "### %s, %s, %s" % (wl, "causal" if causal else "non-causal", pas), "",
                "| configuration | default | best ms | median ms | TFLOP/s (best) | vs fastest |",
                "|---|---|---|---|---|---|"]
        for x in rs:
            out.append("| %s | %s | %.4f | %.4f | %.1f | %.3f |" % (x["name"], "**default**" if x["default"] else "",
                                                                    x["best_ms"], x["median_ms"], x["tflops_best"],
                                                                    x["best_ms"] / best))
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="b4_h16_n2048_d128")
    ap.add_argument("--causal", type=int, default=-1)
    ap.add_argument("--passes", default="0,1,2,3")
    ap.add_argument("--d", type=int, default=0, help="head dim in place of the workload's")
    ap.add_argument("--all", action="store_true", help="every head dim and mask plus the benchmark workloads")
    ap.add_argument("--jsonl", default=None)
    ap.add_argument("--md", default=None)
    args = ap.parse_args()
    passes = tuple(int(x) for x in args.passes.split(","))
    if not args.all:
        recs = sweep(args.workload, None if args.causal < 0 else args.causal, passes, args.d)
    else:
        recs = []
        for wl, d, causal in ALL_SWEEPS:
            print("# sweep %s d=%s causal=%d" % (wl, d or "-", causal), file=sys.stderr, flush=True)
            recs += sweep(wl, int(causal), passes, d)
    if args.jsonl:
        with open(args.jsonl, "w") as fh:
            for r in recs:
                fh.write(json.dumps(r) + "\n")
    if args.md:
        with open(args.md, "w") as fh:
            # the command as run from the repository root, writing the committed file
            cmd = "python -m exact_attention_102_amd.sweep " + (
                "--all" if args.all else "--workload %s --causal %d --passes %s%s" % (
                    args.workload, args.causal, args.passes, " --d %d" % args.d if args.d else ""))
            fh.write("# Block-shape sweep: every configuration of each pass (one MI355X)\n\n"
                     "Command (from the repository root): `%s --md profiles/%s`\n\n"
                     "Best and median of 5 trials x 5 dispatches; `default` marks the configuration the "
                     "library picks for that head dim and mask; `vs fastest` = best time / fastest best "
                     "time in the table.\n" % (cmd, os.path.basename(args.md)))
            fh.write(markdown(recs) + "\n")


if __name__ == "__main__":
    main()
