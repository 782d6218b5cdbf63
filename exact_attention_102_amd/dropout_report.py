"""What fused dropout costs: each pass with and without dropout on P.

    python -m exact_attention_102_amd.dropout_report [--p 0.1] [--out profiles/dropout_b4_h16_n2048_d128.md]

For the head-dim workloads (d = 128, 256, 64; full and causal masks) it times the
forward and both backward designs through the public entry points -- fa_fwd /
fa_bwd against fa_fwd_dropout / fa_bwd_dropout -- with the protocol of the
benchmark snippet in "Potential algorithmic improvements for backward pass" (5
trials of 5 back-to-back dispatches, best).  Throughput is credited with the
undropped attention's flop (4 d per unmasked pair forward, 10 d backward), so the
"with dropout" column shows the same work done slower.  Each kept/dropped
decision costs one sixteenth of a Philox4x32-10 call per pass that uses it (eight
draws per call), with an 8 x 8 lane transpose of the draws in the dK/dV kernel.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = 2500.0
RUNS = [("b4_h16_n2048_d128", False), ("b4_h16_n2048_d128", True), ("b4_h8_n4096_d256", False),
        ("b1_h32_n16384_d64_causal_sharp", True)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--p", type=float, default=0.1)
    ap.add_argument("--seed", type=int, default=0x5EED)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()

    import torch

    import workloads
    from exact_attention_102_amd import (FA_BWD_5GEMM_ATOMIC, FA_BWD_7GEMM, fa_bwd, fa_bwd_dropout,
                                         fa_bwd_workspace_size, fa_fwd, fa_fwd_dropout, lib)
    from exact_attention_102_amd.flops import attention_flops
    from exact_attention_102_amd.sweep import time_calls

    lib()
    if not torch.cuda.is_available():
        raise SystemExit("dropout_report needs a GPU")
    p, seed = args.p, args.seed
    rows = []
    for wname, causal in RUNS:
        w = workloads.WORKLOADS[wname]
        B, H, N, d = w.B, w.H, w.N, w.d
        q, k, v, do = (workloads.to_bf16(x).cuda() for x in workloads.draw_workload(w))
        f32 = dict(dtype=torch.float32, device="cuda")
        o = torch.empty((B, H, N, d), **f32)
        lse = torch.empty((B, H, N), **f32)
        dq, dk, dv = (torch.empty((B, H, N, d), **f32) for _ in range(3))
        ws = torch.empty(fa_bwd_workspace_size(B, H, N, d, FA_BWD_7GEMM), dtype=torch.uint8, device="cuda")
        calls = {
            "fwd": lambda: fa_fwd(q, k, v, causal, w.scale, o=o, lse=lse),
            "fwd_drop": lambda: fa_fwd_dropout(q, k, v, causal, w.scale, p, seed, 0, o=o, lse=lse),
        }
        for key, var in (("bwd5", FA_BWD_5GEMM_ATOMIC), ("bwd7", FA_BWD_7GEMM)):
            calls[key] = (lambda var=var: fa_bwd(q, k, v, o, lse, do, causal, w.scale, var, dq=dq, dk=dk, dv=dv,
                                                 workspace=ws))
            calls[key + "_drop"] = (lambda var=var: fa_bwd_dropout(q, k, v, o, lse, do, causal, w.scale, p, seed, 0,
                                                                   variant=var, dq=dq, dk=dk, dv=dv, workspace=ws))
        fl = attention_flops(B, H, N, d, causal)
        res = {"workload": w.name, "causal": causal, "p": p}
        for key, fn in calls.items():
            if key.startswith("bwd"):   # the backward reads the matching forward's o / lse
                (calls["fwd_drop"] if key.endswith("_drop") else calls["fwd"])()
                torch.cuda.synchronize()
            best, _ = time_calls(fn, torch)
            flops = fl["fwd"] if key.startswith("fwd") else fl["bwd_effective"]
            res[key + "_ms"] = round(best, 4)
            res[key + "_tflops"] = round(flops / best / 1e9, 1)
        for key in ("fwd", "bwd5", "bwd7"):
            res[key + "_slowdown"] = round(res[key + "_drop_ms"] / res[key + "_ms"], 3)
        print(json.dumps(res), flush=True)
        rows.append(res)
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()

    if args.out:
        with open(args.out, "w") as fh:
            fh.write("# Fused dropout on P: cost per pass (one MI355X), p = %g\n\n" % p)
            # the command as run from the repository root, writing the committed file
            fh.write("Command (from the repository root): `python -m exact_attention_102_amd.dropout_report --out "
                     "profiles/%s`\n\n" % os.path.basename(args.out))
            fh.write("Best of 5 trials x 5 dispatches.  TFLOP/s credit the undropped attention (4d fwd, 10d bwd "
                     "flop per unmasked pair; peak 2500).  Slowdown = time with dropout / time without.\n\n")
            fh.write("| workload | mask | fwd TF | fwd+drop TF | x | 5-GEMM TF | +drop TF | x | 7-GEMM TF | +drop TF | x "
                     "|\n|---|---|---|---|---|---|---|---|---|---|---|\n")
            for r in rows:
                fh.write("| %s | %s | %.1f | %.1f | %.2f | %.1f | %.1f | %.2f | %.1f | %.1f | %.2f |\n" % (
                    r["workload"], "causal" if r["causal"] else "full", r["fwd_tflops"], r["fwd_drop_tflops"],
                    r["fwd_slowdown"], r["bwd5_tflops"], r["bwd5_drop_tflops"], r["bwd5_slowdown"],
                    r["bwd7_tflops"], r["bwd7_drop_tflops"], r["bwd7_slowdown"]))


if __name__ == "__main__":
    main()
