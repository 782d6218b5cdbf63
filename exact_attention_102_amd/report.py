"""Per-configuration throughput report: every workload, every mask, both backward designs.

    python -m exact_attention_102_amd.report [--out profiles/results_all_configs.md]

For each workload (and for the causal long-sequence shape also without the mask,
to show what skipping fully masked tiles saves) it times, with the protocol of the
benchmark snippet in "Potential algorithmic improvements for backward pass"
(5 trials of 5 back-to-back dispatches; best and median):

* the forward;
* the 5-GEMM backward: preprocess (delta, dq cleared) + dK/dV with atomic dQ;
* the 7-GEMM backward: dQ kernel (computing delta) + dK/dV.

Throughput is credited with 4 d flop per unmasked pair (forward) and 10 d per pair
(both backward designs, the 5-GEMM count, as that page compares them); the 7-GEMM
row also shows what it issues (14 d).  "tiles" counts the (row block x column
block) tiles each pass's default configuration loads, against the full grid.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = 2500.0
# (workload, causal) pairs reported; the long causal shape is repeated without the mask
RUNS = [("tiny_b1_h1_n128_d64", False), ("b4_h16_n2048_d128", False), ("b4_h16_n2048_d128", True),
        ("b2_h16_n8192_d128_causal", True), ("b2_h16_n8192_d128_full", False), ("b4_h8_n4096_d256", False),
        ("b1_h32_n16384_d64_causal_sharp", True)]


def tile_shape(name: str):
    """(row block, column block) of a configuration from its name ("... Br32x4 Bc64", "... Bk32x4 Bq64")."""
    m = re.search(r"B[rqk](\d+)x(\d+)\s+B[cq](\d+)", name)
    return int(m.group(1)) * int(m.group(2)), int(m.group(3))


def tiles(N: int, rows: int, cols: int, causal: bool, keys_major: bool):
    """(visited, total) tiles per head.  Query-major passes (forward, dQ) walk key tiles up to the
    workgroup's last query; the dK/dV pass (keys_major) walks query tiles from its first key on."""
    nr, nc = -(-N // rows), -(-N // cols)
    if not causal:
        return nr * nc, nr * nc
    visited = 0
    for r in range(nr):
        if keys_major:
            visited += nc - (r * rows) // cols
        else:
            last = min(N, (r + 1) * rows) - 1
            visited += last // cols + 1
    return visited, nr * nc


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    args = ap.parse_args()

    import torch

    import workloads
    from exact_attention_102_amd import (fa_bwd_dkdv, fa_bwd_dq_delta, fa_bwd_preprocess, fa_config_name,
                                         fa_default_config, fa_fwd, lib)
    from exact_attention_102_amd.flops import attention_flops, mfa_op_counts
    from exact_attention_102_amd.sweep import time_calls

    lib()
    if not torch.cuda.is_available():
        raise SystemExit("report needs a GPU")
    rows = []
    for wname, causal in RUNS:
        w = workloads.WORKLOADS[wname]
        B, H, N, d = w.B, w.H, w.N, w.d
        q, k, v, do = (workloads.to_bf16(x).cuda() for x in workloads.draw_workload(w))
        f32 = dict(dtype=torch.float32, device="cuda")
        o = torch.empty((B, H, N, d), **f32)
        lse = torch.empty((B, H, N), **f32)
        delta = torch.empty((B, H, N), **f32)
        dq, dk, dv = (torch.empty((B, H, N, d), **f32) for _ in range(3))

        def fwd():
            fa_fwd(q, k, v, causal, w.scale, o=o, lse=lse)

        def bwd5():
            fa_bwd_preprocess(o, do, delta=delta, dq=dq)
            fa_bwd_dkdv(q, k, v, do, lse, delta, causal, w.scale, True, dk, dv, dq=dq)

        def bwd7():
            fa_bwd_dq_delta(q, k, v, o, do, lse, causal, w.scale, delta, dq)
            fa_bwd_dkdv(q, k, v, do, lse, delta, causal, w.scale, False, dk, dv)

        fwd()
        torch.cuda.synchronize()
        fl = attention_flops(B, H, N, d, causal)
        res = {"workload": w.name, "causal": causal, "B": B, "H": H, "N": N, "d": d, "pairs": fl["pairs"]}
        for key, fn, flops in (("fwd", fwd, fl["fwd"]), ("bwd_5gemm", bwd5, fl["bwd_effective"]),
                               ("bwd_7gemm", bwd7, fl["bwd_effective"])):
            best, med = time_calls(fn, torch)
            res[key + "_ms_best"] = round(best, 4)
            res[key + "_ms_median"] = round(med, 4)
            res[key + "_tflops"] = round(flops / best / 1e9, 1)
            res[key + "_pct_peak"] = round(100 * flops / best / 1e9 / PEAK, 1)
        res["bwd_7gemm_issued_tflops"] = round(fl["bwd_7gemm_issued"] / res["bwd_7gemm_ms_best"] / 1e9, 1)
        res["t7_over_t5"] = round(res["bwd_7gemm_ms_best"] / res["bwd_5gemm_ms_best"], 3)
        res["faster_bwd"] = "7-GEMM" if res["t7_over_t5"] < 1 else "5-GEMM"
        for pid, key, keys_major in ((0, "fwd", False), (1, "dkdv", True), (3, "dq", False)):
            name = fa_config_name(pid, d, causal, fa_default_config(pid, d, causal))
            r_, c_ = tile_shape(name)
            vis, tot = tiles(N, r_, c_, causal, keys_major)
            res["tiles_" + key] = "%d/%d" % (vis, tot)
            res["cfg_" + key] = name
        res["mfa_op_counts"] = mfa_op_counts(N, d, B * H)
        print(json.dumps(res), flush=True)
        rows.append(res)
        del q, k, v, do, o, lse, delta, dq, dk, dv
        torch.cuda.empty_cache()

    if args.out:
        with open(args.out, "w") as fh:
            fh.write("# Throughput per configuration (one MI355X)\n\n")
            fh.write("Command (from the repository root): `python -m exact_attention_102_amd.report --out "
                     "profiles/results_all_configs.md`\n\n")
            fh.write("Best of 5 trials x 5 dispatches; TFLOP/s credit 4d (fwd) and 10d (both bwd designs) flop "
                     "per unmasked pair; % of the 2500 TFLOP/s bf16 dense peak.  7-GEMM issued = 14d per pair.  "
                     "Tiles: default configuration, loaded/total per head.\n\n")
            fh.write("| workload | mask | fwd TF (%) | 5-GEMM bwd TF (%) | 7-GEMM bwd TF (%) | 7-GEMM issued TF | "
                     "t7/t5 | fwd tiles | dK/dV tiles | dQ tiles |\n|---|---|---|---|---|---|---|---|---|---|\n")
            for r in rows:
                fh.write("| %s | %s | %.1f (%.1f) | %.1f (%.1f) | %.1f (%.1f) | %.1f | %.3f | %s | %s | %s |\n" % (
                    r["workload"], "causal" if r["causal"] else "full", r["fwd_tflops"], r["fwd_pct_peak"],
                    r["bwd_5gemm_tflops"], r["bwd_5gemm_pct_peak"], r["bwd_7gemm_tflops"], r["bwd_7gemm_pct_peak"],
                    r["bwd_7gemm_issued_tflops"], r["t7_over_t5"], r["tiles_fwd"], r["tiles_dkdv"], r["tiles_dq"]))
            fh.write("\nMedians (ms): " + "; ".join(
                "%s %s fwd %.4f / bwd5 %.4f / bwd7 %.4f" % (r["workload"], "causal" if r["causal"] else "full",
                                                             r["fwd_ms_median"], r["bwd_5gemm_ms_median"],
                                                             r["bwd_7gemm_ms_median"]) for r in rows) + "\n")


if __name__ == "__main__":
    main()
